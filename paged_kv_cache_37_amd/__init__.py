"""Paged KV-cache decode attention for AMD MI355X (gfx950).

* ``blockpool`` -- host bookkeeping (block pool, free queue, chained prefix
  hashes, reference counts) producing block tables and slot mappings;
* ``ops`` -- the C-ABI library libkvpool.so (``kv_pool_create``,
  ``cache_write``, ``paged_decode_attention``) called with torch tensors.

``ops`` is loaded on first use; it needs the built library (``python -m
paged_kv_cache_37_amd.build``) and fails loudly without it.
"""
from .blockpool import BlockPool, FreeBlockQueue, KVCacheBlock, NoFreeBlocks, hash_block  # noqa: F401

_OPS = ("KVPool", "KVPoolError", "kv_pool_create", "cache_write", "paged_decode_workspace_bytes",
        "make_workspace", "paged_decode_attention")


def __getattr__(name):
    if name in _OPS or name == "ops":
        import importlib

        ops = importlib.import_module(__name__ + ".ops")
        return ops if name == "ops" else getattr(ops, name)
    raise AttributeError(name)
