"""Python face of libkvpool: the C-ABI calls under the same names, taking
torch tensors.  Argument marshalling only -- shapes are checked, pointers and
the current HIP stream are handed to the library, every computation runs in
the library's kernels.  torch provides device memory and streams.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import DecodeArgs, KVPoolError, PoolDesc, PrefillArgs, check, lib

BLOCK_SIZE = 16  # the default block size (32 is the other one the library takes)

_DTYPES = {torch.float32: _lib.KVP_F32, torch.bfloat16: _lib.KVP_BF16, torch.float8_e4m3fn: _lib.KVP_FP8_E4M3}
_VARIANTS = {"auto": _lib.KVP_VARIANT_AUTO, "valu": _lib.KVP_VARIANT_VALU, "mfma": _lib.KVP_VARIANT_MFMA,
             "stream": _lib.KVP_VARIANT_STREAM}


def _torch_stream(device: torch.device, stream: Optional[torch.cuda.Stream]) -> torch.cuda.Stream:
    return stream if stream is not None else torch.cuda.current_stream(device)


def _stream(device: torch.device, stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    return ctypes.c_void_p(_torch_stream(device, stream).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the pool on {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class KVPool:
    """A pool of 16-token KV blocks in one torch allocation, with the
    library handle over it.  Layout: include/kvpool.h.

    dtype is the storage type: float32, bfloat16, or float8_e4m3fn (E4M3
    codes with one K and one V scale per layer, set by set_fp8_scales).
    act_dtype is the type of queries, outputs and new tokens: the pool's own
    type, bfloat16 for an FP8 pool.  The host helpers (flat, load_logical,
    to_logical) see an FP8 pool's codes as uint8."""

    def __init__(self, num_layers: int, num_blocks: int, num_kv_heads: int, head_dim: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", block_size: int = BLOCK_SIZE):
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported pool dtype {dtype}")
        self.desc = PoolDesc(num_layers, num_blocks, block_size, num_kv_heads, head_dim, _DTYPES[dtype])
        nbytes = lib.kv_pool_bytes(ctypes.byref(self.desc))
        if nbytes == 0:
            check(_lib.KVP_ERR_UNSUPPORTED if head_dim not in (64, 128) or block_size not in (16, 32)
                  else _lib.KVP_ERR_INVALID_ARG, "kv_pool_bytes")
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.act_dtype = torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype
        self.elem_dtype = torch.uint8 if dtype == torch.float8_e4m3fn else dtype
        self.num_layers, self.num_blocks, self.block_size = num_layers, num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.nbytes = int(nbytes)
        self.storage = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        handle = ctypes.c_void_p()
        check(lib.kv_pool_create(ctypes.byref(self.desc), ctypes.c_void_p(self.storage.data_ptr()),
                                 self.nbytes, ctypes.byref(handle)), "kv_pool_create")
        self.handle = handle
        # held by the pool itself: at interpreter exit the module's globals
        # may be cleared before the last pool is collected
        self._destroy = lib.kv_pool_destroy

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self._destroy(h)
            self.handle = None

    # -- layout helpers (host side; loading and inspecting pools) --------

    def set_fp8_scales(self, layer: int, k_scale: float, v_scale: float) -> None:
        """An FP8 pool's scales for `layer`: a stored code c stands for
        c * k_scale (K) or c * v_scale (V).  Both default to 1."""
        check(lib.kv_pool_set_fp8_scales(self.handle, layer, float(k_scale), float(v_scale)),
              "kv_pool_set_fp8_scales")

    def flat(self) -> torch.Tensor:
        """The pool as a flat tensor of its elements (uint8 codes for FP8)."""
        return self.storage.view(self.elem_dtype)

    def offset(self, layer: int, block: int, kv: int, head: int, slot: int, dim: int) -> int:
        return int(lib.kv_pool_offset(self.handle, layer, block, kv, head, slot, dim))

    def _tiles(self) -> torch.Tensor:
        L, NB, H, D = self.num_layers, self.num_blocks, self.num_kv_heads, self.head_dim
        return self.flat().view(L, NB, 2, H, self.block_size * D)

    def load_logical(self, logical: torch.Tensor) -> None:
        """Fill the pool from a tensor in the logical block shape
        [L, NB, 2, B, Hkv, D] (K = 0, V = 1; B = block_size)."""
        L, NB, H, D, B = self.num_layers, self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size
        if tuple(logical.shape) != (L, NB, 2, B, H, D):
            raise ValueError(f"logical pool must be {(L, NB, 2, B, H, D)}, got {tuple(logical.shape)}")
        src = logical.to(device=self.device)
        if src.dtype == torch.float8_e4m3fn:
            src = src.view(torch.uint8)
        if src.dtype != self.elem_dtype:
            raise ValueError(f"logical pool dtype {src.dtype} != pool elements {self.elem_dtype}")
        tiles = self._tiles()
        # K tile [B][D] per (block, head); V tile [B/4][D][4] (slot t -> (t//4, d, t%4))
        Q = B // 4
        tiles[:, :, 0].view(L, NB, H, B, D).copy_(src[:, :, 0].permute(0, 1, 3, 2, 4))
        tiles[:, :, 1].view(L, NB, H, Q, D, 4).copy_(
            src[:, :, 1].reshape(L, NB, Q, 4, H, D).permute(0, 1, 4, 2, 5, 3))

    def to_logical(self) -> torch.Tensor:
        """The pool in the logical block shape [L, NB, 2, B, Hkv, D]."""
        L, NB, H, D, B = self.num_layers, self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size
        Q = B // 4
        tiles = self._tiles()
        k = tiles[:, :, 0].reshape(L, NB, H, B, D).permute(0, 1, 3, 2, 4)
        v = tiles[:, :, 1].reshape(L, NB, H, Q, D, 4).permute(0, 1, 3, 5, 2, 4).reshape(L, NB, B, H, D)
        return torch.stack([k, v], dim=2).contiguous()


def kv_pool_create(num_layers: int, num_blocks: int, num_kv_heads: int, head_dim: int,
                   dtype: torch.dtype = torch.bfloat16, device="cuda", block_size: int = BLOCK_SIZE) -> KVPool:
    return KVPool(num_layers, num_blocks, num_kv_heads, head_dim, dtype, device, block_size)


def cache_write(pool: KVPool, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                slot_mapping: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Store token t's K/V ([T, Hkv, D]) at slot slot_mapping[t] of `layer`."""
    T = int(slot_mapping.shape[0]) if slot_mapping.dim() == 1 else -1
    if T < 0:
        raise ValueError("slot_mapping must be 1-D")
    shape = (T, pool.num_kv_heads, pool.head_dim)
    _need(k_new, "k_new", pool.act_dtype, pool.device, shape)
    _need(v_new, "v_new", pool.act_dtype, pool.device, shape)
    _need(slot_mapping, "slot_mapping", torch.int32, pool.device)
    check(lib.cache_write(pool.handle, layer, ctypes.c_void_p(k_new.data_ptr()),
                          ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(slot_mapping.data_ptr()), T,
                          _stream(pool.device, stream)), "cache_write")


def paged_decode_workspace_bytes(pool: KVPool, num_seqs: int, num_q_heads: int, max_blocks_per_seq: int,
                                 partition_tokens: int = 0) -> int:
    return int(lib.paged_decode_workspace_bytes(pool.handle, num_seqs, num_q_heads, max_blocks_per_seq,
                                                partition_tokens))


def make_workspace(pool: KVPool, num_seqs: int, num_q_heads: int, max_blocks_per_seq: int,
                   partition_tokens: int = 0) -> Optional[torch.Tensor]:
    """Workspace for split launches of these sizes (None when a single pass
    suffices).  Calls that share one workspace must not overlap."""
    n = paged_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=pool.device) if n else None


def _decode_args(pool: KVPool, layer: int, q: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                 scale: float, out: Optional[torch.Tensor], sliding_window: int, partition_tokens: int, variant: str,
                 workspace: Optional[torch.Tensor], stream: Optional[torch.cuda.Stream],
                 shared_prefix_blocks: int = 0, shared_blocks: bool = False, alloc: bool = True):
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    S, Hq, D = q.shape
    _need(q, "q", pool.act_dtype, pool.device)
    if D != pool.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {pool.head_dim}")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _need(block_tables, "block_tables", torch.int32, pool.device)
    _need(seq_lens, "seq_lens", torch.int32, pool.device, (S,))
    if variant not in _VARIANTS:
        raise ValueError(f"variant must be one of {sorted(_VARIANTS)}")
    mb = int(block_tables.shape[1])
    if workspace is not None and (workspace.device != pool.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the pool's device")
    # Memory made here comes from the launch stream's pool: the caching
    # allocator hands it out again only to work queued on that stream after
    # this call's kernels (memory from another stream's pool could still be
    # in use there, or be given to that stream's work while the kernels run).
    if alloc:
        with torch.cuda.stream(_torch_stream(pool.device, stream)):
            if out is None:
                out = torch.empty_like(q)
            if workspace is None:
                workspace = make_workspace(pool, S, Hq, mb, partition_tokens)
    elif out is None:
        raise ValueError("out must be given: this call allocates nothing")
    _need(out, "out", pool.act_dtype, pool.device, tuple(q.shape))
    args = DecodeArgs(
        layer=layer, q=q.data_ptr(), out=out.data_ptr(), block_tables=block_tables.data_ptr(),
        max_blocks_per_seq=mb, seq_lens=seq_lens.data_ptr(), sliding_window=sliding_window,
        num_seqs=S, num_q_heads=Hq, scale=float(scale), partition_tokens=partition_tokens,
        variant=_VARIANTS[variant],
        workspace=workspace.data_ptr() if workspace is not None else None,
        workspace_bytes=workspace.numel() * workspace.element_size() if workspace is not None else 0,
        shared_prefix_blocks=shared_prefix_blocks,
        shared_blocks=1 if shared_blocks else 0,
    )
    return args, out


def paged_decode_attention(pool: KVPool, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
                           seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                           sliding_window: int = 0, partition_tokens: int = 0, variant: str = "auto",
                           workspace: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None,
                           shared_prefix_blocks: int = 0, shared_blocks: bool = False) -> torch.Tensor:
    """Decode attention of q [S, Hq, D] over the pool through block_tables
    [S, max_blocks] and seq_lens [S]; returns out [S, Hq, D].  With
    shared_prefix_blocks = P > 0 the first P entries of every row must be
    the same full blocks: the prefix is attended once for all sequences.
    shared_blocks: some block past that prefix is listed by several rows
    (tiles are then read with cached loads; the result is the same)."""
    args, out = _decode_args(pool, layer, q, block_tables, seq_lens, scale, out, sliding_window, partition_tokens,
                             variant, workspace, stream, shared_prefix_blocks, shared_blocks)
    check(lib.paged_decode_attention(pool.handle, ctypes.byref(args), _stream(pool.device, stream)),
          "paged_decode_attention")
    return out


def paged_decode_step(pool: KVPool, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
                      seq_lens: torch.Tensor, scale: float, k_new: torch.Tensor, v_new: torch.Tensor,
                      slot_mapping: torch.Tensor, out: Optional[torch.Tensor] = None, sliding_window: int = 0,
                      partition_tokens: int = 0, variant: str = "auto", workspace: Optional[torch.Tensor] = None,
                      stream: Optional[torch.cuda.Stream] = None, shared_prefix_blocks: int = 0,
                      shared_blocks: bool = False) -> torch.Tensor:
    """Store each sequence's new token (k_new/v_new [S, Hkv, D] at
    slot_mapping [S], the slot of position seq_lens[s]-1) and attend with it;
    the same result as cache_write followed by paged_decode_attention."""
    args, out = _decode_args(pool, layer, q, block_tables, seq_lens, scale, out, sliding_window, partition_tokens,
                             variant, workspace, stream, shared_prefix_blocks, shared_blocks)
    shape = (q.shape[0], pool.num_kv_heads, pool.head_dim)
    _need(k_new, "k_new", pool.act_dtype, pool.device, shape)
    _need(v_new, "v_new", pool.act_dtype, pool.device, shape)
    _need(slot_mapping, "slot_mapping", torch.int32, pool.device, (q.shape[0],))
    check(lib.paged_decode_step(pool.handle, ctypes.byref(args), ctypes.c_void_p(k_new.data_ptr()),
                                ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(slot_mapping.data_ptr()),
                                _stream(pool.device, stream)), "paged_decode_step")
    return out


def paged_decode_step_noalloc(pool: KVPool, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
                              seq_lens: torch.Tensor, scale: float, k_new: torch.Tensor, v_new: torch.Tensor,
                              slot_mapping: torch.Tensor, out: torch.Tensor, sliding_window: int = 0,
                              partition_tokens: int = 0, variant: str = "auto",
                              stream: Optional[torch.cuda.Stream] = None, shared_prefix_blocks: int = 0,
                              shared_blocks: bool = False) -> torch.Tensor:
    """paged_decode_step without any allocation: `out` is the caller's, the
    workspace is the library's static scratch (at most
    NOALLOC_SCRATCH_BYTES per call; calls that overlap on one GPU race)."""
    args, out = _decode_args(pool, layer, q, block_tables, seq_lens, scale, out, sliding_window, partition_tokens,
                             variant, None, stream, shared_prefix_blocks, shared_blocks, alloc=False)
    shape = (q.shape[0], pool.num_kv_heads, pool.head_dim)
    _need(k_new, "k_new", pool.act_dtype, pool.device, shape)
    _need(v_new, "v_new", pool.act_dtype, pool.device, shape)
    _need(slot_mapping, "slot_mapping", torch.int32, pool.device, (q.shape[0],))
    check(lib.paged_decode_step_noalloc(pool.handle, ctypes.byref(args), ctypes.c_void_p(k_new.data_ptr()),
                                        ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(slot_mapping.data_ptr()),
                                        _stream(pool.device, stream)), "paged_decode_step_noalloc")
    return out


def _prefill_args(pool: KVPool, layer: int, q: torch.Tensor, cu_q_lens: torch.Tensor, block_tables: torch.Tensor,
                  seq_lens: torch.Tensor, scale: float, max_q_len: int, out: Optional[torch.Tensor],
                  sliding_window: int, stream: Optional[torch.cuda.Stream]):
    if q.dim() != 3 or q.shape[2] != pool.head_dim:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    T, Hq, _ = q.shape
    _need(q, "q", pool.act_dtype, pool.device)
    if cu_q_lens.dim() != 1 or cu_q_lens.shape[0] < 1:
        raise ValueError("cu_q_lens must be [num_seqs + 1]")
    S = int(cu_q_lens.shape[0]) - 1
    _need(cu_q_lens, "cu_q_lens", torch.int32, pool.device)
    _need(seq_lens, "seq_lens", torch.int32, pool.device, (S,))
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _need(block_tables, "block_tables", torch.int32, pool.device)
    if out is None:
        with torch.cuda.stream(_torch_stream(pool.device, stream)):  # the launch stream's pool, as in _decode_args
            out = torch.empty_like(q)
    _need(out, "out", pool.act_dtype, pool.device, tuple(q.shape))
    args = PrefillArgs(layer=layer, q=q.data_ptr(), out=out.data_ptr(), cu_q_lens=cu_q_lens.data_ptr(),
                       seq_lens=seq_lens.data_ptr(), block_tables=block_tables.data_ptr(),
                       max_blocks_per_seq=int(block_tables.shape[1]), num_seqs=S, num_q_heads=Hq, total_q=T,
                       max_q_len=int(max_q_len), sliding_window=sliding_window, scale=float(scale))
    return args, out


def paged_prefill_attention(pool: KVPool, layer: int, q: torch.Tensor, cu_q_lens: torch.Tensor,
                            block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_q_len: int,
                            out: Optional[torch.Tensor] = None, sliding_window: int = 0,
                            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Causal attention of multi-token chunks (q [T, Hq, D], chunk s at rows
    cu_q_lens[s] .. cu_q_lens[s+1]-1, the last positions of a context of
    seq_lens[s] tokens whose K/V are in the pool); max_q_len bounds every
    chunk length."""
    args, out = _prefill_args(pool, layer, q, cu_q_lens, block_tables, seq_lens, scale, max_q_len, out,
                              sliding_window, stream)
    check(lib.paged_prefill_attention(pool.handle, ctypes.byref(args), _stream(pool.device, stream)),
          "paged_prefill_attention")
    return out


def paged_prefill_step(pool: KVPool, layer: int, q: torch.Tensor, cu_q_lens: torch.Tensor,
                       block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_q_len: int,
                       k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                       out: Optional[torch.Tensor] = None, sliding_window: int = 0,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Store the chunks' K/V (k_new/v_new [T, Hkv, D] at slot_mapping [T]),
    then paged_prefill_attention."""
    args, out = _prefill_args(pool, layer, q, cu_q_lens, block_tables, seq_lens, scale, max_q_len, out,
                              sliding_window, stream)
    shape = (q.shape[0], pool.num_kv_heads, pool.head_dim)
    _need(k_new, "k_new", pool.act_dtype, pool.device, shape)
    _need(v_new, "v_new", pool.act_dtype, pool.device, shape)
    _need(slot_mapping, "slot_mapping", torch.int32, pool.device, (q.shape[0],))
    check(lib.paged_prefill_step(pool.handle, ctypes.byref(args), ctypes.c_void_p(k_new.data_ptr()),
                                 ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(slot_mapping.data_ptr()),
                                 _stream(pool.device, stream)), "paged_prefill_step")
    return out


def copy_blocks(pool: KVPool, src: torch.Tensor, dst: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None) -> None:
    """Copy every layer's K/V of physical block src[i] into dst[i] (int32
    device tensors of equal length): the device side of copy-on-write."""
    if src.dim() != 1 or dst.shape != src.shape:
        raise ValueError("src and dst must be 1-D of equal length")
    _need(src, "src", torch.int32, pool.device)
    _need(dst, "dst", torch.int32, pool.device)
    check(lib.kv_pool_copy_blocks(pool.handle, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                  int(src.shape[0]), _stream(pool.device, stream)), "kv_pool_copy_blocks")


__all__ = ["KVPool", "KVPoolError", "kv_pool_create", "cache_write", "paged_decode_workspace_bytes",
           "make_workspace", "paged_decode_attention", "paged_decode_step", "paged_decode_step_noalloc", "copy_blocks",
           "paged_prefill_attention", "paged_prefill_step", "BLOCK_SIZE"]
