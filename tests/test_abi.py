"""The C-ABI library without a GPU: it loads, exports what include/kvpool.h
declares, computes geometry and layout offsets, and rejects bad arguments
before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvpool.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def ops():
    from paged_kv_cache_37_amd import ops as m

    return m


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ("kv_pool_create", "cache_write", "paged_decode_attention"):
        assert n in names


def test_every_declared_symbol_is_exported(ops):
    names = header_functions()
    assert names, "no functions parsed from the header"
    for n in names:
        assert hasattr(ops.lib, n), n
    assert sorted(names) == sorted(ops._lib.EXPORTS)


def test_library_is_the_in_tree_build(ops):
    maps = open("/proc/self/maps").read()
    assert os.path.join(ROOT, "paged_kv_cache_37_amd", "libkvpool.so") in maps
    hip = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hip) == 1, f"more than one HIP runtime mapped: {hip}"


def desc(ops, L=2, NB=10, H=3, D=64, dtype=0, B=16):
    return ops.PoolDesc(L, NB, B, H, D, dtype)


def test_pool_bytes(ops):
    d = desc(ops)
    assert ops.lib.kv_pool_bytes(ctypes.byref(d)) == 2 * 10 * 2 * 16 * 3 * 64 * 4
    d = desc(ops, dtype=1, D=128)
    assert ops.lib.kv_pool_bytes(ctypes.byref(d)) == 2 * 10 * 2 * 16 * 3 * 128 * 2
    assert ops.lib.kv_pool_bytes(ctypes.byref(desc(ops, B=32))) == 2 * 10 * 2 * 32 * 3 * 64 * 4
    assert ops.lib.kv_pool_bytes(ctypes.byref(desc(ops, B=64))) == 0
    assert ops.lib.kv_pool_bytes(ctypes.byref(desc(ops, B=8))) == 0
    assert ops.lib.kv_pool_bytes(ctypes.byref(desc(ops, D=96))) == 0


def _handle(ops, d, base=0x100000):
    h = ctypes.c_void_p()
    nbytes = ops.lib.kv_pool_bytes(ctypes.byref(d))
    st = ops.lib.kv_pool_create(ctypes.byref(d), ctypes.c_void_p(base), nbytes, ctypes.byref(h))
    return st, h


def test_create_checks_arguments(ops):
    d = desc(ops)
    st, h = _handle(ops, d, base=0x100010)  # misaligned
    assert st == ops._lib.KVP_ERR_INVALID_ARG
    assert b"aligned" in ops.lib.kvp_last_error()
    h = ctypes.c_void_p()
    assert ops.lib.kv_pool_create(ctypes.byref(d), ctypes.c_void_p(0x100000), 16, ctypes.byref(h)) == \
        ops._lib.KVP_ERR_INVALID_ARG
    bad = desc(ops, B=64)
    assert _handle(ops, bad)[0] == ops._lib.KVP_ERR_UNSUPPORTED
    st, h = _handle(ops, d)
    assert st == 0 and h.value
    out = ops.PoolDesc()
    assert ops.lib.kv_pool_describe(h, ctypes.byref(out)) == 0
    assert (out.num_layers, out.num_blocks, out.num_kv_heads, out.head_dim) == (2, 10, 3, 64)
    assert ops.lib.kv_pool_destroy(h) == 0


@pytest.mark.parametrize("D,B", [(64, 16), (128, 16), (128, 32)])
def test_offsets_follow_documented_layout(ops, D, B):
    L, NB, H = 2, 5, 3
    st, h = _handle(ops, desc(ops, L, NB, H, D, dtype=1, B=B))
    assert st == 0
    seen = set()
    for layer in range(L):
        for b in range(NB):
            for kv in range(2):
                for hh in range(H):
                    for t in range(B):
                        for d in (0, 1, D - 1):
                            off = ops.lib.kv_pool_offset(h, layer, b, kv, hh, t, d)
                            block_base = ((layer * NB + b) * 2 * H) * B * D
                            if kv == 0:
                                exp = block_base + hh * B * D + t * D + d
                            else:
                                exp = block_base + (H + hh) * B * D + ((t // 4) * D + d) * 4 + t % 4
                            assert off == exp
                            seen.add(off)
    assert len(seen) == L * NB * 2 * H * B * 3
    assert ops.lib.kv_pool_offset(h, 0, 0, 0, 0, B, 0) == -1
    assert ops.lib.kv_pool_offset(h, L, 0, 0, 0, 0, 0) == -1
    assert ops.lib.kv_pool_offset(h, 0, 0, 2, 0, 0, 0) == -1
    ops.lib.kv_pool_destroy(h)


def test_decode_rejects_bad_arguments_before_launch(ops):
    st, h = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=0))
    A = ops.DecodeArgs
    base = dict(layer=0, q=0x1000, out=0x2000, block_tables=0x3000, max_blocks_per_seq=4, seq_lens=0x4000,
                sliding_window=0, num_seqs=2, num_q_heads=8, scale=0.125, partition_tokens=0, variant=0,
                workspace=None, workspace_bytes=0)

    def call(**kw):
        a = A(**{**base, **kw})
        return ops.lib.paged_decode_attention(h, ctypes.byref(a), None)

    E = ops._lib
    assert call(layer=1) == E.KVP_ERR_INVALID_ARG
    assert call(num_q_heads=7) == E.KVP_ERR_INVALID_ARG
    assert call(q=None) == E.KVP_ERR_INVALID_ARG
    assert call(partition_tokens=24) == E.KVP_ERR_INVALID_ARG
    assert call(partition_tokens=2048) == E.KVP_ERR_INVALID_ARG
    assert call(variant=2) == E.KVP_ERR_UNSUPPORTED       # MFMA needs bf16
    assert call(variant=7) == E.KVP_ERR_INVALID_ARG
    assert call(sliding_window=-1) == E.KVP_ERR_INVALID_ARG
    assert call(scale=float("nan")) == E.KVP_ERR_INVALID_ARG
    assert call(max_blocks_per_seq=0) == E.KVP_ERR_INVALID_ARG
    assert call(q=0x1004) == E.KVP_ERR_INVALID_ARG       # misaligned
    # long rows need the split workspace
    assert call(max_blocks_per_seq=64, partition_tokens=256) == E.KVP_ERR_WORKSPACE_TOO_SMALL
    need = ops.lib.paged_decode_workspace_bytes(h, 2, 8, 64, 256)
    rows = 2 * 8 * 4
    assert need == rows * 64 * 4 + rows * 2 * 4  # partial outputs and their (max, sum) pairs
    assert ops.lib.paged_decode_workspace_bytes(h, 2, 8, 4, 256) == 0
    assert call(num_seqs=0) == 0  # nothing to do
    ops.lib.kv_pool_destroy(h)


def test_cache_write_rejects_bad_arguments(ops):
    st, h = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=1))
    E = ops._lib
    assert ops.lib.cache_write(h, 3, 0x1000, 0x2000, 0x3000, 4, None) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.cache_write(h, 0, None, 0x2000, 0x3000, 4, None) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.cache_write(h, 0, 0x1008, 0x2000, 0x3000, 4, None) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.cache_write(h, 0, 0x1000, 0x2000, 0x3000, -1, None) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.cache_write(h, 0, None, None, None, 0, None) == 0
    assert ops.lib.kvp_status_str(E.KVP_ERR_WORKSPACE_TOO_SMALL) == b"workspace too small"
    ops.lib.kv_pool_destroy(h)


def test_fp8_pool_geometry_and_scales(ops):
    """An FP8 pool: one byte per element, the same element offsets as the
    other dtypes, per-layer scales validated on the host."""
    E = ops._lib
    d = desc(ops, 3, 10, 2, 128, dtype=E.KVP_FP8_E4M3)
    assert ops.lib.kv_pool_bytes(ctypes.byref(d)) == 3 * 10 * 2 * 16 * 2 * 128
    st, h = _handle(ops, d)
    assert st == 0
    ref_st, ref = _handle(ops, desc(ops, 3, 10, 2, 128, dtype=E.KVP_BF16))
    for args in ((0, 0, 0, 0, 0, 0), (2, 9, 1, 1, 15, 127), (1, 4, 1, 0, 6, 33)):
        assert ops.lib.kv_pool_offset(h, *args) == ops.lib.kv_pool_offset(ref, *args)
    assert ops.lib.kv_pool_set_fp8_scales(h, 2, 0.5, 3.0) == 0
    assert ops.lib.kv_pool_set_fp8_scales(h, 3, 0.5, 3.0) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.kv_pool_set_fp8_scales(h, -1, 0.5, 3.0) == E.KVP_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert ops.lib.kv_pool_set_fp8_scales(h, 0, bad, 1.0) == E.KVP_ERR_INVALID_ARG
        assert ops.lib.kv_pool_set_fp8_scales(h, 0, 1.0, bad) == E.KVP_ERR_INVALID_ARG
    assert ops.lib.kv_pool_set_fp8_scales(ref, 0, 1.0, 1.0) == E.KVP_ERR_UNSUPPORTED
    assert ops.lib.kv_pool_set_fp8_scales(None, 0, 1.0, 1.0) == E.KVP_ERR_INVALID_ARG
    ops.lib.kv_pool_destroy(h)
    ops.lib.kv_pool_destroy(ref)


def test_fp8_pool_variant_checks(ops):
    """The VALU variant takes no FP8 pool; the matrix-core variants no fp32
    pool.  Both are refused before any launch."""
    E = ops._lib
    A = ops.DecodeArgs
    base = dict(layer=0, q=0x1000, out=0x2000, block_tables=0x3000, max_blocks_per_seq=4, seq_lens=0x4000,
                sliding_window=0, num_seqs=2, num_q_heads=8, scale=0.125, partition_tokens=0, variant=0,
                workspace=None, workspace_bytes=0)
    _, h8 = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=E.KVP_FP8_E4M3))
    _, h32 = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=E.KVP_F32))
    a = A(**{**base, "variant": E.KVP_VARIANT_VALU})
    assert ops.lib.paged_decode_attention(h8, ctypes.byref(a), None) == E.KVP_ERR_UNSUPPORTED
    assert b"VALU" in ops.lib.kvp_last_error()
    for v in (E.KVP_VARIANT_MFMA, E.KVP_VARIANT_STREAM):
        a = A(**{**base, "variant": v})
        assert ops.lib.paged_decode_attention(h32, ctypes.byref(a), None) == E.KVP_ERR_UNSUPPORTED
    ops.lib.kv_pool_destroy(h8)
    ops.lib.kv_pool_destroy(h32)


def test_block_size_32_geometry_checks(ops):
    """32-token blocks: partitions and workspace count 16-token tiles, and
    a table whose rows could hold more than 2^31 slots is refused."""
    E = ops._lib
    _, h = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=E.KVP_BF16, B=32))
    need = ops.lib.paged_decode_workspace_bytes(h, 2, 8, 64, 256)
    rows = 2 * 8 * (64 * 2 // 16)  # 64 entries = 128 tiles = 8 partitions of 16 tiles
    assert need >= rows * 64 * 4 + rows * 2 * 4  # the partitioned variant's partials fit
    A = ops.DecodeArgs
    a = A(layer=0, q=0x1000, out=0x2000, block_tables=0x3000, max_blocks_per_seq=(1 << 26), seq_lens=0x4000,
          sliding_window=0, num_seqs=2, num_q_heads=8, scale=0.125, partition_tokens=256, variant=E.KVP_VARIANT_MFMA,
          workspace=None, workspace_bytes=0)
    assert ops.lib.paged_decode_attention(h, ctypes.byref(a), None) == E.KVP_ERR_INVALID_ARG
    assert b"block_size" in ops.lib.kvp_last_error()
    ops.lib.kv_pool_destroy(h)


def test_prefill_rejects_bad_arguments_before_launch(ops):
    E = ops._lib
    A = ops._lib.PrefillArgs
    base = dict(layer=0, q=0x1000, out=0x2000, cu_q_lens=0x3000, seq_lens=0x4000, block_tables=0x5000,
                max_blocks_per_seq=4, num_seqs=2, num_q_heads=8, total_q=10, max_q_len=8, sliding_window=0,
                scale=0.125)
    _, h = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=E.KVP_BF16))
    _, h32 = _handle(ops, desc(ops, 1, 8, 2, 64, dtype=E.KVP_F32))

    def call(hh=h, **kw):
        a = A(**{**base, **kw})
        return ops.lib.paged_prefill_attention(hh, ctypes.byref(a), None)

    assert call(hh=h32) == E.KVP_ERR_UNSUPPORTED
    assert call(layer=1) == E.KVP_ERR_INVALID_ARG
    assert call(num_q_heads=7) == E.KVP_ERR_INVALID_ARG
    assert call(q=None) == E.KVP_ERR_INVALID_ARG
    assert call(q=0x1008) == E.KVP_ERR_INVALID_ARG
    assert call(max_q_len=-1) == E.KVP_ERR_INVALID_ARG
    assert call(sliding_window=-2) == E.KVP_ERR_INVALID_ARG
    assert call(scale=float("inf")) == E.KVP_ERR_INVALID_ARG
    assert call(max_blocks_per_seq=1 << 28) == E.KVP_ERR_INVALID_ARG
    assert call(num_seqs=0) == 0 and call(total_q=0) == 0  # nothing to do
    # the fused step checks the attention's arguments before writing anything
    a = A(**{**base, "q": None})
    assert ops.lib.paged_prefill_step(h, ctypes.byref(a), 0x6000, 0x7000, 0x8000, None) == E.KVP_ERR_INVALID_ARG
    a = A(**base)
    assert ops.lib.paged_prefill_step(h, ctypes.byref(a), None, 0x7000, 0x8000, None) == E.KVP_ERR_INVALID_ARG
    ops.lib.kv_pool_destroy(h)
    ops.lib.kv_pool_destroy(h32)


def test_struct_layouts_match_the_header(ops, tmp_path):
    """The ctypes mirrors of the header's argument structs have the C
    compiler's sizes and field offsets (a small C program built against
    include/kvpool.h prints them)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    structs = {"kvp_pool_desc": ops._lib.PoolDesc, "kvp_decode_args": ops.DecodeArgs,
               "kvp_prefill_args": ops._lib.PrefillArgs}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "kvpool.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    hip_inc = os.environ.get("ROCM_PATH", "/opt/rocm") + "/include"
    subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", hip_inc,
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        name, field, value = line.split()
        got[(name, field)] = int(value)
    for name, cls in structs.items():
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)
