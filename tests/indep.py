"""Test-side widening of stored elements to float64 by torch's own dtypes.

The oracle widens a bf16 pool's uint16 bit patterns and an FP8 pool's uint8
E4M3 codes with code of its own (oracle.paged.to_f64, oracle.fp8).  The
cross-checks that pin it (torch's scaled_dot_product_attention over an
independent gather) must not reuse that code, or a slip in it would move
both sides alike.  Here the bits are reinterpreted as torch.bfloat16 and
torch.float8_e4m3fn tensors and widened by torch: bf16 is the upper half of
an IEEE float32 (the 2-byte element of "Optimizing KV Cache Memory
Management in vLLM with PagedAttention and Dynamic Block Allocation", The
Math of the KV Cache Bottleneck), and float8_e4m3fn is the OCP E4M3 format
with no infinities that an FP8 pool stores.
"""
from __future__ import annotations

import numpy as np
import torch


def widen(x) -> np.ndarray:
    """float64 values of stored elements: uint16 = bf16 bit patterns, uint8 =
    E4M3 codes (unscaled), float32/float64 as they are."""
    x = np.ascontiguousarray(np.asarray(x))
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    if x.dtype == np.uint8:
        return torch.from_numpy(x).view(torch.float8_e4m3fn).double().numpy()
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")
