"""Test helpers shared by the GPU tests of the paged cache formats: layouts
and the oracle's stored values per format (test infrastructure: uses the
oracle).

  "fp4"   E2M1 elements, an E4M3 scale per 16 channels
  "fp8"   E4M3 elements, one scale per tensor (0.03 for K, 0.02 for V here)
  "fp8t"  E4M3 elements, one fp16 scale per (token, KV head)
"""
import numpy as np

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl
import oracle

FP8_SCALES = (0.03, 0.02)


def layout(fmt: str, H: int, D: int, pages: int):
    if fmt == "fp8":
        return fk.cache_layout(H, D, pages, format=fk.FORMAT_FP8_E4M3, k_scale=FP8_SCALES[0],
                               v_scale=FP8_SCALES[1])
    if fmt == "fp8t":
        return fk.cache_layout(H, D, pages, format=fk.FORMAT_FP8_E4M3_TOKEN)
    if fmt == "fp4":
        return fk.cache_layout(H, D, pages)
    raise ValueError(fmt)


def stored_values(fmt: str, L, x) -> np.ndarray:
    """float64 [n][H][D]: the oracle's stored values of bf16 rows x [n][H][D]
    (K or V alike for these formats) in a cache of layout L."""
    bits = wl.bf16_bits(x)
    if bits.shape[0] == 0:
        return np.zeros(bits.shape, np.float64)
    if fmt == "fp8t":
        c, s = oracle.quantize_fp8_groups(bits, "token")
        return oracle.dequantize_fp8_groups(c, s, "token")
    raise ValueError("use the format's own oracle attention for " + fmt)
