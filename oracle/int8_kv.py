"""CPU oracle for the int8 KV cache (quantised write, dequantising decode).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the tests, the smoke
check and the benchmark's CPU-baseline leg may use it.

The pages name int8 KV-cache quantisation as a way to shrink the cache (the
"model-infer-kvcache" skill page, its table of FA operator parameters:
``antiquant_mode`` / ``antiquant_scale`` on one API and
``dequant_scale_key`` / ``dequant_scale_value`` on the other; its list of
further KV-cache techniques: "INT8 / W8A8C8" cache quantisation). They fix
neither the granularity nor the rounding. Readings taken: symmetric codes with one float32 scale per kv head and per
tensor (K and V have their own), value = code * scale; a stored code is
``clamp(rne(x / scale), -127, 127)`` with the division done in float32 (the
precision the kernel takes the same decision in) and rounding half to even.

``decode_int8`` is the decode definition of ``paged_attention.decode``
applied to the exactly dequantised cache (float64).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import decode, widen, write_kv

QMAX = 127


def quantize_int8(x: np.ndarray, scale: np.ndarray, dtype: str) -> np.ndarray:
    """Codes of ``x`` ([..., Hkv, D] in ``dtype`` storage) for per-head
    ``scale`` ([Hkv] float32): clamp(rne(float32(x) / scale[h]), -127, 127)."""
    xf = widen(x, dtype, np.float32)
    s = np.asarray(scale, dtype=np.float32)
    if s.ndim != 1 or s.shape[0] != xf.shape[-2]:
        raise ValueError("scale must be [num_kv_heads]")
    if not np.all(s > 0):
        raise ValueError("scales must be positive")
    r = np.rint(xf / s[:, None])                     # float32 division, ties to even
    return np.clip(r, -QMAX, QMAX).astype(np.int8)


def dequantize_int8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """code * scale[h] in float64 (exact: 8-bit code times a float32)."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return codes.astype(np.float64) * s[:, None]


def write_kv_int8(k_cache, v_cache, key, value, k_scale, v_scale, slot_mapping, block_size,
                  dtype):
    """Quantise the new rows with the per-head scales, then scatter the codes
    by ``slot_mapping`` exactly like ``write_kv`` (negative slots skipped)."""
    if k_cache.dtype != np.int8 or v_cache.dtype != np.int8:
        raise TypeError("int8 caches must be numpy int8")
    kq = quantize_int8(key, k_scale, dtype)
    vq = quantize_int8(value, v_scale, dtype)
    return write_kv(k_cache, v_cache, kq, vq, slot_mapping, block_size)


def decode_int8(q, k_codes, v_codes, k_scale, v_scale, block_table, context_lens, block_size,
                scale, dtype, pairs=None):
    """Single-token paged decode over an int8 cache: keys and values are the
    dequantised codes; everything else is ``decode``."""
    kd = dequantize_int8(k_codes, k_scale)
    vd = dequantize_int8(v_codes, v_scale)
    return decode(q, kd, vd, block_table, context_lens, block_size, scale, dtype,
                  pairs=pairs, kv_dtype="f64")
