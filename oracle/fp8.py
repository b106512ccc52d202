"""FP8 (E4M3) KV-cache arithmetic for the oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the library never calls it and shares no code with it.

The pages list an FP8 KV cache with per-head quantisation scales among the
features of the FlashAttention-3 and FlashInfer backends ("FlashAttention 在
vLLM 中的实现分析" and the backend-abstraction page: the fp8 / fp8_e4m3 cache
dtype, "per-head quant scales").  They give no formula, so the plainest reading
is taken, as in the scaled conversions those libraries use:

* format: the OCP 8-bit float E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9;
  no infinities; S.1111.111 is NaN; the largest finite value is 448;
* quantise (the cache write): code = E4M3(fp32(x) / fp32(scale)), the
  division in IEEE fp32 and the conversion rounding to nearest, ties to the
  even code, saturating to +-448 (inputs beyond it, infinities included);
  NaN -> 0x7F;
* dequantise (the attention's K/V walk): value = E4M3 value * scale, with one
  scale per KV head for K (k_scale[h]) and one for V (v_scale[h]).

The conversion is written from the format's definition: the encoder picks
the nearest of the representable values by enumeration, not by bit tricks.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64 by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    norm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = sign * np.where(e == 0, sub, norm)
    return np.where((e == 15) & (m == 7), np.nan, v)


# the 127 non-negative finite values, in code order (code k <-> value k)
_GRID = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))


def f32_to_e4m3(x) -> np.ndarray:
    """Round fp32 values to E4M3 codes: nearest representable value, ties to
    the even code, saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    sign = np.where(np.signbit(x), 0x80, 0x00)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_GRID, a, side="left")          # first grid value >= a
    hi = np.minimum(hi, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _GRID[hi], hi, np.where(pick_hi, hi, lo))
    out = (code | sign).astype(np.uint8)
    return np.where(nan, np.uint8(NAN_CODE), out).astype(np.uint8)


def quantize(x_bf16_bits: np.ndarray, scale) -> np.ndarray:
    """E4M3 codes of bf16 values divided by an fp32 scale (division in fp32)."""
    b = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    x = b.view(np.float32)
    return f32_to_e4m3(x / np.float32(scale))


def reshape_and_cache_fp8(key: np.ndarray, value: np.ndarray, kv_cache: np.ndarray,
                          slot_mapping: np.ndarray, k_scale: np.ndarray,
                          v_scale: np.ndarray) -> np.ndarray:
    """Return a copy of the uint8 cache [2, NB, BS, Hkv, D] with token t's key
    and value rows (bf16 bits [T, Hkv, D]) quantised per KV head h with
    k_scale[h] / v_scale[h] and written at slot ``slot_mapping[t]`` (block
    ``s // BS``, offset ``s % BS``); a negative slot is skipped."""
    out = np.asarray(kv_cache, dtype=np.uint8).copy()
    BS = out.shape[2]
    Hkv = out.shape[3]
    for t in range(key.shape[0]):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        for h in range(Hkv):
            out[0, s // BS, s % BS, h] = quantize(key[t, h], np.float32(k_scale[h]))
            out[1, s // BS, s % BS, h] = quantize(value[t, h], np.float32(v_scale[h]))
    return out


def dequantize(codes: np.ndarray, scale) -> np.ndarray:
    """float64 values of E4M3 codes times an fp32 scale."""
    return e4m3_to_f64(codes) * float(np.float32(scale))
