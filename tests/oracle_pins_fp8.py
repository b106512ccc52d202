"""Pins of the oracle's FP8 (E4M3) KV-cache arithmetic (oracle/fp8.py and the
E4M3 path of oracle.attention.varlen_attention).

The pages name an FP8 (fp8_e4m3) KV cache with per-head scales but print no
encoding, so the facts used here are those of the OCP 8-bit floating-point
format E4M3 itself (bias 7, 3 mantissa bits, subnormals m * 2^-9, no
infinities, S.1111.111 = NaN, largest finite 448): a table of closed-form
code values, a second encoder written independently (frexp + Python's
round-half-even on exact binary fractions) compared on every code, every
midpoint and random fp32 values, and invariants of the scaled attention."""
import math

import numpy as np

import oracle.attention as OA
import oracle.fp8 as OF8
from paged_kv_varlen_flash_amd import workloads as W

# code -> value, closed forms of the E4M3 definition
DECODE_TABLE = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x09: 1.125 * 2.0 ** -6,
    0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x70: 128.0, 0x77: 240.0, 0x7E: 448.0,
    0x80: -0.0, 0xB8: -1.0, 0xC4: -3.0, 0xFE: -448.0,
}


def _encode_ref(x: float) -> int:
    """Independent E4M3 encoder: nearest value, ties to even, saturating."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a >= 448.0:
        return sign | 0x7E
    if a < 2.0 ** -6:                       # subnormal range: multiples of 2^-9
        r = round(a * 2.0 ** 9)             # exact scaling; round half to even
        return sign | r                     # r == 8 is the smallest normal, code 0x08
    mant, e = math.frexp(a)                 # a = mant * 2^e, mant in [0.5, 1)
    q = a * 2.0 ** (4 - e)                  # in [8, 16): 1.mmm * 8
    r = round(q)
    if r == 16:
        r, e = 8, e + 1
    code = ((e - 1 + 7) << 3) | (r - 8)
    return sign | min(code, 0x7E)


def pin_e4m3_decode_table():
    c = np.array(sorted(DECODE_TABLE), dtype=np.uint8)
    v = OF8.e4m3_to_f64(c)
    for code, got in zip(c, v):
        want = DECODE_TABLE[int(code)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(code), got, want)
    nan = OF8.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(nan).all()
    pos = OF8.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase"
    neg = OF8.e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def pin_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = OF8.f32_to_e4m3(OF8.e4m3_to_f64(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def pin_e4m3_encoder_against_independent_rounding():
    vals = OF8.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                      # exact in fp32
    rng = np.random.default_rng(8)
    rand = np.concatenate([
        rng.standard_normal(4000) * s for s in (1e-3, 0.03, 1.0, 30.0, 300.0)])
    xs = np.concatenate([mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20), rand,
                         [448.0, 460.0, 463.9, 464.0, 470.0, 1e30, 2.0 ** -10, 2.0 ** -10 * 1.001,
                          3 * 2.0 ** -10, 0.0]])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    got = OF8.f32_to_e4m3(xs)
    want = np.array([_encode_ref(float(x)) for x in xs], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_e4m3_saturation_and_nan():
    x = np.array([np.inf, -np.inf, np.nan, 1e38, -1e38, 448.0, -448.0], dtype=np.float32)
    assert list(OF8.f32_to_e4m3(x)) == [0x7E, 0xFE, 0x7F, 0x7E, 0xFE, 0x7E, 0xFE]


def pin_quantize_divides_in_fp32():
    rng = np.random.default_rng(9)
    x = W.randn_bf16(rng, (512,))
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(OF8.quantize(x, 1.0), OF8.f32_to_e4m3(xf))
    assert np.array_equal(OF8.quantize(x, 0.25), OF8.f32_to_e4m3(xf * np.float32(4)))
    s = np.float32(0.0371)
    assert np.array_equal(OF8.quantize(x, s), OF8.f32_to_e4m3(xf / s))


def _fp8_case(seed, Hkv=2, G=2, D=16, BS=16, causal=True):
    rng = np.random.default_rng(seed)
    q_lens = np.array([5, 1, 9], np.int32)
    k_lens = np.array([5, 30, 40], np.int32)
    B, H = len(q_lens), G * Hkv
    nblk = [(int(k) + BS - 1) // BS for k in k_lens]
    NB = sum(nblk) + 2
    perm = rng.permutation(NB)
    MB = max(nblk)
    bt = np.full((B, MB), -1, np.int32)
    c = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = W.randn_bf16(rng, (int(cu[-1]), H, D))
    codes = rng.integers(0, 256, size=(2, NB, BS, Hkv, D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                    # no NaN codes
    return q, codes, cu, k_lens, bt, np.float32(1 / math.sqrt(D)), causal


def pin_fp8_attention_reduces_to_bf16():
    """With unit scales the E4M3 path equals the bf16 path on the same values
    (every E4M3 value is exact in bf16)."""
    q, codes, cu, sk, bt, scale, causal = _fp8_case(11)
    Hkv = codes.shape[3]
    vals = OF8.e4m3_to_f64(codes).astype(np.float32)
    bits = W.f32_to_bf16_bits(vals)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), vals)
    o8, l8 = OA.varlen_attention(q, codes, cu, sk, bt, scale, causal,
                                 k_scale=np.ones(Hkv), v_scale=np.ones(Hkv))
    ob, lb = OA.varlen_attention(q, bits, cu, sk, bt, scale, causal)
    assert np.allclose(o8, ob, rtol=0, atol=1e-12) and np.allclose(l8, lb, rtol=0, atol=1e-12)


def pin_fp8_attention_scales():
    """k_scale multiplies the scores of its KV head (same as scaling the
    softmax scale), v_scale multiplies that head's output and leaves the LSE."""
    q, codes, cu, sk, bt, scale, causal = _fp8_case(12)
    Hkv = codes.shape[3]
    H = q.shape[1]
    G = H // Hkv
    one = np.ones(Hkv)
    ks = np.array([0.5, 2.0], np.float32)
    vs = np.array([3.0, 0.125], np.float32)
    o1, l1 = OA.varlen_attention(q, codes, cu, sk, bt, scale, causal, k_scale=one, v_scale=one)
    for h in range(Hkv):
        oh, lh = OA.varlen_attention(q, codes, cu, sk, bt, np.float32(scale * ks[h]), causal,
                                     k_scale=one, v_scale=one)
        o2, l2 = OA.varlen_attention(q, codes, cu, sk, bt, scale, causal, k_scale=ks, v_scale=vs)
        heads = slice(h * G, (h + 1) * G)
        fin = ~np.isneginf(lh[:, heads])
        assert np.allclose(o2[:, heads], oh[:, heads] * vs[h], rtol=1e-12, atol=1e-12)
        assert np.allclose(l2[:, heads][fin], lh[:, heads][fin], rtol=0, atol=1e-12)
    assert not np.allclose(o1, OA.varlen_attention(q, codes, cu, sk, bt, scale, causal,
                                                   k_scale=ks, v_scale=one)[0])


def pin_reshape_and_cache_fp8():
    """Scatter then gather returns every token's quantised rows (per-head
    scales), untouched slots keep their bytes, negative slots are skipped."""
    rng = np.random.default_rng(13)
    T, Hkv, D, NB, BS = 10, 2, 8, 4, 16
    key = W.randn_bf16(rng, (T, Hkv, D))
    value = W.randn_bf16(rng, (T, Hkv, D))
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[3] = -1
    ks = np.array([0.02, 0.5], np.float32)
    vs = np.array([0.25, 0.03], np.float32)      # |x| / scale stays below 448
    before = rng.integers(0, 256, size=(2, NB, BS, Hkv, D), dtype=np.uint8)
    after = OF8.reshape_and_cache_fp8(key, value, before, slots, ks, vs)
    written = np.zeros(NB * BS, bool)
    written[slots[slots >= 0]] = True
    fa, fb = after.reshape(2, NB * BS, Hkv, D), before.reshape(2, NB * BS, Hkv, D)
    assert np.array_equal(fa[:, ~written], fb[:, ~written])
    for t in range(T):
        if slots[t] < 0:
            continue
        for h in range(Hkv):
            assert np.array_equal(fa[0, slots[t], h], OF8.quantize(key[t, h], ks[h]))
            assert np.array_equal(fa[1, slots[t], h], OF8.quantize(value[t, h], vs[h]))
            back = OF8.dequantize(fa[1, slots[t], h], vs[h])
            xv = (value[t, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            # within half a step of E4M3 (relative 2^-4) or the subnormal step
            assert np.all(np.abs(back - xv) <= np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * vs[h]) * 1.0001)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
