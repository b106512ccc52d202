"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one.  A mutant that no pin catches means the pins are too weak."""
import math

import numpy as np
import pytest

import oracle.attention as OA
import oracle_pins

_orig_visible = OA._visible
_orig_softmax = OA._softmax_rows
_orig_gather = OA.gather_kv
_orig_merge = OA.merge_states
_orig_varlen = OA.varlen_attention


def _top_left_visible(Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    i = np.arange(Lq)[:, None]
    return (j <= i) if causal else np.ones((Lq, Lk), bool)


def _off_by_one_visible(Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    i = np.arange(Lq)[:, None]
    return (j < i + (Lk - Lq)) if causal else np.ones((Lq, Lk), bool)


def _log2_lse(s, vis, v):
    out, lse = _orig_softmax(s, vis, v)
    return out, lse / math.log(2.0)


def _no_max_shift_in_lse(s, vis, v):
    out, lse = _orig_softmax(s, vis, v)
    m = np.where(vis, s, -np.inf).max(axis=1) if s.shape[1] else lse
    return out, np.where(np.isneginf(lse), lse, lse - m)


def _unnormalised(s, vis, v):
    out, lse = _orig_softmax(s, vis, v)
    fin = ~np.isneginf(lse)
    m = np.where(vis, s, -np.inf).max(axis=1) if s.shape[1] else lse
    l = np.where(fin, np.exp(lse - np.where(fin, m, 0.0)), 1.0)
    return out * l[:, None], lse


def _gather_swapped(cf, row, Lk):
    BS = cf.shape[2]
    j = np.arange(Lk)
    nb = max((Lk + BS - 1) // BS, 1)
    phys = row[np.minimum(j % nb, len(row) - 1)]
    off = np.minimum(j // nb, BS - 1)
    return cf[0, phys, off], cf[1, phys, off]


def _gather_kv_swapped_planes(cf, row, Lk):
    k, v = _orig_gather(cf, row, Lk)
    return v, k


def _merge_no_weights(outs, lses):
    o, l = _orig_merge(outs, lses)
    O = np.stack([np.asarray(x, float) for x in outs])
    return O.mean(axis=0), l


def _merge_log2(outs, lses):
    o, l = _orig_merge(outs, lses)
    L = np.stack([np.asarray(x, float) for x in lses])
    M = L.max(axis=0)
    return o, np.where(np.isneginf(l), l, M + np.log2(np.exp(l - np.where(np.isneginf(M), 0, M))))


def _scale_dropped(q, kv_cache, cu, sk, bt, scale, causal, num_kv_heads=None, **kw):
    return _orig_varlen(q, kv_cache, cu, sk, bt, 1.0, causal, num_kv_heads, **kw)


def _window_off_by_one(*args, sliding_window=0, **kw):
    return _orig_varlen(*args, sliding_window=(sliding_window + 1 if sliding_window else 0), **kw)


def _sink_dropped(*args, s_aux=None, **kw):
    return _orig_varlen(*args, **kw)


def _sink_as_value_one(*args, s_aux=None, **kw):
    out, lse = _orig_varlen(*args, s_aux=s_aux, **kw)
    if s_aux is None:
        return out, lse
    sink = np.asarray(s_aux, dtype=np.float64)[None, :]
    return out + np.exp(sink - lse)[..., None], lse


MUTANTS = {
    "gqa_modulo": ("_kv_head", lambda h, H, Hkv: h % Hkv),
    "causal_top_left": ("_visible", _top_left_visible),
    "causal_off_by_one": ("_visible", _off_by_one_visible),
    "lse_log2": ("_softmax_rows", _log2_lse),
    "lse_missing_max": ("_softmax_rows", _no_max_shift_in_lse),
    "out_unnormalised": ("_softmax_rows", _unnormalised),
    "block_index_swapped": ("gather_kv", _gather_swapped),
    "k_v_planes_swapped": ("gather_kv", _gather_kv_swapped_planes),
    "merge_unweighted": ("merge_states", _merge_no_weights),
    "merge_log2": ("merge_states", _merge_log2),
    "scale_dropped": ("varlen_attention", _scale_dropped),
    "window_off_by_one": ("varlen_attention", _window_off_by_one),
    "sink_dropped": ("varlen_attention", _sink_dropped),
    "sink_carries_a_value": ("varlen_attention", _sink_as_value_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


# ------------------------------------------------------------ FP8 (E4M3) path
import oracle.fp8 as OF8
import oracle_pins_fp8

_orig_dec = OF8.e4m3_to_f64
_orig_enc = OF8.f32_to_e4m3
_orig_quant = OF8.quantize


def _dec_bias8(codes):
    v = _orig_dec(codes)
    return v / 2.0


def _dec_no_subnormals(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = _orig_dec(c)
    e = (c.astype(np.int64) >> 3) & 0xF
    m = c.astype(np.int64) & 7
    sign = np.where(c & 0x80, -1.0, 1.0)
    return np.where(e == 0, sign * (1 + m / 8.0) * 2.0 ** -7, v)


def _enc_ties_away(x):
    x = np.asarray(x, dtype=np.float32)
    out = _orig_enc(x)
    # on an exact midpoint, step the even pick away from zero when it went down
    up = _orig_enc(x * np.float32(1 + 2.0 ** -22))
    mid = (out != up) & (np.abs(_orig_dec(out)) < np.abs(x.astype(np.float64)))
    return np.where(mid, up, out)


def _enc_no_saturation(x):
    x = np.asarray(x, dtype=np.float32)
    out = _orig_enc(x)
    big = np.abs(x) > 448
    return np.where(big, (out | 0x7F).astype(np.uint8), out)


def _quant_multiply(bits, scale):
    return _orig_quant(bits, 1.0 / float(np.float32(scale)))


def _attn_k_scale_ignored(*args, k_scale=None, v_scale=None, **kw):
    if k_scale is not None:
        k_scale = np.ones_like(np.asarray(k_scale, dtype=np.float32))
    return _orig_varlen(*args, k_scale=k_scale, v_scale=v_scale, **kw)


def _attn_scales_swapped(*args, k_scale=None, v_scale=None, **kw):
    return _orig_varlen(*args, k_scale=v_scale, v_scale=k_scale, **kw)


FP8_MUTANTS = {
    "e4m3_bias_8": (OF8, "e4m3_to_f64", _dec_bias8),
    "e4m3_no_subnormals": (OF8, "e4m3_to_f64", _dec_no_subnormals),
    "e4m3_ties_away": (OF8, "f32_to_e4m3", _enc_ties_away),
    "e4m3_no_saturation": (OF8, "f32_to_e4m3", _enc_no_saturation),
    "quantize_multiplies": (OF8, "quantize", _quant_multiply),
    "k_scale_ignored": (OA, "varlen_attention", _attn_k_scale_ignored),
    "k_v_scales_swapped": (OA, "varlen_attention", _attn_scales_swapped),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    mod, attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in oracle_pins_fp8.ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
