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


def _scale_dropped(q, kv_cache, cu, sk, bt, scale, causal, num_kv_heads=None):
    return _orig_varlen(q, kv_cache, cu, sk, bt, 1.0, causal, num_kv_heads)


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
