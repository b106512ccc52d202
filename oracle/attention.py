"""fp64 CPU oracle for paged varlen attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The library (HIP kernels + C ABI) never calls it and
shares no code with it; it takes plain numpy arrays (bf16 held as uint16 bit
patterns) and returns float64 results.

What is computed, and where the pages define it:

* ``reshape_and_cache``: scatter the new tokens' K/V rows into the paged cache
  at ``slot_mapping`` ("FlashAttention 在 vLLM 中的实现分析", section 4.2; the
  helper-kernel table of section 8.2).  A negative slot is skipped (padding
  token; the pages are silent, this is the reading chosen for it).
* ``varlen_attention``: exact softmax attention per sequence over the keys
  gathered through ``block_table`` (section 5: logical block ->
  ``block_table[seq][logical_block]`` -> physical block -> offset), queries
  packed by ``cu_seqlens_q`` and keys limited to ``seqused_k`` (section 4, the
  standard decode/prefill call).  Tiling plus online softmax (section 1.1) is
  an exact reformulation of this, so the oracle is the plain definition:
  ``out = softmax(scale * q K^T) V`` over the visible keys and
  ``lse = ln sum_j exp(scale * q.k_j)`` (natural log; the backend-abstraction
  page, "境界と失敗", warns that ln and log2 must not be mixed).
  Readings where the pages are silent: query head h reads KV head
  ``h // (H // Hkv)``; causal masking is bottom-right aligned (query i of a
  sequence with Lq queries and Lk keys sees keys ``j <= i + Lk - Lq``); a
  query that sees no key gets ``out = 0`` and ``lse = -inf``.
* attention sinks (the ``s_aux`` argument of the FA3 path, "FlashAttention
  在 vLLM 中的实现分析" section 1.2, a learnable sink token): one logit per
  query head that joins the softmax denominator and carries no value:
  ``out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink_h})`` and
  ``lse = ln(sum_j e^{s_j} + e^{sink_h})``, where ``s_j`` are the scaled
  scores (the sink is in the same units).  A row with no visible key gets
  out = 0 and lse = sink_h.  Reading: the pages name the argument only.
* sliding window (named among the cascade conditions, section 6.2): with a
  window of W keys, query i sees keys ``i + Lk - Lq - (W - 1) <= j <= i + Lk - Lq``
  (the causal bound and the W - 1 keys before it); W = 0 means no window.
  Reading: the pages name the feature only; this is the usual decoder form.
* ``merge_states`` / ``merge_attn_states``: LSE-weighted merge of partial
  attentions over disjoint key sets (section 6.3, step 3).
* ``cascade_attention``: prefix pass (all queries as one pseudo-sequence,
  non-causal, over the first ``common_prefix_len / BS`` entries of block-table
  row 0), suffix pass (causal, over ``block_table[:, prefix_blocks:]``), then
  the merge (section 6.3).

Every function here is pinned by the ``-m "not gpu"`` tests (closed forms,
brute force, a library special case, invariants).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# reshape_and_cache
# --------------------------------------------------------------------------
def reshape_and_cache(key: np.ndarray, value: np.ndarray, kv_cache: np.ndarray,
                      slot_mapping: np.ndarray) -> np.ndarray:
    """Return a copy of ``kv_cache`` [2, NB, BS, Hkv, D] with token t's key and
    value rows written at slot ``slot_mapping[t]`` (block ``s // BS``, offset
    ``s % BS``).  Bit copy: dtype is preserved, nothing is converted."""
    out = kv_cache.copy()
    BS = kv_cache.shape[2]
    for t in range(key.shape[0]):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        out[0, s // BS, s % BS] = key[t]
        out[1, s // BS, s % BS] = value[t]
    return out


# --------------------------------------------------------------------------
# varlen attention
# --------------------------------------------------------------------------
def _kv_head(h: int, num_heads: int, num_kv_heads: int) -> int:
    """GQA grouping: contiguous groups of H/Hkv query heads share a KV head."""
    return h // (num_heads // num_kv_heads)


def _visible(Lq: int, Lk: int, causal: bool) -> np.ndarray:
    """Boolean [Lq, Lk]: may query i (0-based within its sequence) see key j?

    Bottom-right alignment: query i is token ``Lk - Lq + i`` of the sequence."""
    j = np.arange(Lk)[None, :]
    i = np.arange(Lq)[:, None]
    if not causal:
        return np.ones((Lq, Lk), dtype=bool)
    return j <= i + (Lk - Lq)


def gather_kv(kv_cache: np.ndarray, block_table_row: np.ndarray, Lk: int):
    """Keys/values 0..Lk-1 of one sequence: key j lives in physical block
    ``block_table_row[j // BS]`` at offset ``j % BS``.  Returns (K, V), each
    [Lk, Hkv, D], in the cache's dtype."""
    BS = kv_cache.shape[2]
    j = np.arange(Lk)
    phys = block_table_row[j // BS]
    off = j % BS
    return kv_cache[0, phys, off], kv_cache[1, phys, off]


def _softmax_rows(s: np.ndarray, vis: np.ndarray, v: np.ndarray):
    """Masked softmax of score rows s [R, Lk] times v [Lk, D].

    Returns (out [R, D], lse [R]); rows with no visible key give 0, -inf."""
    R = s.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full(R, NEG_INF, dtype=np.float64)
    any_vis = vis.any(axis=1)
    if not any_vis.any():
        return out, lse
    s = np.where(vis, s, NEG_INF)
    rows = np.nonzero(any_vis)[0]
    sr = s[rows]
    m = sr.max(axis=1, keepdims=True)
    w = np.exp(sr - m)                      # exp(-inf) = 0 for masked keys
    l = w.sum(axis=1, keepdims=True)
    out[rows] = (w @ v) / l
    lse[rows] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def varlen_attention(q: np.ndarray, kv_cache: np.ndarray, cu_seqlens_q: np.ndarray,
                     seqused_k: np.ndarray, block_table: np.ndarray, scale,
                     causal: bool, num_kv_heads: int = None, k_scale=None, v_scale=None,
                     s_aux=None, sliding_window: int = 0):
    """Paged varlen (GQA, optionally bottom-right causal) attention.

    q: bf16 bits [T, H, D]; kv_cache: bf16 bits (uint16) [2, NB, BS, Hkv, D],
    or E4M3 codes (uint8) of the same shape together with the per-KV-head
    fp32 dequantisation scales k_scale[Hkv], v_scale[Hkv] (key/value =
    E4M3 value * scale, see oracle.fp8);
    cu_seqlens_q: [B+1]; seqused_k: [B]; block_table: [B, max_blocks];
    scale: the fp32 softmax scale (promoted exactly to fp64);
    s_aux: None or fp32 [H] sink logits; sliding_window: W >= 0 keys (0 = none,
    causal only).
    Returns out float64 [T, H, D] and lse float64 [T, H] (natural log)."""
    T, H, D = q.shape
    Hkv = kv_cache.shape[3] if num_kv_heads is None else num_kv_heads
    scale = float(np.float32(scale))
    fp8 = np.asarray(kv_cache).dtype == np.uint8
    if fp8:
        from .fp8 import e4m3_to_f64
        ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
        vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)
        widen = lambda x, sc: e4m3_to_f64(x) * sc[None, :, None]
    elif k_scale is not None or v_scale is not None:
        raise ValueError("scales apply to an E4M3 (uint8) cache only")
    qf = bf16_to_f64(q)
    out = np.zeros((T, H, D), dtype=np.float64)
    lse = np.full((T, H), NEG_INF, dtype=np.float64)
    B = len(seqused_k)
    for b in range(B):
        t0, t1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        Lq, Lk = t1 - t0, int(seqused_k[b])
        if Lq == 0:
            continue
        Kb, Vb = gather_kv(kv_cache, np.asarray(block_table[b]), Lk)
        if fp8:
            K, V = widen(Kb, ks), widen(Vb, vs)
        else:
            K, V = bf16_to_f64(Kb), bf16_to_f64(Vb)
        vis = _visible(Lq, Lk, causal)
        if sliding_window:
            if not causal:
                raise ValueError("a sliding window is defined for causal attention")
            j = np.arange(Lk)[None, :]
            i = np.arange(Lq)[:, None]
            vis = vis & (j >= i + (Lk - Lq) - (int(sliding_window) - 1))
        for h in range(H):
            kvh = _kv_head(h, H, Hkv)
            s = scale * (qf[t0:t1, h, :] @ K[:, kvh, :].T)          # [Lq, Lk]
            o, l = _softmax_rows(s, vis, V[:, kvh, :])
            if s_aux is not None:
                # the sink's term joins the denominator: rescale by
                # e^{lse} / (e^{lse} + e^{sink}), in a stable form
                sink = float(np.float32(s_aux[h]))
                M = np.maximum(l, sink)
                a = np.where(np.isneginf(l), 0.0, np.exp(l - M))
                b = np.exp(sink - M)
                o = o * (a / (a + b))[:, None]
                l = M + np.log(a + b)
            out[t0:t1, h] = o
            lse[t0:t1, h] = l
    return out, lse


# --------------------------------------------------------------------------
# merges
# --------------------------------------------------------------------------
def merge_states(outs, lses):
    """n-ary LSE merge of partial attentions over disjoint key sets.

    outs: sequence of arrays [..., D]; lses: matching arrays [...].
    With M = max_k lse_k and a_k = exp(lse_k - M):
    out = sum_k a_k out_k / sum_k a_k, lse = M + ln sum_k a_k; if every
    lse_k is -inf the merged row is out = 0, lse = -inf."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])        # [n, ...]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])        # [n, ..., D]
    M = L.max(axis=0)
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    a = np.where(np.isneginf(L), 0.0, np.exp(L - Msafe))                 # [n, ...]
    den = a.sum(axis=0)
    den_safe = np.where(empty, 1.0, den)
    out = (a[..., None] * O).sum(axis=0) / den_safe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, NEG_INF, Msafe + np.log(den_safe))
    return out, lse


def merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse):
    """Two-way merge (the cascade's third step)."""
    return merge_states([prefix_out, suffix_out], [prefix_lse, suffix_lse])


# --------------------------------------------------------------------------
# cascade
# --------------------------------------------------------------------------
def cascade_attention(q, kv_cache, cu_seqlens_q, seqused_k, block_table, scale,
                      common_prefix_len: int, num_kv_heads: int = None):
    """Shared-prefix (cascade) attention: returns (out, lse, parts) where
    parts = (prefix_out, prefix_lse, suffix_out, suffix_lse).

    Prefix pass: all T query tokens form one pseudo-sequence over the
    ``common_prefix_len`` keys addressed by block-table row 0, non-causal.
    Suffix pass: each sequence over its remaining keys, addressed by
    ``block_table[:, prefix_blocks:]``, causal.  Then the LSE merge."""
    BS = kv_cache.shape[2]
    P = int(common_prefix_len)
    if P % BS:
        raise ValueError("common prefix must be a whole number of blocks")
    nblk = P // BS
    T = q.shape[0]
    cu_p = np.array([0, T], dtype=np.int64)
    p_out, p_lse = varlen_attention(q, kv_cache, cu_p, np.array([P]),
                                    np.asarray(block_table)[:1, :nblk], scale, False,
                                    num_kv_heads)
    s_out, s_lse = varlen_attention(q, kv_cache, cu_seqlens_q,
                                    np.asarray(seqused_k) - P,
                                    np.asarray(block_table)[:, nblk:], scale, True,
                                    num_kv_heads)
    out, lse = merge_attn_states(p_out, p_lse, s_out, s_lse)
    return out, lse, (p_out, p_lse, s_out, s_lse)
