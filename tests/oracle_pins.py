"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form from the golden file, with the pure-Python brute force, with a
library routine on a special case, or with an invariant of the mathematics.
``test_oracle.py`` runs them against the oracle as written;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle (on the
CPU) and checks that at least one pin catches each."""
import json
import math
import os

import numpy as np

import oracle.attention as OA
import brute
from paged_kv_varlen_flash_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _bits(x):
    """float array -> bf16 bits, asserting every value is exact in bf16."""
    x = np.asarray(x, dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x), "golden input not exact in bf16"
    return bits


def golden_inputs(case):
    H, Hkv, D, BS, NB = case["H"], case["Hkv"], case["D"], case["BS"], case["NB"]
    seqs = case["seqs"]
    q = _bits(np.array(case["q"], dtype=np.float64).reshape(-1, H, D))
    cache = np.zeros((2, NB, BS, Hkv, D), dtype=np.uint16)
    mb = max(len(s["blocks"]) for s in seqs)
    bt = np.full((len(seqs), mb), -1, dtype=np.int32)
    cu = [0]
    lk = []
    for b, s in enumerate(seqs):
        bt[b, :len(s["blocks"])] = s["blocks"]
        cu.append(cu[-1] + s["Lq"])
        lk.append(s["Lk"])
        for j in range(s["Lk"]):
            blk = s["blocks"][j // BS]
            cache[0, blk, j % BS] = _bits(np.array(s["k"][j]).reshape(Hkv, D))
            cache[1, blk, j % BS] = _bits(np.array(s["v"][j]).reshape(Hkv, D))
    scale = case["scale"]
    scale = np.float32(math.log(2.0)) if scale == "ln2_f32" else np.float32(scale)
    return q, cache, np.array(cu, np.int32), np.array(lk, np.int32), bt, scale


def _lse_expect(x):
    return np.array([[(-np.inf if v is None else v) for v in row] for row in x], dtype=np.float64)


def _close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_inf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    assert not np.isnan(diff).any(), "nan in comparison"
    assert diff.max(initial=0.0) <= tol, f"max diff {diff.max()} > {tol}"


# ---------------------------------------------------------------- closed forms
def pin_golden_attention():
    for case in load_golden()["attention"]:
        q, cache, cu, lk, bt, scale = golden_inputs(case)
        out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, case["causal"])
        _close(out, np.array(case["expect_out"]), case["tol"])
        _close(lse, _lse_expect(case["expect_lse"]), case["tol"])


def pin_golden_merge():
    for case in load_golden()["merge"]:
        f = lambda v: -np.inf if v is None else v  # noqa: E731
        out, lse = OA.merge_attn_states(np.array([case["prefix_out"]]), np.array([f(case["prefix_lse"])]),
                                        np.array([case["suffix_out"]]), np.array([f(case["suffix_lse"])]))
        _close(out[0], np.array(case["expect_out"]), case["tol"])
        _close(lse, np.array([f(case["expect_lse"])]), case["tol"])


def pin_golden_cascade():
    for case in load_golden()["cascade"]:
        q, cache, cu, lk, bt, scale = golden_inputs(case)
        out, lse, _ = OA.cascade_attention(q, cache, cu, lk, bt, scale, case["common_prefix_len"])
        _close(out, np.array(case["expect_out"]), case["tol"])
        _close(lse, _lse_expect(case["expect_lse"]), case["tol"])


# ---------------------------------------------------------------- brute force
def random_case(seed, B=3, H=4, Hkv=2, D=8, BS=16, causal=True, max_lk=40, allow_q_gt_k=False):
    rng = np.random.default_rng(seed)
    q_lens, k_lens = [], []
    for _ in range(B):
        lk = int(rng.integers(0 if allow_q_gt_k else 1, max_lk + 1))
        hi = lk + 3 if allow_q_gt_k else lk
        lq = int(rng.integers(1, max(hi, 1) + 1))
        q_lens.append(lq)
        k_lens.append(lk)
    nblk = [(k + BS - 1) // BS for k in k_lens]
    NB = sum(nblk) + 2
    perm = rng.permutation(NB)
    bt = np.full((B, max(max(nblk), 1)), -1, dtype=np.int32)
    c = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = W.f32_to_bf16_bits(rng.standard_normal((T, H, D), dtype=np.float32))
    cache = W.f32_to_bf16_bits(rng.standard_normal((2, NB, BS, Hkv, D), dtype=np.float32))
    scale = np.float32(1.0 / math.sqrt(D))
    return q, cache, cu, np.array(k_lens, np.int32), bt, scale, causal


def pin_brute_force():
    for seed in range(6):
        for causal in (True, False):
            q, cache, cu, lk, bt, scale, causal = random_case(seed, causal=causal,
                                                              allow_q_gt_k=(seed % 2 == 1))
            out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal)
            bo, bl = brute.attention(q.tolist(), cache.tolist(), cu.tolist(), lk.tolist(),
                                     bt.tolist(), float(scale), causal)
            _close(out, np.array(bo), 1e-12)
            _close(lse, np.array(bl), 1e-12)


def pin_brute_force_merge():
    rng = np.random.default_rng(7)
    for n in (2, 3, 5):
        outs = rng.standard_normal((n, 6))
        lses = rng.standard_normal(n) * 3
        lses[rng.integers(0, n)] = -np.inf if n > 2 else lses[0]
        o, l = OA.merge_states([outs[k][None] for k in range(n)], [lses[k:k + 1] for k in range(n)])
        bo, bl = brute.merge([list(outs[k]) for k in range(n)], list(lses))
        _close(o[0], np.array(bo), 1e-12)
        _close(l, np.array([bl]), 1e-12)


# ---------------------------------------------------------------- library case
def pin_sdpa_special_case():
    """One sequence, identity block table: torch fp64 scaled_dot_product_attention
    with KV heads repeated and an explicit bottom-right mask."""
    import torch
    for (lq, lk, causal, H, Hkv) in ((5, 23, True, 4, 2), (7, 7, True, 2, 2), (3, 19, False, 8, 2)):
        rng = np.random.default_rng(lq * 100 + lk)
        D, BS = 16, 16
        nb = (lk + BS - 1) // BS
        q = W.f32_to_bf16_bits(rng.standard_normal((lq, H, D), dtype=np.float32))
        cache = W.f32_to_bf16_bits(rng.standard_normal((2, nb, BS, Hkv, D), dtype=np.float32))
        bt = np.arange(nb, dtype=np.int32)[None]
        scale = np.float32(0.3)
        out, lse = OA.varlen_attention(q, cache, np.array([0, lq]), np.array([lk]), bt, scale, causal)
        Q = torch.from_numpy(OA.bf16_to_f64(q)).permute(1, 0, 2)                   # [H, lq, D]
        Kc = torch.from_numpy(OA.bf16_to_f64(cache[0]).reshape(nb * BS, Hkv, D)[:lk])
        Vc = torch.from_numpy(OA.bf16_to_f64(cache[1]).reshape(nb * BS, Hkv, D)[:lk])
        K = Kc.repeat_interleave(H // Hkv, dim=1).permute(1, 0, 2).contiguous()
        V = Vc.repeat_interleave(H // Hkv, dim=1).permute(1, 0, 2).contiguous()
        i = torch.arange(lq)[:, None]
        j = torch.arange(lk)[None, :]
        mask = (j <= i + (lk - lq)) if causal else torch.ones(lq, lk, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=float(scale))
        s = float(scale) * torch.matmul(Q, K.transpose(1, 2).contiguous())
        ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)   # [H, lq]
        _close(out, ref.permute(1, 0, 2).numpy(), 1e-12)
        _close(lse, ref_lse.T.numpy(), 1e-12)


# ---------------------------------------------------------------- invariants
def pin_block_permutation():
    """Paged result == contiguous result under any permutation of physical blocks."""
    q, cache, cu, lk, bt, scale, causal = random_case(11, B=3, D=8)
    out0, lse0 = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal)
    NB = cache.shape[1]
    rng = np.random.default_rng(5)
    for _ in range(3):
        perm = rng.permutation(NB)         # new physical id of old block b = perm[b]
        c2 = np.empty_like(cache)
        c2[:, perm] = cache
        bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
        out, lse = OA.varlen_attention(q, c2, cu, lk, bt2, scale, causal)
        _close(out, out0, 0.0)
        _close(lse, lse0, 0.0)
    # contiguous: each sequence laid out in consecutive blocks 0..n-1 of its own cache
    for b in range(len(lk)):
        t0, t1 = cu[b], cu[b + 1]
        nb = max((int(lk[b]) + 15) // 16, 1)
        cc = cache[:, bt[b, :nb]] if lk[b] > 0 else cache[:, :1]
        o, l = OA.varlen_attention(q[t0:t1], cc, np.array([0, t1 - t0]), lk[b:b + 1],
                                   np.arange(nb, dtype=np.int32)[None], scale, causal)
        _close(o, out0[t0:t1], 0.0)
        _close(l, lse0[t0:t1], 0.0)


def pin_gqa_repeat():
    """Repeating each KV head H/Hkv times (Hkv' = H) leaves the result unchanged."""
    q, cache, cu, lk, bt, scale, causal = random_case(12, H=8, Hkv=2)
    out0, lse0 = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal)
    rep = np.repeat(cache, 4, axis=3)
    out, lse = OA.varlen_attention(q, rep, cu, lk, bt, scale, causal)
    _close(out, out0, 1e-13)
    _close(lse, lse0, 1e-13)


def pin_batch_permutation():
    q, cache, cu, lk, bt, scale, causal = random_case(13, B=4)
    out0, lse0 = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal)
    order = [2, 0, 3, 1]
    q_parts = [q[cu[b]:cu[b + 1]] for b in order]
    q2 = np.concatenate(q_parts)
    cu2 = np.concatenate([[0], np.cumsum([len(p) for p in q_parts])]).astype(np.int32)
    out, lse = OA.varlen_attention(q2, cache, cu2, lk[order], bt[order], scale, causal)
    ref_o = np.concatenate([out0[cu[b]:cu[b + 1]] for b in order])
    ref_l = np.concatenate([lse0[cu[b]:cu[b + 1]] for b in order])
    _close(out, ref_o, 0.0)
    _close(lse, ref_l, 0.0)


def pin_decode_causal_equals_noncausal():
    rng = np.random.default_rng(14)
    H, Hkv, D, BS = 4, 2, 8, 16
    lk = np.array([1, 17, 33, 5], np.int32)
    nb = (lk + BS - 1) // BS
    NB = int(nb.sum())
    bt = np.full((4, nb.max()), -1, np.int32)
    c = 0
    for b in range(4):
        bt[b, :nb[b]] = np.arange(c, c + nb[b])[::-1]
        c += nb[b]
    q = W.f32_to_bf16_bits(rng.standard_normal((4, H, D), dtype=np.float32))
    cache = W.f32_to_bf16_bits(rng.standard_normal((2, NB, BS, Hkv, D), dtype=np.float32))
    cu = np.arange(5, dtype=np.int32)
    a = OA.varlen_attention(q, cache, cu, lk, bt, np.float32(0.7), True)
    b_ = OA.varlen_attention(q, cache, cu, lk, bt, np.float32(0.7), False)
    _close(a[0], b_[0], 0.0)
    _close(a[1], b_[1], 0.0)


def pin_lse_is_log_rowsum():
    """lse == ln(sum_j exp(s_j)) evaluated with no max shift (small logits)."""
    q, cache, cu, lk, bt, scale, causal = random_case(15, B=2, D=8, causal=False)
    out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal)
    qf, cf = OA.bf16_to_f64(q), OA.bf16_to_f64(cache)
    H, Hkv = q.shape[1], cache.shape[3]
    for b in range(len(lk)):
        for t in range(cu[b], cu[b + 1]):
            for h in range(H):
                kvh = h // (H // Hkv)
                tot = 0.0
                acc = np.zeros(q.shape[2])
                for j in range(lk[b]):
                    blk = bt[b, j // 16]
                    e = math.exp(float(scale) * float(qf[t, h] @ cf[0, blk, j % 16, kvh]))
                    tot += e
                    acc += e * cf[1, blk, j % 16, kvh]
                assert abs(lse[t, h] - math.log(tot)) < 1e-12
                _close(out[t, h], acc / tot, 1e-12)


def pin_constant_v():
    q, cache, cu, lk, bt, scale, causal = random_case(16, B=3, D=8)
    c = cache.copy()
    c[1] = W.f32_to_bf16_bits(np.full(c[1].shape, -1.375, np.float32))
    out, lse = OA.varlen_attention(q, c, cu, lk, bt, scale, causal)
    vis = ~np.isneginf(lse)
    assert np.allclose(out[vis], -1.375, atol=1e-14, rtol=0)


def pin_split_invariance():
    """Splitting the keys into disjoint ranges, attending to each, and merging
    gives the unsplit result (the split-KV / distributed-merge identity)."""
    q, cache, cu, lk, bt, scale, _ = random_case(17, B=3, max_lk=48)
    out0, lse0 = OA.varlen_attention(q, cache, cu, lk, bt, scale, False)
    BS = cache.shape[2]
    # split at block boundaries: piece p covers blocks [c_p, c_{p+1})
    outs, lses = [], []
    maxb = bt.shape[1]
    cuts = [0] + [c for c in (1, 2) if c < maxb] + [maxb]
    for p in range(len(cuts) - 1):
        lo, hi = cuts[p], cuts[p + 1]
        lk_p = np.clip(lk - lo * BS, 0, (hi - lo) * BS).astype(np.int32)
        bt_p = bt[:, lo:hi] if hi > lo else bt[:, :1]
        o, l = OA.varlen_attention(q, cache, cu, lk_p, bt_p, scale, False)
        outs.append(o)
        lses.append(l)
    o, l = OA.merge_states(outs, lses)
    _close(o, out0, 1e-12)
    _close(l, lse0, 1e-12)


def pin_merge_symmetry_and_self():
    rng = np.random.default_rng(18)
    o1, o2 = rng.standard_normal((2, 5, 3, 8))
    l1, l2 = rng.standard_normal((2, 5, 3))
    a = OA.merge_attn_states(o1, l1, o2, l2)
    b = OA.merge_attn_states(o2, l2, o1, l1)
    _close(a[0], b[0], 1e-15)
    _close(a[1], b[1], 1e-15)
    s = OA.merge_attn_states(o1, l1, o1, l1)
    _close(s[0], o1, 1e-15)
    _close(s[1], l1 + math.log(2.0), 1e-14)


def pin_cascade_equals_single_pass():
    """Cascade (prefix pass + suffix pass + merge) equals one causal pass."""
    spec = W.Spec(name="t", num_heads=4, num_kv_heads=2, head_size=16, block_size=16,
                  causal=True, seed=77, groups=(("decode", 6, 3, 40),), shared_prefix=32)
    wl = W.make(spec)
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    out0, lse0 = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens, wl.block_table,
                                     wl.scale, True)
    out, lse, _ = OA.cascade_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens, wl.block_table,
                                       wl.scale, 32)
    _close(out, out0, 1e-12)
    _close(lse, lse0, 1e-12)


def pin_reshape_and_cache():
    """Scatter then gather through block_table returns every sequence's keys in
    token order; untouched slots keep their bits; negative slots are skipped."""
    wl = W.make("tiny_mixed")
    key, value = wl.key.copy(), wl.value.copy()
    sm = wl.slot_mapping.copy()
    sm_pad = np.concatenate([sm, [-1]])
    key_pad = np.concatenate([key, np.full((1,) + key.shape[1:], 0x1234, np.uint16)])
    val_pad = np.concatenate([value, np.full((1,) + value.shape[1:], 0x4321, np.uint16)])
    before = wl.kv_cache
    after = OA.reshape_and_cache(key_pad, val_pad, before, sm_pad)
    BS = wl.BS
    written = np.zeros(before.shape[1] * BS, dtype=bool)
    written[sm] = True
    flat_b = before.reshape(2, -1, *before.shape[3:])
    flat_a = after.reshape(2, -1, *after.shape[3:])
    assert np.array_equal(flat_a[:, ~written], flat_b[:, ~written])
    assert not np.any(flat_a == 0x1234) and not np.any(flat_a == 0x4321)
    for b in range(wl.B):
        Kb, Vb = W.sequence_kv(wl, b)
        Lk = int(wl.k_lens[b])
        j = np.arange(Lk)
        phys = wl.block_table[b, j // BS]
        assert np.array_equal(after[0, phys, j % BS], Kb)
        assert np.array_equal(after[1, phys, j % BS], Vb)


def pin_sliding_window_brute_force():
    for seed in range(4):
        q, cache, cu, lk, bt, scale, causal = random_case(40 + seed, max_lk=45,
                                                          allow_q_gt_k=(seed % 2 == 1))
        for win in (1, 5, 17):
            out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, True, sliding_window=win)
            bo, bl = brute.attention(q.tolist(), cache.tolist(), cu.tolist(), lk.tolist(),
                                     bt.tolist(), float(scale), True, window=win)
            _close(out, np.array(bo), 1e-12)
            _close(lse, np.array(bl), 1e-12)


def pin_sliding_window_limits():
    """A window of one key returns that key's value; a window at least as
    long as every context is no window."""
    q, cache, cu, lk, bt, scale, causal = random_case(50, max_lk=30)
    big = OA.varlen_attention(q, cache, cu, lk, bt, scale, True, sliding_window=1000)
    full = OA.varlen_attention(q, cache, cu, lk, bt, scale, True)
    _close(big[0], full[0], 0.0)
    _close(big[1], full[1], 0.0)
    out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, True, sliding_window=1)
    H = q.shape[1]
    for b in range(len(lk)):
        Lq, Lk = int(cu[b + 1] - cu[b]), int(lk[b])
        for i in range(Lq):
            j = i + Lk - Lq
            if j < 0:
                assert np.isneginf(lse[cu[b] + i]).all()
                continue
            K, V = OA.gather_kv(cache, bt[b], Lk)
            for h in range(H):
                kvh = h // (H // cache.shape[3])
                assert np.allclose(out[cu[b] + i, h], OA.bf16_to_f64(V[j, kvh]), atol=1e-12)


def pin_sinks_brute_force():
    rng = np.random.default_rng(60)
    for seed in range(4):
        q, cache, cu, lk, bt, scale, causal = random_case(60 + seed, allow_q_gt_k=(seed % 2 == 0))
        sinks = rng.standard_normal(q.shape[1]).astype(np.float32) * 2
        out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, causal, s_aux=sinks)
        bo, bl = brute.attention(q.tolist(), cache.tolist(), cu.tolist(), lk.tolist(),
                                 bt.tolist(), float(scale), causal, sinks=sinks.tolist())
        _close(out, np.array(bo), 1e-12)
        _close(lse, np.array(bl), 1e-12)


def pin_sinks_are_a_merge_with_an_empty_state():
    """A sink equals merging the attention with a state of out = 0 and
    lse = sink (a key with logit sink and value 0)."""
    q, cache, cu, lk, bt, scale, causal = random_case(70, allow_q_gt_k=True)
    sinks = np.array([0.5, -3.0, 4.0, 0.0], np.float32)
    out, lse = OA.varlen_attention(q, cache, cu, lk, bt, scale, True, s_aux=sinks)
    o0, l0 = OA.varlen_attention(q, cache, cu, lk, bt, scale, True)
    T, H, D = o0.shape
    mo, ml = OA.merge_states([o0, np.zeros_like(o0)], [l0, np.broadcast_to(sinks, (T, H))])
    _close(out, mo, 1e-12)
    _close(lse, ml, 1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
