"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

reshape_and_cache is compared bit for bit; out within 1e-2 max-abs and lse
within 1e-3 max-abs, element by element.  Outputs are pre-filled with NaN so
an element the kernels never write fails the comparison.  The five
workloads run at full size in the launch configuration the benchmark uses;
the long-context one is checked on a seeded sample of 4 sequences."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from paged_kv_varlen_flash_amd import ops, workloads as W
from gpu_harness import compare, run_library, say, sub_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import os
    assert os.path.exists(ops.LIB_PATH), "libpagedattn.so is not built"


# ------------------------------------------------------------ reshape_and_cache
@pytest.mark.parametrize("name", ["tiny_mixed", "decode_llama8b", "chunked_prefill_mix",
                                  "cascade_prefix"])
def test_reshape_and_cache_bitexact(name):
    say(f"reshape_and_cache {name}")
    wl = W.make(name)
    d = W.to_device(wl)
    ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    torch.cuda.synchronize()
    got = W.bf16_tensor_bits(d["kv_cache"])
    ref = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    assert np.array_equal(got, ref)


def test_reshape_and_cache_strided_and_skipped():
    """Token rows with a row stride wider than Hkv*D (a slice of a fused QKV
    buffer) and padding tokens with slot -1."""
    say("reshape_and_cache strided/skip")
    wl = W.make("tiny_mixed")
    T, Hkv, D = wl.key.shape
    rng = np.random.default_rng(3)
    slots = wl.slot_mapping.copy()
    slots[rng.choice(T, 5, replace=False)] = -1
    fused = np.full((T, 3, Hkv, D), 0x1357, np.uint16)      # [T, (q,k,v)-ish, Hkv, D]
    fused[:, 1] = wl.key
    fused[:, 2] = wl.value
    dev = torch.from_numpy(fused.view(np.int16)).cuda().view(torch.bfloat16)
    key, value = dev[:, 1], dev[:, 2]
    assert key.stride(0) == 3 * Hkv * D
    cache = torch.from_numpy(wl.kv_cache.view(np.int16)).cuda().view(torch.bfloat16)
    sm = torch.from_numpy(slots).cuda()
    ops.pa_reshape_and_cache(key, value, cache, sm)
    torch.cuda.synchronize()
    ref = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, slots)
    assert np.array_equal(W.bf16_tensor_bits(cache), ref)


# ------------------------------------------------------------ attention
@pytest.mark.parametrize("name", ["tiny_mixed", "decode_llama8b", "chunked_prefill_mix",
                                  "chunked_prefill_mix_prefill", "cascade_prefix",
                                  "prefill_causal_8k"])
def test_varlen_fwd_workload(name):
    say(f"varlen_fwd {name}")
    wl = W.make(name)
    out, lse, d, plan = run_library(wl)
    say(f"  plan: {plan.info.as_dict()}")
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, wl.causal)
    compare(out, lse, ref_out, ref_lse, label=name)


def test_varlen_fwd_long_context_sample():
    """16 sequences of 32K-128K keys, D=256, GQA 8, split-KV; oracle on a
    seeded sample of 4 sequences."""
    say("varlen_fwd long_decode_d256 (generating ~2.7 GB of KV)")
    wl = W.make("long_decode_d256")
    out, lse, d, plan = run_library(wl)
    say(f"  plan: {plan.info.as_dict()}")
    assert plan.info.num_reduce_items > 0
    seqs = W.sample_sequences(wl, 4)
    cache_after = W.bf16_tensor_bits(d["kv_cache"])
    ref = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    assert np.array_equal(cache_after, ref)
    rows, cu, sk, bt = sub_problem(wl, seqs)
    ref_out, ref_lse = OA.varlen_attention(wl.q[rows], cache_after, cu, sk, bt, wl.scale, True)
    compare(out[rows], lse[rows], ref_out, ref_lse, label=f"long seqs {seqs}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_forced_splits(splits):
    say(f"forced splits {splits}")
    wl = W.make("tiny_mixed")
    out, lse, d, plan = run_library(wl, force_splits=splits)
    if splits > 1:
        assert plan.info.num_reduce_items > 0
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)
    compare(out, lse, ref_out, ref_lse, label=f"splits={splits}")


def test_cascade_equals_single_pass():
    """Prefix pass + suffix pass + merge (through the library) against the
    oracle's single pass and the library's own single pass."""
    say("cascade_prefix cascade vs single pass")
    wl = W.make("cascade_prefix")
    single_out, single_lse, d, _ = run_library(wl)
    cplan = ops.CascadePlan(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                            tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens, wl.scale,
                            wl.spec.shared_prefix)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ops.cascade_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["block_table"], cplan,
                    out=out, lse=lse)
    torch.cuda.synchronize()
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label="cascade")
    assert np.abs(out.float().cpu().numpy() - single_out).max() <= 2e-2


# ------------------------------------------------------------ fuzz
def _fuzz_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3]))
    BS = int(rng.choice([16, 32, 48, 64]))
    causal = bool(rng.integers(0, 2))
    B = int(rng.integers(1, 7))
    fixed = []
    for _ in range(B):
        kind = rng.integers(0, 4)
        if kind == 0:
            lk = int(rng.integers(0, 300))
            fixed.append((1, max(lk, 1)))
        elif kind == 1:
            lq = int(rng.integers(1, 70))
            fixed.append((lq, lq + int(rng.integers(0, 200))))
        elif kind == 2:
            lq = int(rng.integers(1, 4))                  # speculative-decode-like
            fixed.append((lq, lq + int(rng.integers(0, 500))))
        else:
            lk = int(rng.integers(0, 20))
            fixed.append((int(rng.integers(1, 30)), lk))  # may have Lq > Lk
    spec = W.Spec(name=f"fuzz{seed}", num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                  block_size=BS, causal=causal, seed=5000 + seed, fixed=tuple(fixed),
                  min_num_blocks=3)
    return spec


@pytest.mark.parametrize("seed", range(24))
def test_fuzz(seed):
    spec = _fuzz_case(seed)
    say(f"fuzz seed={seed} D={spec.head_size} H={spec.num_heads} Hkv={spec.num_kv_heads} "
        f"BS={spec.block_size} causal={spec.causal} seqs={spec.fixed}")
    rng = np.random.default_rng(seed)
    force = int(rng.choice([0, 0, 2, 5]))
    _check_case(spec, rng, force, f"fuzz{seed}")


# Scores spread over hundreds of natural-log units: a row maximum taken over
# only part of a row's keys (a wrong cross-lane exchange) overflows exp2, and
# a wrong reference shifts the LSE.  Decode rows (small-row kernel: maxima
# across 16- and 32-lane groups) and prefill rows (tiled kernel).
EXTREME = [
    # D, G, Hkv, BS, causal, (Lq, Lk) per sequence, q multiplier, scale multiplier
    (128, 4, 2, 16, True, ((1, 700), (1, 40), (2, 300)), 8.0, 4.0),
    (128, 4, 2, 32, True, ((100, 100), (40, 500)), 8.0, 4.0),
    (64, 8, 1, 16, False, ((1, 200), (60, 90)), 6.0, 6.0),
    (256, 8, 2, 64, True, ((1, 1000), (30, 200)), 6.0, 3.0),
]


@pytest.mark.parametrize("case", range(len(EXTREME)))
def test_extreme_scores(case):
    D, G, Hkv, BS, causal, seqs, qmul, smul = EXTREME[case]
    spec = W.Spec(name=f"extreme{case}", num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                  block_size=BS, causal=causal, seed=7300 + case, fixed=seqs, min_num_blocks=3)
    say(f"extreme scores case={case} D={D} G={G} seqs={seqs} q x{qmul} scale x{smul}")
    _check_case(spec, np.random.default_rng(7300 + case), 0, f"extreme{case}", qmul=qmul,
                smul=smul)


# Batches whose every sequence has more than 16 rows (query tokens x heads
# per KV head), so that the launch holds tiled items only: ragged tails,
# rows that see no key (Lq > Lk under the causal mask), split key ranges.
PREFILL_ONLY = [
    # D, G, Hkv, BS, causal, (Lq, Lk) per sequence, forced splits
    (128, 4, 2, 32, True, ((300, 300), (77, 200), (5, 5), (129, 1000)), 0),
    (128, 4, 2, 16, False, ((64, 64), (33, 97), (200, 450)), 3),
    (64, 8, 1, 48, True, ((40, 40), (17, 300), (250, 260)), 0),
    (64, 2, 3, 64, False, ((100, 130), (9, 9)), 2),
    (128, 1, 2, 16, True, ((600, 600), (20, 10)), 5),
    (256, 4, 1, 32, True, ((70, 70), (33, 180)), 0),
    # long enough for 256-row blocks at D = 128 (2048+ query tokens on average):
    # one token per row at G = 1, eight rows per token at G = 8, rows that see
    # no key where Lq > Lk, block sizes 16 to 128 and 48
    (128, 4, 2, 32, True, ((2100, 2100), (2050, 2400)), 0),
    (128, 4, 2, 16, False, ((2300, 2300), (1900, 2000)), 3),
    (128, 1, 3, 64, True, ((2500, 2400), (1700, 1900)), 0),
    (128, 8, 1, 128, True, ((2049, 4100), (2100, 2100)), 2),
    (128, 4, 2, 48, True, ((2100, 2100), (2050, 2400)), 0),
    # LDS-DMA tiles (32 keys) inside 256-token blocks, split into forced
    # pieces whose ends fall inside a tile, and short prefills
    (128, 4, 2, 256, True, ((333, 333), (45, 1000), (5, 77), (130, 531)), 3),
    (128, 2, 4, 128, False, ((97, 1201), (300, 300)), 7),
]


@pytest.mark.parametrize("case", range(len(PREFILL_ONLY)))
def test_prefill_only(case):
    D, G, Hkv, BS, causal, seqs, force = PREFILL_ONLY[case]
    spec = W.Spec(name=f"prefill_only{case}", num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                  block_size=BS, causal=causal, seed=7000 + case, fixed=seqs, min_num_blocks=3)
    say(f"prefill-only case={case} D={D} G={G} Hkv={Hkv} BS={BS} causal={causal} seqs={seqs} "
        f"force={force}")
    plan = _check_case(spec, np.random.default_rng(7000 + case), force, f"prefill_only{case}")
    assert plan.info.num_small_items == 0 and plan.info.num_tiled_items > 0
    # 256-row blocks (8-wave workgroups) at D = 64, or for long prefills at
    # D = 128 unless the DMA kernel runs them (power-of-two block size)
    wide = D <= 64 or (D <= 128 and np.mean([q for q, _ in seqs]) >= 2048 and BS & (BS - 1) != 0)
    assert plan.info.tiled_rows == (256 if wide else 128)


# Degenerate batches: sequences with no query tokens (anywhere in the
# batch, or every one: nothing to compute, nothing written), sequences with
# no keys (rows with no visible key: out 0, lse -inf), one-key decodes, a
# 256-token block size, and a batch of 1024 short decodes.
DEGENERATE = [
    # D, G, Hkv, BS, causal, (Lq, Lk) per sequence
    (128, 4, 2, 32, True, ((0, 100), (1, 50), (0, 0), (5, 5), (40, 300), (0, 7))),
    (64, 4, 2, 16, True, ((0, 0), (0, 30), (0, 1))),
    (128, 4, 2, 16, False, ((1, 0), (3, 0), (20, 0))),
    (128, 8, 1, 16, True, ((1, 0), (1, 1), (1, 1), (2, 1))),
    (128, 4, 2, 256, True, ((1, 700), (300, 900), (1, 256), (257, 257))),
    (128, 4, 2, 16, True, tuple((1, 64) for _ in range(1024))),
]


@pytest.mark.parametrize("case", range(len(DEGENERATE)))
def test_degenerate_batches(case):
    D, G, Hkv, BS, causal, seqs = DEGENERATE[case]
    spec = W.Spec(name=f"degenerate{case}", num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                  block_size=BS, causal=causal, seed=7600 + case, fixed=seqs, min_num_blocks=3)
    say(f"degenerate case={case} D={D} G={G} Hkv={Hkv} BS={BS} causal={causal} "
        f"seqs={seqs[:6]}{'...' if len(seqs) > 6 else ''} ({len(seqs)} sequences)")
    plan = _check_case(spec, np.random.default_rng(7600 + case), 0, f"degenerate{case}")
    if sum(q for q, _ in seqs) == 0:
        assert plan.info.num_small_items + plan.info.num_tiled_items == 0


def _check_case(spec, rng, force, label, qmul=1.0, smul=1.0):
    q_lens = np.array([a for a, _ in spec.fixed], np.int32)
    k_lens = np.array([b for _, b in spec.fixed], np.int32)
    B, H, Hkv, D, BS = len(q_lens), spec.num_heads, spec.num_kv_heads, spec.head_size, spec.block_size
    nblk = [(int(k) + BS - 1) // BS for k in k_lens]
    NB = sum(nblk) + 3
    perm = rng.permutation(NB).astype(np.int32)
    MB = max(max(nblk), 1)
    bt = np.full((B, MB), -1, np.int32)
    c = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = W.randn_bf16(rng, (T, H, D))
    if qmul != 1.0:                        # exact: a power of two times bf16, or rounded again
        q = W.f32_to_bf16_bits((q.astype(np.uint32) << 16).view(np.float32) * np.float32(qmul))
    cache = W.randn_bf16(rng, (2, NB, BS, Hkv, D))
    # slack slots hold NaN: they must never reach an output
    for b in range(B):
        for j in range(k_lens[b], nblk[b] * BS):
            cache[:, bt[b, j // BS], j % BS] = W.SENTINEL
    scale = np.float32(smul / np.sqrt(D))
    p = ops.make_params(B, H, Hkv, D, BS, NB, MB, spec.causal, scale)
    plan = ops.VarlenPlan(p, cu, k_lens, force)
    tq = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    tc = torch.from_numpy(cache.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full_like(tq, float("nan"))
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ops.varlen_fwd(tq, tc, torch.from_numpy(cu).cuda(), torch.from_numpy(k_lens).cuda(),
                   torch.from_numpy(bt).cuda(), plan, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = OA.varlen_attention(q, cache, cu, k_lens, bt, scale, spec.causal)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            label=f"{label} force={force}")
    return plan


# ------------------------------------------------------------ merge
@pytest.mark.parametrize("D", [64, 128, 256])
def test_merge_attn_states(D):
    say(f"merge D={D}")
    rng = np.random.default_rng(D)
    T, H = 37, 8
    po = W.randn_bf16(rng, (T, H, D))
    so = W.randn_bf16(rng, (T, H, D))
    pl = (rng.standard_normal((T, H)) * 4).astype(np.float32)
    sl = (rng.standard_normal((T, H)) * 4).astype(np.float32)
    pl[0, :3] = -np.inf
    sl[1, :3] = -np.inf
    pl[2, 0] = sl[2, 0] = -np.inf
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ops.pa_merge_attn_states(out, out_lse, dev(po), torch.from_numpy(pl).cuda(), dev(so),
                             torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = OA.merge_attn_states(OA.bf16_to_f64(po), pl.astype(np.float64),
                                        OA.bf16_to_f64(so), sl.astype(np.float64))
    compare(out.float().cpu().numpy(), out_lse.cpu().numpy(), ref_o, ref_l, label=f"merge D={D}")
    # in place: out aliases prefix_out
    pin = dev(po)
    ops.pa_merge_attn_states(pin, None, pin, torch.from_numpy(pl).cuda(), dev(so),
                             torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    assert torch.equal(pin, out)


# ------------------------------------------------------------ determinism
def test_deterministic_with_fixed_plan():
    say("determinism chunked_prefill_mix")
    wl = W.make("chunked_prefill_mix")
    out1, lse1, d, plan = run_library(wl)
    out2 = torch.empty_like(d["q"])
    lse2 = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ops.varlen_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"], d["block_table"],
                   plan, out=out2, lse=lse2)
    torch.cuda.synchronize()
    assert np.array_equal(out1.view(np.uint32), out2.float().cpu().numpy().view(np.uint32))
    assert np.array_equal(lse1.view(np.uint32), lse2.cpu().numpy().view(np.uint32))
