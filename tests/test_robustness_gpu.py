"""GPU checks of behaviour around the hot path, through the C ABI against the
fp64 oracle:

* device-side contents out of range: a slot at or past num_blocks *
  block_size is skipped by the cache write like a negative one, and a
  block-table entry outside [0, num_blocks) is not followed (its keys and
  values read as zeros, which the oracle states as an extra all-zero block);
* the host cascade decision ("FlashAttention 在 vLLM 中的实现分析", section
  6.2) followed end to end: decide, run the chosen path, compare with the
  oracle's single pass;
* the calls captured into a HIP graph and replayed (the ahead-of-time
  schedule of section 7 exists so that they can be): every replay, with the
  program's own eager work between replays, matches the oracle;
* the work-list upload kernel copies exactly, and refuses host memory the
  device cannot read."""
import ctypes

import numpy as np
import pytest
import torch

import oracle.attention as OA
from paged_kv_varlen_flash_amd import ops, workloads as W
from gpu_harness import compare, run_library, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import os
    assert os.path.exists(ops.LIB_PATH), "libpagedattn.so is not built"


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


# ------------------------------------------------------------ out-of-range slots
def test_reshape_and_cache_skips_slots_past_the_cache():
    say("reshape_and_cache: slots >= NB*BS and < 0 skipped")
    wl = W.make("tiny_mixed")
    T = wl.T
    NBS = wl.num_blocks * wl.BS
    slots = wl.slot_mapping.copy()
    slots[[0, 5, 11]] = NBS + np.array([0, 3, 1000])
    slots[[2, 7]] = -1
    cache = _dev_bf16(wl.kv_cache)
    ops.pa_reshape_and_cache(_dev_bf16(wl.key), _dev_bf16(wl.value), cache,
                             torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ref_slots = np.where(slots >= NBS, -1, slots)
    ref = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, ref_slots)
    assert np.array_equal(W.bf16_tensor_bits(cache), ref)
    assert T == len(slots)


# ------------------------------------------------------------ out-of-range block entries
# D, G, Hkv, BS, causal, (Lq, Lk) per sequence, cache format
BAD_ENTRY = [
    (128, 4, 2, 16, True, ((1, 300), (1, 45), (70, 400)), "bf16"),     # small + tiled items
    (64, 8, 1, 16, True, ((1, 200), (40, 170)), "bf16"),               # D = 64 tiled loader
    (256, 2, 2, 64, True, ((1, 500), (20, 300)), "bf16"),
    (128, 4, 2, 32, True, ((1, 300), (60, 260)), "e4m3"),              # E4M3 loaders
    (128, 4, 1, 32, True, ((2100, 2300), (2050, 2050)), "bf16"),       # DMA loads, no decode rows
    (128, 4, 1, 48, True, ((2100, 2300), (2050, 2050)), "bf16"),       # 256-row blocks (BS = 48)
]


@pytest.mark.parametrize("case", range(len(BAD_ENTRY)))
def test_block_entry_out_of_range_reads_zeros(case):
    D, G, Hkv, BS, causal, seqs, fmt = BAD_ENTRY[case]
    say(f"bad block entries case={case} D={D} G={G} BS={BS} seqs={seqs} {fmt}")
    rng = np.random.default_rng(8100 + case)
    H = G * Hkv
    q_lens = np.array([a for a, _ in seqs], np.int32)
    k_lens = np.array([b for _, b in seqs], np.int32)
    B = len(seqs)
    nblk = [(int(k) + BS - 1) // BS for k in k_lens]
    NB = sum(nblk) + 2
    perm = rng.permutation(NB).astype(np.int32)
    MB = max(nblk)
    bt = np.full((B, MB), -1, np.int32)
    c = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    # one entry past the cache and one negative entry inside each sequence's range
    bad = bt.copy()
    for b in range(B):
        bad[b, nblk[b] // 2] = NB + 7 + b
        if nblk[b] > 2:
            bad[b, nblk[b] - 1] = -5
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = W.randn_bf16(rng, (T, H, D))
    scale = np.float32(1.0 / np.sqrt(D))
    # the oracle's cache: one more block, all zeros, where the bad entries point
    oracle_bt = np.where((bad < 0) | (bad >= NB), NB, bad).astype(np.int32)
    for b in range(B):
        oracle_bt[b, nblk[b]:] = -1
    p = ops.make_params(B, H, Hkv, D, BS, NB, MB, causal, scale)
    plan = ops.VarlenPlan(p, cu, k_lens, 0)
    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    targs = (torch.from_numpy(cu).cuda(), torch.from_numpy(k_lens).cuda(),
             torch.from_numpy(bad).cuda())
    if fmt == "bf16":
        cache = W.randn_bf16(rng, (2, NB, BS, Hkv, D))
        ops.varlen_fwd(_dev_bf16(q), _dev_bf16(cache), *targs, plan, out=out, lse=lse)
        ocache = np.concatenate([cache, np.zeros((2, 1, BS, Hkv, D), np.uint16)], axis=1)
        ref_out, ref_lse = OA.varlen_attention(q, ocache, cu, k_lens, oracle_bt, scale, causal)
    else:
        # codes of magnitude 0x00..0x57 (|value| <= 15) with random signs, as
        # the workloads draw them
        shape = (2, NB, BS, Hkv, D)
        codes = (rng.integers(0, 0x58, size=shape, dtype=np.uint8)
                 | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)).astype(np.uint8)
        ks, vs = W.fp8_scales(Hkv, 8200 + case)
        ops.varlen_fwd(_dev_bf16(q), torch.from_numpy(codes).cuda(), *targs, plan, out=out,
                       lse=lse, k_scale=torch.from_numpy(ks).cuda(),
                       v_scale=torch.from_numpy(vs).cuda())
        ocodes = np.concatenate([codes, np.zeros((2, 1, BS, Hkv, D), np.uint8)], axis=1)
        ref_out, ref_lse = OA.varlen_attention(q, ocodes, cu, k_lens, oracle_bt, scale, causal,
                                               k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            label=f"bad entries {case}")


# ------------------------------------------------------------ cascade decision end to end
@pytest.mark.parametrize("name,expect_cascade", [("cascade_prefix", False),
                                                 ("cascade_prefix_16k", True)])
def test_cascade_decision_end_to_end(name, expect_cascade):
    """pa_cascade_decide on the host, then the path it chose, against the
    oracle's single pass: a 2048-token prefix over 32 requests stays single
    pass on this chip (the prefix is re-read from the last-level cache), a
    16384-token prefix over 64 requests takes the cascade."""
    say(f"cascade decision {name}")
    wl = W.make(name)
    d = W.to_device(wl)
    ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale, num_cus=ops.device_cus())
    P, use = ops.pa_cascade_decide(p, wl.cu_seqlens_q, wl.k_lens, wl.block_table)
    say(f"  decision: common_prefix_len={P} use_cascade={use}")
    assert P == wl.spec.shared_prefix
    assert use == expect_cascade
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    if use:
        cplan = ops.CascadePlan(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                                tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens,
                                wl.scale, P)
        ops.cascade_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["block_table"], cplan,
                        out=out, lse=lse)
    else:
        plan = ops.plan_varlen(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                               tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens,
                               wl.scale, True)
        ops.varlen_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"],
                       d["block_table"], plan, out=out, lse=lse)
    torch.cuda.synchronize()
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            label=f"{name} {'cascade' if use else 'single pass'}")


# ------------------------------------------------------------ graph capture
def _replays(g, check, reset, n=4):
    for k in range(n):
        reset()                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {k}")


def test_graph_capture_scatter_attention():
    """reshape_and_cache + varlen_fwd (split into 2 pieces per unit, so the
    split reduce is in the graph too) captured once and replayed: the
    outputs are poisoned with NaN by eager fills between replays."""
    say("graph capture: scatter + attention (forced splits)")
    wl = W.make("tiny_mixed")
    d = W.to_device(wl)
    ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    plan = ops.plan_varlen(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                           tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens,
                           wl.scale, True, force_splits=2)
    assert plan.info.num_reduce_items > 0
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ops.varlen_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"], d["block_table"],
                   plan, out=out, lse=lse)       # eager warm-up of every kernel
    torch.cuda.synchronize()
    cache0 = d["kv_cache"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
        ops.varlen_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"],
                       d["block_table"], plan, out=out, lse=lse)
    ref_cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, ref_cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)
    sentinel = torch.from_numpy(wl.kv_cache.view(np.int16)).cuda().view(torch.bfloat16)

    def reset():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        d["kv_cache"].copy_(sentinel)            # new-token slots back to NaN

    def check(label):
        assert np.array_equal(W.bf16_tensor_bits(d["kv_cache"]), ref_cache), label
        compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label=label)

    _replays(g, check, reset)
    # bit patterns (the slack slots hold NaN sentinels)
    assert torch.equal(d["kv_cache"].view(torch.int16), cache0.view(torch.int16))


def test_graph_capture_cascade():
    """Prefix pass + suffix pass + merge_attn_states captured once and
    replayed, against the oracle's single pass."""
    say("graph capture: cascade")
    wl = W.make("cascade_prefix")
    d = W.to_device(wl)
    ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    cplan = ops.CascadePlan(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                            tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens, wl.scale,
                            wl.spec.shared_prefix)
    bufs = dict(out=torch.empty_like(d["q"]), prefix_out=torch.empty_like(d["q"]),
                suffix_out=torch.empty_like(d["q"]))
    for k in ("lse", "prefix_lse", "suffix_lse"):
        bufs[k] = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    ops.cascade_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["block_table"], cplan, **bufs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.cascade_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["block_table"], cplan,
                        **bufs)
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)

    def reset():
        for t in bufs.values():
            t.fill_(float("nan"))

    def check(label):
        compare(bufs["out"].float().cpu().numpy(), bufs["lse"].cpu().numpy(), ref_out, ref_lse,
                label=label)

    _replays(g, check, reset)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 70001])
def test_upload_words_copies_exactly(n):
    """pa_upload_words: the device copy of a pinned host buffer equals it word
    for word, for sizes that end inside a 16-byte chunk too."""
    say(f"upload words n={n}")
    rng = np.random.default_rng(9000 + n)
    host = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, size=n, dtype=np.int32)).pin_memory()
    dev = torch.full((n,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ops.pa_upload_words(host, dev)
    torch.cuda.synchronize()
    assert torch.equal(dev.cpu(), host)


def test_upload_words_rejects_unpinned_host_memory():
    """A host buffer the device cannot read is an error, not a launch."""
    host = np.arange(64, dtype=np.int32)
    dev = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = ops.lib().pa_upload_words(host.ctypes.data_as(ctypes.c_void_p),
                                   ctypes.c_void_p(dev.data_ptr()), 64, None)
    torch.cuda.synchronize()
    assert st == 1
    assert int(dev.abs().sum()) == 0
