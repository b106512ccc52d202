"""GPU parity of attention sinks (s_aux) and causal sliding windows through
the C ABI (pa_varlen_fwd_ex) against the fp64 oracle, on decode, prefill and
mixed batches, with and without split key ranges, on the bf16 and the E4M3
cache.  Cache slack slots hold NaN (or the E4M3 NaN code), so a read outside
a sequence shows up in the output."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from paged_kv_varlen_flash_amd import ops, workloads as W
from gpu_harness import compare, say

pytestmark = pytest.mark.gpu

CASES = [
    # D, G, Hkv, BS, (Lq, Lk) per sequence, window, sinks, forced splits, fp8
    (128, 4, 2, 16, ((1, 900), (1, 70), (1, 2000), (1, 5)), 512, True, 0, False),
    (64, 4, 2, 32, ((1, 300), (1, 33), (2, 90)), 16, True, 3, False),
    (128, 4, 2, 16, ((200, 200), (77, 300), (40, 40)), 100, True, 0, False),
    (64, 8, 1, 48, ((60, 60), (17, 200)), 1, False, 0, False),
    (128, 4, 2, 32, ((1, 700), (90, 400), (1, 64), (130, 130)), 300, True, 2, False),
    (128, 4, 2, 16, ((1, 900), (90, 400), (1, 64)), 200, True, 0, True),
    (256, 8, 2, 64, ((1, 3000), (1, 700)), 1000, True, 0, False),
    (128, 4, 2, 32, ((1, 700), (90, 400), (1, 64), (130, 130)), 0, True, 0, False),
    (128, 4, 2, 32, ((1, 700), (90, 400), (1, 64)), 0, True, 3, True),
    # prefill-only batches on 256-row blocks (8-wave workgroups): D = 64, and
    # prefills of 2000+ tokens at D = 128, with windows, sinks, splits, E4M3
    (64, 4, 2, 32, ((300, 300), (100, 400)), 64, True, 0, False),
    (128, 4, 2, 32, ((2100, 2100), (2050, 2300)), 700, True, 0, False),
    (128, 4, 2, 16, ((2200, 2200), (2000, 2000)), 1500, True, 2, True),
    (128, 2, 2, 64, ((2300, 2300), (2100, 2600)), 100, True, 0, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sinks_and_window(case):
    D, G, Hkv, BS, seqs, win, sinks, force, fp8 = CASES[case]
    say(f"sinks/window case={case} D={D} G={G} Hkv={Hkv} BS={BS} seqs={seqs} window={win} "
        f"sinks={sinks} force={force} fp8={fp8}")
    rng = np.random.default_rng(8000 + case)
    q_lens = np.array([a for a, _ in seqs], np.int32)
    k_lens = np.array([b for _, b in seqs], np.int32)
    B, H = len(seqs), G * Hkv
    nblk = [(int(k) + BS - 1) // BS for k in k_lens]
    NB = sum(nblk) + 3
    perm = rng.permutation(NB).astype(np.int32)
    MB = max(nblk)
    bt = np.full((B, MB), -1, np.int32)
    c = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = W.randn_bf16(rng, (T, H, D))
    s_aux = (rng.standard_normal(H) * 2).astype(np.float32) if sinks else None
    slack = np.zeros((NB, BS), bool)
    for b in range(B):
        for j in range(k_lens[b], nblk[b] * BS):
            slack[bt[b, j // BS], j % BS] = True
    if fp8:
        cache = rng.integers(0, 0x58, size=(2, NB, BS, Hkv, D), dtype=np.uint8)
        cache |= (rng.integers(0, 2, size=cache.shape, dtype=np.uint8) << 7).astype(np.uint8)
        cache[:, slack] = 0x7F
        ks, vs = W.fp8_scales(Hkv, 8100 + case)
        tc = torch.from_numpy(cache).cuda()
        kst, vst = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    else:
        cache = W.randn_bf16(rng, (2, NB, BS, Hkv, D))
        cache[:, slack] = W.SENTINEL
        ks = vs = kst = vst = None
        tc = torch.from_numpy(cache.view(np.int16)).cuda().view(torch.bfloat16)
    scale = np.float32(1.0 / np.sqrt(D))
    p = ops.make_params(B, H, Hkv, D, BS, NB, MB, True, scale, sliding_window=win, kv_cache_fp8=fp8)
    plan = ops.VarlenPlan(p, cu, k_lens, force)
    if force:
        assert plan.info.num_reduce_items > 0
    tq = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full_like(tq, float("nan"))
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ops.pa_varlen_fwd_ex(plan.params, plan.info, plan.worklist, tq, tc,
                         torch.from_numpy(cu).cuda(), torch.from_numpy(k_lens).cuda(),
                         torch.from_numpy(bt).cuda(), out, lse, plan.workspace, None,
                         kst, vst, None if s_aux is None else torch.from_numpy(s_aux).cuda())
    torch.cuda.synchronize()
    ref_out, ref_lse = OA.varlen_attention(q, cache, cu, k_lens, bt, scale, True, k_scale=ks,
                                           v_scale=vs, s_aux=s_aux, sliding_window=win)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            label=f"sinks/window case {case}")
