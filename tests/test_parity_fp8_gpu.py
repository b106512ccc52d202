"""GPU parity of the E4M3 (FP8) KV-cache path through the C ABI against the
fp64 oracle (oracle.fp8 + oracle.attention with per-KV-head scales).

The cache write is compared byte for byte (including ties, subnormals,
saturation and NaN); attention within the same tolerances as the bf16 path
(out 1e-2 max-abs, lse 1e-3), since the kernels widen E4M3 to bf16 exactly and
apply the scales in fp32.  Cache slots outside every sequence's keys hold
the NaN code, so a read past a sequence shows up in the output."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import oracle.fp8 as OF8
from paged_kv_varlen_flash_amd import ops, workloads as W
from gpu_harness import compare, say

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _run_fp8(wl, seed, force_splits=0):
    """GPU: cache write + attention; oracle: the same two steps."""
    codes = W.fp8_cache_codes(wl, seed)
    ks, vs = W.fp8_scales(wl.Hkv, seed + 1)
    d = W.to_device(wl)
    cache = _u8(codes)
    kst, vst = _f32(ks), _f32(vs)
    ops.pa_reshape_and_cache_fp8(d["key"], d["value"], cache, d["slot_mapping"], kst, vst)
    plan = ops.plan_varlen(tuple(d["q"].shape), tuple(cache.shape), tuple(d["block_table"].shape),
                           wl.cu_seqlens_q, wl.k_lens, wl.scale, wl.causal, force_splits=force_splits,
                           kv_cache_fp8=True)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ops.varlen_fwd(d["q"], cache, d["cu_seqlens_q"], d["seqused_k"], d["block_table"], plan,
                   out=out, lse=lse, k_scale=kst, v_scale=vst)
    torch.cuda.synchronize()
    ref_cache = OF8.reshape_and_cache_fp8(wl.key, wl.value, codes, wl.slot_mapping, ks, vs)
    return out.float().cpu().numpy(), lse.cpu().numpy(), cache.cpu().numpy(), ref_cache, ks, vs, plan


@pytest.mark.parametrize("name", ["tiny_mixed", "decode_llama8b", "chunked_prefill_mix"])
def test_fp8_workload(name):
    say(f"fp8 cache: write + attention {name}")
    wl = W.make(name)
    out, lse, cache, ref_cache, ks, vs, plan = _run_fp8(wl, 2000 + len(name))
    assert np.array_equal(cache, ref_cache), "E4M3 cache write differs from the oracle"
    ref_out, ref_lse = OA.varlen_attention(wl.q, ref_cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, wl.causal,
                                           k_scale=ks, v_scale=vs)
    compare(out, lse, ref_out, ref_lse, label=f"fp8 {name}")


@pytest.mark.parametrize("splits", [2, 5])
def test_fp8_forced_splits(splits):
    say(f"fp8 forced splits {splits}")
    wl = W.make("tiny_mixed")
    out, lse, cache, ref_cache, ks, vs, plan = _run_fp8(wl, 2100 + splits, force_splits=splits)
    assert plan.info.num_reduce_items > 0
    assert np.array_equal(cache, ref_cache)
    ref_out, ref_lse = OA.varlen_attention(wl.q, ref_cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True, k_scale=ks, v_scale=vs)
    compare(out, lse, ref_out, ref_lse, label=f"fp8 splits={splits}")


# decode-only and prefill-only batches at every head size (small-row and
# tiled kernels on their own)
FP8_SHAPES = [
    # D, G, Hkv, BS, causal, (Lq, Lk) per sequence, forced splits
    (64, 4, 2, 16, True, ((1, 300), (1, 17), (2, 90), (1, 1)), 0),
    (128, 8, 1, 32, True, ((1, 700), (1, 33), (1, 2048)), 3),
    (256, 8, 2, 64, True, ((1, 1500), (1, 64), (1, 777)), 0),
    (64, 8, 1, 48, True, ((40, 40), (17, 300), (250, 260)), 0),
    (128, 4, 2, 16, False, ((64, 64), (33, 97), (200, 450)), 2),
    (256, 4, 1, 32, True, ((70, 70), (33, 180)), 0),
    (128, 4, 2, 32, True, ((2100, 2100), (2050, 2200)), 0),   # 256-row tiled blocks
]


@pytest.mark.parametrize("case", range(len(FP8_SHAPES)))
def test_fp8_shapes(case):
    D, G, Hkv, BS, causal, seqs, force = FP8_SHAPES[case]
    spec = W.Spec(name=f"fp8_shape{case}", num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                  block_size=BS, causal=causal, seed=7100 + case, fixed=seqs, min_num_blocks=3)
    say(f"fp8 shape case={case} D={D} G={G} Hkv={Hkv} BS={BS} causal={causal} seqs={seqs} "
        f"force={force}")
    wl = W.make(spec)
    out, lse, cache, ref_cache, ks, vs, plan = _run_fp8(wl, 2200 + case, force_splits=force)
    assert np.array_equal(cache, ref_cache)
    ref_out, ref_lse = OA.varlen_attention(wl.q, ref_cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, causal, k_scale=ks, v_scale=vs)
    compare(out, lse, ref_out, ref_lse, label=f"fp8 shape{case}")


def test_fp8_cache_write_edge_values():
    """Ties to even, subnormals, saturation, NaN and infinities, at scale 1
    and at a non-power-of-two scale."""
    say("fp8 cache write: edge values")
    grid = OF8.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)           # exact in bf16
    special = np.array([448, 450, 464, 500, 10240, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12,
                        np.inf, -np.inf, np.nan, 0.0, -0.0], np.float32)
    vals = np.concatenate([mids, -mids, grid.astype(np.float32), special])
    bits = W.f32_to_bf16_bits(vals)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32)[~np.isnan(vals)],
                          vals[~np.isnan(vals)])
    Hkv, D = 1, 16
    n = (len(bits) + D - 1) // D
    pad = np.zeros(n * D, np.uint16)
    pad[:len(bits)] = bits
    key = pad.reshape(n, Hkv, D)
    value = key[::-1].copy()
    NB, BS = (n + 15) // 16, 16
    slots = np.arange(n, dtype=np.int64)
    for ks_val in (1.0, 0.37):
        ks = np.array([ks_val], np.float32)
        vs = np.array([ks_val * 2], np.float32)
        before = np.full((2, NB, BS, Hkv, D), 0x55, np.uint8)
        cache = _u8(before)
        dk = torch.from_numpy(key.view(np.int16)).cuda().view(torch.bfloat16)
        dv = torch.from_numpy(value.view(np.int16)).cuda().view(torch.bfloat16)
        ops.pa_reshape_and_cache_fp8(dk, dv, cache, torch.from_numpy(slots).cuda(), _f32(ks), _f32(vs))
        torch.cuda.synchronize()
        ref = OF8.reshape_and_cache_fp8(key, value, before, slots, ks, vs)
        got = cache.cpu().numpy()
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"scale {ks_val}: {len(bad)} bytes differ, first {bad[:4].tolist()}"
