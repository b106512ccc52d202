"""pa_varlen_fwd_noalloc (the entry point for callers that cannot allocate:
its split-KV partials live in the library's own device scratch) against
pa_varlen_fwd_ex on the same plan and inputs: outputs bit for bit, on calls
in a row whose plans shrink, so that the second reuses a scratch that still
holds the first call's partials."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from paged_kv_varlen_flash_amd import ops, workloads as W
from gpu_harness import compare, say

pytestmark = pytest.mark.gpu


def _call(name, force, fp8=False, sinks=False):
    wl = W.make(name)
    d = W.to_device(wl)
    kw = {}
    if fp8:
        d["kv_cache"] = torch.from_numpy(W.fp8_cache_codes(wl, 4000)).cuda()
        ks, vs = W.fp8_scales(wl.Hkv, 4001)
        kw = dict(k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda())
        ops.pa_reshape_and_cache_fp8(d["key"], d["value"], d["kv_cache"], d["slot_mapping"],
                                     kw["k_scale"], kw["v_scale"])
    else:
        ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    if sinks:
        kw["s_aux"] = torch.from_numpy(np.linspace(-2, 2, wl.H).astype(np.float32)).cuda()
    plan = ops.plan_varlen(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                           tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens, wl.scale,
                           wl.causal, force_splits=force, kv_cache_fp8=fp8)
    assert 0 < plan.info.workspace_bytes <= ops.NOALLOC_SCRATCH_BYTES
    say(f"noalloc {name} force={force} fp8={fp8} sinks={sinks}: "
        f"partials {plan.info.workspace_bytes} bytes")
    args = (d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"], d["block_table"])
    ref_out = torch.full_like(d["q"], float("nan"))
    ref_lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ops.pa_varlen_fwd_ex(plan.params, plan.info, plan.worklist, *args, ref_out, ref_lse,
                         plan.workspace, None, **kw)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ops.pa_varlen_fwd_noalloc(plan.params, plan.info, plan.worklist, *args, out, lse, None, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"{name}: out differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), f"{name}: lse differs"
    return wl, d, out, lse


def test_noalloc_matches_workspace_entry_point():
    # largest plan first, then smaller ones: each call reuses the scratch
    wl, d, out, lse = _call("decode_llama8b", 0)
    cache = OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping)
    ref_out, ref_lse = OA.varlen_attention(wl.q, cache, wl.cu_seqlens_q, wl.k_lens,
                                           wl.block_table, wl.scale, True)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            label="noalloc decode_llama8b")
    _call("tiny_mixed", 3)
    _call("tiny_mixed", 2, fp8=True, sinks=True)
