"""Shared steps of the GPU parity tests: run the library on a workload and
compare with the oracle.  Imported only by tests marked ``gpu``."""
import math

import numpy as np
import torch

import oracle.attention as OA
from paged_kv_varlen_flash_amd import ops, workloads as W

OUT_TOL = 1e-2     # max |out - oracle| (bf16 output)
LSE_TOL = 1e-3     # max |lse - oracle| (fp32 lse)


def say(*a):
    print(*a, flush=True)


def run_library(wl, force_splits=0, dev_tensors=None):
    """scatter + attention on the GPU; returns (out fp32 numpy, lse numpy,
    cache-after bits, plan)."""
    d = dev_tensors or W.to_device(wl)
    ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])
    plan = ops.plan_varlen(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                           tuple(d["block_table"].shape), wl.cu_seqlens_q, wl.k_lens,
                           wl.scale, wl.causal, force_splits=force_splits)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device=d["q"].device)
    ops.varlen_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["seqused_k"], d["block_table"],
                   plan, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), d, plan


def compare(out, lse, ref_out, ref_lse, rows=None, label=""):
    """Element-wise comparison to the tolerances; rows selects token rows."""
    if rows is not None:
        out, lse, ref_out, ref_lse = out[rows], lse[rows], ref_out[rows], ref_lse[rows]
    assert not np.isnan(out).any(), f"{label}: unwritten or NaN output"
    assert not np.isnan(lse).any(), f"{label}: unwritten or NaN lse"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{label}: -inf lse pattern differs"
    d_out = np.abs(out.astype(np.float64) - ref_out)
    d_lse = np.abs(np.where(empty, 0.0, lse.astype(np.float64) - np.where(empty, 0.0, ref_lse)))
    mo, ml = float(d_out.max(initial=0)), float(d_lse.max(initial=0))
    say(f"  [{label}] max|out-ref|={mo:.3e} max|lse-ref|={ml:.3e} "
        f"max|ref out|={float(np.abs(ref_out).max(initial=0)):.3f} rows={out.shape[0]}")
    assert mo <= OUT_TOL, f"{label}: out error {mo}"
    assert ml <= LSE_TOL, f"{label}: lse error {ml}"
    return mo, ml


def sub_problem(wl, seqs):
    """Rows of the sampled sequences and their (cu, seqused, block table)."""
    rows = np.concatenate([np.arange(wl.cu_seqlens_q[b], wl.cu_seqlens_q[b + 1]) for b in seqs])
    lq = wl.q_lens[seqs]
    cu = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    return rows, cu, wl.k_lens[seqs], wl.block_table[seqs]
