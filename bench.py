"""Benchmark of the paged varlen attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--secondary]
                    [--kv-dtype bf16|fp8]

A step is one pass of the whole path over one batch that is already resident
in HBM: the host planner (pa_plan_varlen, whose work list is copied to the
device from pinned memory), pa_reshape_and_cache for the batch's new tokens,
and pa_varlen_fwd (attention kernels + split-KV reduce); the cascade workload
adds its two passes and pa_merge_attn_states.  The headline workload is the
64-sequence Llama-3-8B-shaped decode batch.  With --kv-dtype fp8 the cache
holds E4M3 codes (one byte per element, per-KV-head scales): the cache write
is pa_reshape_and_cache_fp8, attention pa_varlen_fwd_fp8, and the
algorithmic KV bytes are one per element.

Printed: one JSON line with the whole-step throughput (algorithmic KV bytes
per second), a roofline object for the attention call -- its algorithmic
bytes (or flops) divided by its average duration, measured with HIP events
on the launch stream over separate timed launches with the caches flushed
in between -- and the fp64 oracle timed on the host cores on a bounded
sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
CALIB_BYTES = 256 << 20        # size of the counter-calibration copy
BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PLAN_RING = 8                  # pinned work-list buffers in flight


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_llama8b")
    ap.add_argument("--kernel-reps", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="budget for each oracle CPU baseline")
    ap.add_argument("--prefill-workload", default="chunked_prefill_mix_prefill",
                    help="causal-prefill workload of the line's prefill object")
    ap.add_argument("--mixed-workload", default="chunked_prefill_mix",
                    help="decode+prefill workload of the line's mixed object")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the --workload only (no prefill or mixed object)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", action="store_true",
                    help="also time the prefill mix and the long-context decode")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="KV-cache format: bf16, or E4M3 codes with per-KV-head scales")
    return ap.parse_args()


class Step:
    """Everything one step needs, resident on the GPU."""

    def __init__(self, wl, dev, fp8=False, single_pass=False, window=0, sinks=False):
        import torch
        from paged_kv_varlen_flash_amd import ops, workloads as W
        self.ops, self.wl, self.fp8 = ops, wl, fp8
        self.d = W.to_device(wl, dev)
        d = self.d
        if fp8:
            if wl.spec.shared_prefix:
                raise SystemExit("--kv-dtype fp8 covers the single-pass workloads")
            self.codes = W.fp8_cache_codes(wl, 4000)
            self.k_scale, self.v_scale = W.fp8_scales(wl.Hkv, 4001)
            d["kv_cache"] = torch.from_numpy(self.codes).to(dev)
            d["k_scale"] = torch.from_numpy(self.k_scale).to(dev)
            d["v_scale"] = torch.from_numpy(self.v_scale).to(dev)
        self.params = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks,
                                      wl.block_table.shape[1], wl.causal, wl.scale,
                                      sliding_window=window, kv_cache_fp8=fp8,
                                      num_cus=ops.device_cus(dev))
        self.s_aux = None
        if sinks:
            rng = np.random.default_rng(4002)
            self.s_aux = torch.from_numpy((rng.standard_normal(wl.H) * 2).astype(np.float32)).to(dev)
        self.cu = np.ascontiguousarray(wl.cu_seqlens_q, np.int32)
        self.sk = np.ascontiguousarray(wl.k_lens, np.int32)
        words, info = ops.pa_plan_varlen(self.params, self.cu, self.sk)
        self.cap = words.nbytes
        # a ring of pinned host buffers: the plan of step t is written while the
        # copies of earlier steps may still be queued; the host blocks only when
        # it is PLAN_RING steps ahead of the GPU, so a late wake-up of the host
        # thread does not drain the GPU queue
        self.pinned = [torch.empty(words.size, dtype=torch.int32).pin_memory()
                       for _ in range(PLAN_RING)]
        self.copy_done = [None] * PLAN_RING
        self.worklist = torch.from_numpy(words).to(dev)
        self.info = info
        self.workspace = torch.empty(max(info.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(d["q"])
        self.lse = torch.empty(wl.T, wl.H, dtype=torch.float32, device=dev)
        self.i = 0
        self.cascade = None
        if wl.spec.shared_prefix and not single_pass:
            self.cascade = ops.CascadePlan(tuple(d["q"].shape), tuple(d["kv_cache"].shape),
                                           tuple(d["block_table"].shape), wl.cu_seqlens_q,
                                           wl.k_lens, wl.scale, wl.spec.shared_prefix)
            self.parts = [torch.empty_like(self.out), torch.empty_like(self.lse),
                          torch.empty_like(self.out), torch.empty_like(self.lse)]

    def plan(self):
        import torch
        ops = self.ops
        k = self.i % PLAN_RING
        self.i += 1
        if self.copy_done[k] is not None:
            self.copy_done[k].synchronize()
        buf = self.pinned[k]
        info = ops.PlanInfo()
        st = ops.lib().pa_plan_varlen(ctypes.byref(self.params),
                                      self.cu.ctypes.data_as(ops._I32P),
                                      self.sk.ctypes.data_as(ops._I32P), 0,
                                      ctypes.cast(buf.data_ptr(), ops._I32P), self.cap,
                                      ctypes.byref(info))
        if st != 0:
            raise ops.PaError(st, "pa_plan_varlen")
        # the upload is a kernel of the compute stream (a copy-engine transfer
        # would make the next kernel wait for the engine's completion signal)
        ops.pa_upload_words(buf, self.worklist)
        ev = torch.cuda.Event()
        ev.record()
        self.copy_done[k] = ev
        self.info = info

    def scatter(self):
        d = self.d
        if self.fp8:
            self.ops.pa_reshape_and_cache_fp8(d["key"], d["value"], d["kv_cache"],
                                              d["slot_mapping"], d["k_scale"], d["v_scale"])
        else:
            self.ops.pa_reshape_and_cache(d["key"], d["value"], d["kv_cache"], d["slot_mapping"])

    def attention(self):
        d, ops = self.d, self.ops
        if self.s_aux is not None:
            ops.pa_varlen_fwd_ex(self.params, self.info, self.worklist, d["q"], d["kv_cache"],
                                 d["cu_seqlens_q"], d["seqused_k"], d["block_table"], self.out,
                                 self.lse, self.workspace, None,
                                 d.get("k_scale") if self.fp8 else None,
                                 d.get("v_scale") if self.fp8 else None, self.s_aux)
        elif self.fp8:
            ops.pa_varlen_fwd_fp8(self.params, self.info, self.worklist, d["q"], d["kv_cache"],
                                  d["cu_seqlens_q"], d["seqused_k"], d["block_table"],
                                  d["k_scale"], d["v_scale"], self.out, self.lse, self.workspace)
        elif self.cascade is None:
            ops.pa_varlen_fwd(self.params, self.info, self.worklist, d["q"], d["kv_cache"],
                              d["cu_seqlens_q"], d["seqused_k"], d["block_table"], self.out,
                              self.lse, self.workspace)
        else:
            ops.cascade_fwd(d["q"], d["kv_cache"], d["cu_seqlens_q"], d["block_table"],
                            self.cascade, out=self.out, lse=self.lse,
                            prefix_out=self.parts[0], prefix_lse=self.parts[1],
                            suffix_out=self.parts[2], suffix_lse=self.parts[3])

    def __call__(self):
        if self.cascade is None:
            self.plan()
        self.scatter()
        self.attention()


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_attention(step, reps, flush):
    """Average duration of the attention call, HIP events on its stream, with
    a cache-flushing write between launches (outside the timed interval)."""
    import torch
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.fill_(1)
        # a short spin keeps the GPU busy while the host enqueues the call, so
        # the interval below holds device time only
        torch.cuda._sleep(400000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        step.attention()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    times = np.array(times)
    return float(times.mean()), float(np.median(times))


def source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ("pagedattn.hip", "plan.cpp", "plan_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_varlen_flash_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the attention call from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE passes (profiles/traffic.json), or None
    when the kernel sources changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_sha256():
        return None
    return rec


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def _cores():
    """Threads the oracle uses (its products run in BLAS) and the host cores
    this process may run on."""
    return {"cores": blas_threads(), "affinity_cores": len(os.sched_getaffinity(0))}


def _oracle_cache(wl, fp8_step):
    import oracle.attention as OA
    if fp8_step is None:
        return OA.reshape_and_cache(wl.key, wl.value, wl.kv_cache, wl.slot_mapping), {}, 2
    import oracle.fp8 as OF8
    ks, vs = fp8_step.k_scale, fp8_step.v_scale
    cache = OF8.reshape_and_cache_fp8(wl.key, wl.value, fp8_step.codes, wl.slot_mapping, ks, vs)
    return cache, {"k_scale": ks, "v_scale": vs}, 1


def cpu_baseline(wl, budget_s, fp8_step=None, unit="GB/s"):
    """The fp64 oracle (as it stands) on whole sequences of the same batch,
    cycling through them until the time budget is used.  unit "GB/s": KV
    bytes read per second; "TFLOP/s": the algorithmic flops (4·D·H per
    visible (query, key) pair) of the sequences done per second."""
    import oracle.attention as OA
    cache, scales, es = _oracle_cache(wl, fp8_step)
    pairs = wl.causal_pairs()
    done, nbytes, flops = 0, 0, 0
    t0 = time.perf_counter()
    # whole sequences, cycling through the batch, until the budget is spent
    while time.perf_counter() - t0 < budget_s:
        b = done % wl.B
        t_a, t_b = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        OA.varlen_attention(wl.q[t_a:t_b], cache, np.array([0, t_b - t_a]), wl.k_lens[b:b + 1],
                            wl.block_table[b:b + 1], wl.scale, wl.causal, **scales)
        nbytes += 2 * int(wl.k_lens[b]) * wl.Hkv * wl.D * es
        flops += 4 * wl.D * wl.H * int(pairs[b])
        done += 1
    el = time.perf_counter() - t0
    val = nbytes / el / 1e9 if unit == "GB/s" else flops / el / 1e12
    return dict({"value": round(val, 6 if unit != "GB/s" else 4), "unit": unit, "kind": "oracle",
                 "sample": f"{done} whole-sequence passes over the {wl.B} sequences of "
                           f"{wl.spec.name} ({nbytes/1e6:.1f} MB of KV, {flops/1e9:.2f} GFLOP), "
                           f"fp64 numpy, {el:.1f} s wall"}, **_cores())


_WORKLOADS = {}


def measure(name, args, dev, flush, cpu_unit=None, fp8=False, single_pass=False, window=0,
            sinks=False):
    import torch
    from paged_kv_varlen_flash_amd import workloads as W
    if name not in _WORKLOADS:
        print(f"bench: building workload {name}", file=sys.stderr, flush=True)
        _WORKLOADS[name] = W.make(name)
    wl = _WORKLOADS[name]
    step = Step(wl, dev, fp8, single_pass, window, sinks)
    print(f"bench: timing {name}{' (E4M3 cache)' if fp8 else ''}", file=sys.stderr, flush=True)
    per_step = time_steps(step, args.steps, args.warmup)
    t_mean, t_med = time_attention(step, args.kernel_reps, flush)
    kv = wl.kv_read_bytes() // (2 if fp8 else 1)
    single_pass_kv = None
    if step.cascade is not None:
        # the cascade reads the shared prefix once (prefix pass) and each
        # sequence's own suffix (suffix pass): those are its algorithmic bytes;
        # the single-pass bytes (every sequence reading the prefix) are context
        P = wl.spec.shared_prefix
        single_pass_kv = kv
        kv = int(2 * (P + (wl.k_lens.astype(np.int64) - P).sum()) * wl.Hkv * wl.D * 2)
    if window:
        # keys inside the window only (decode rows: the last W keys)
        kv = int(2 * np.minimum(wl.k_lens.astype(np.int64), window).sum() * wl.Hkv * wl.D
                 * (1 if fp8 else 2))
    flops = wl.attention_flops()
    res = {"workload": name, "wl": wl, "ms_per_step": per_step * 1e3, "attn_mean_s": t_mean,
           "attn_median_s": t_med, "kv_bytes": kv, "flops": flops, "plan": step.info.as_dict(),
           "single_pass_kv_bytes": single_pass_kv,
           "cascade_plans": None if step.cascade is None else
           (step.cascade.prefix.info.as_dict(), step.cascade.suffix.info.as_dict())}
    if cpu_unit:
        print(f"bench: oracle CPU baseline on {name}", file=sys.stderr, flush=True)
        res["cpu"] = cpu_baseline(wl, args.cpu_seconds, step if fp8 else None, cpu_unit)
    del step
    torch.cuda.empty_cache()
    return res


def kernel_names(res, fp8):
    """The kernels of one attention call, from its plan (a cascade: both
    passes' kernels and the merge)."""
    if res.get("cascade_plans"):
        pre, suf = res["cascade_plans"]
        return ("prefix pass: " + kernel_names(dict(res, plan=pre, cascade_plans=None), fp8) +
                "; suffix pass: " + kernel_names(dict(res, plan=suf, cascade_plans=None), fp8) +
                "; merge_states_kernel")
    p, D, BS = res["plan"], res["wl"].D, res["wl"].BS
    tag = f"<{D}{', fp8' if fp8 else ''}>"
    dma = D == 128 and not fp8 and BS & (BS - 1) == 0    # tiles loaded into LDS by DMA
    if p["num_small_items"] and p["num_tiled_items"]:
        k = ["attn_mixed_dma_kernel<128>" if dma else "attn_mixed_kernel" + tag]
    elif p["num_small_items"]:
        k = ["attn_small_kernel" + tag]
    elif p["tiled_rows"] == 256:
        k = ["attn_tiled_wide_kernel" + tag]
    else:
        k = ["attn_tiled_dma4_kernel<128>" if dma else "attn_tiled_kernel" + tag]
    if p["num_reduce_items"]:
        k.append(f"split_reduce_kernel<{D}>")
    return " + ".join(k)


def hbm_roofline(res, fp8, traffic_key):
    ach = res["kv_bytes"] / res["attn_mean_s"] / 1e9
    tr = recorded_traffic(traffic_key)
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": (tr["read_bytes"] + tr["write_bytes"]) if tr else None,
            "traffic_read_over_algorithmic": (round(tr["read_bytes"] / res["kv_bytes"], 4)
                                              if tr else None),
            "kernel": "pa_varlen_fwd%s: %s" % ("_fp8" if fp8 else "", kernel_names(res, fp8)),
            "per_launch_bytes": res["kv_bytes"],
            "avg_launch_us": round(res["attn_mean_s"] * 1e6, 2),
            "median_launch_us": round(res["attn_median_s"] * 1e6, 2),
            **({"single_pass_bytes": res["single_pass_kv_bytes"],
                "single_pass_equivalent_GBps": round(res["single_pass_kv_bytes"] /
                                                     res["attn_mean_s"] / 1e9, 1)}
               if res.get("single_pass_kv_bytes") else {})}


def mfma_roofline(res, fp8, traffic_key):
    ach = res["flops"] / res["attn_mean_s"] / 1e12
    tr = recorded_traffic(traffic_key)
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
            "traffic": (tr["read_bytes"] + tr["write_bytes"]) if tr else None,
            "kernel": "pa_varlen_fwd%s: %s" % ("_fp8" if fp8 else "", kernel_names(res, fp8)),
            "per_launch_flops": res["flops"],
            "avg_launch_us": round(res["attn_mean_s"] * 1e6, 2),
            "median_launch_us": round(res["attn_median_s"] * 1e6, 2)}


def is_decode_like(wl, name):
    return wl.q_lens.max() * (wl.H // wl.Hkv) <= 16 or name == "cascade_prefix"


def entry(res, fp8, tkey):
    """Step throughput, roofline and CPU baseline of one measured workload."""
    wl = res["wl"]
    if is_decode_like(wl, res["workload"]):
        value, unit = res["kv_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9, "GB/s"
        roof = hbm_roofline(res, fp8, tkey)
    else:
        value, unit = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
        roof = mfma_roofline(res, fp8, tkey)
    e = {"workload": res["workload"], "value": round(value, 1), "unit": unit,
         "ms_per_step": round(res["ms_per_step"], 4), "config": wl.summary(), "roofline": roof}
    if "cpu" in res:
        e["cpu_baseline"] = res["cpu"]
    return e


def mixed_entry(res, fp8, tkey):
    """A launch of both kinds: its flops and its KV bytes against both peaks,
    and max(bytes / HBM peak, flops / MFMA peak) / time, the fraction of the
    time the busier of the two resources needs at peak."""
    t = res["attn_mean_s"]
    tf, gb = res["flops"] / t / 1e12, res["kv_bytes"] / t / 1e9
    tr = recorded_traffic(tkey)
    e = {"workload": res["workload"], "ms_per_step": round(res["ms_per_step"], 4),
         "config": res["wl"].summary(),
         "roofline": {"bound": "mfma+hbm", "attn_TFLOPs": round(tf, 1),
                      "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4), "kv_GBps": round(gb, 1),
                      "hbm_frac": round(gb / HBM_PEAK_GBS, 4),
                      "frac": round(max(res["kv_bytes"] / (HBM_PEAK_GBS * 1e9),
                                        res["flops"] / (BF16_PEAK_TFLOPS * 1e12)) / t, 4),
                      "traffic": (tr["read_bytes"] + tr["write_bytes"]) if tr else None,
                      "traffic_read_over_algorithmic": (round(tr["read_bytes"] / res["kv_bytes"], 4)
                                                        if tr else None),
                      # the same with the queries (read once) counted as algorithmic
                      "traffic_read_over_kv_and_q": (
                          round(tr["read_bytes"] / (res["kv_bytes"] + tr["q_bytes"]), 4)
                          if tr and "q_bytes" in tr else None),
                      "kernel": "pa_varlen_fwd%s: %s" % ("_fp8" if fp8 else "",
                                                         kernel_names(res, fp8)),
                      "per_launch_flops": res["flops"], "per_launch_bytes": res["kv_bytes"],
                      "avg_launch_us": round(t * 1e6, 2)}}
    if "cpu" in res:
        e["cpu_baseline"] = res["cpu"]
    return e


METRIC = "decode KV-read GB/s + prefill TFLOP/s, as % of MI355X roofline"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_kv_varlen_flash_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        raise SystemExit("libpagedattn.so is not built: python -m paged_kv_varlen_flash_amd.build")
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    # one plain 256 MiB device copy (untimed): under rocprofv3 --pmc its
    # FETCH_SIZE / WRITE_SIZE calibrate the counters against known bytes
    calib_src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    fp8 = args.kv_dtype == "fp8"
    sfx = "_fp8" if fp8 else ""
    cpu = not args.no_cpu_baseline
    W = __import__("paged_kv_varlen_flash_amd.workloads", fromlist=["SPECS"])
    spec = W.SPECS[args.workload]
    head_unit = "GB/s" if (args.workload == "cascade_prefix" or all(
        g[0] == "decode" for g in spec.groups)) and spec.fixed is None else "TFLOP/s"
    head = measure(args.workload, args, dev, flush, head_unit if cpu else None, fp8)
    he = entry(head, fp8, args.workload + sfx)
    line = {
        "metric": METRIC,
        "value": he["value"], "unit": he["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": he["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 KV cache, bf16 MFMA, fp32 softmax" if fp8 else "bf16",
        "data": ("synthetic (seeded random E4M3 cache codes, |code value| <= 15, per-KV-head "
                 "scales in [0.02, 0.1]; new tokens N(0,1) bf16 quantised by the cache write; "
                 "shuffled physical blocks)" if fp8 else
                 "synthetic (seeded N(0,1) bf16, shuffled physical blocks)"),
        "config": dict(he["config"], parallelism="none (1 GPU)",
                       kv_cache_dtype="fp8_e4m3 (per-KV-head scales)" if fp8 else "bf16"),
        "roofline": he["roofline"],
    }
    if "cpu_baseline" in he:
        line["cpu_baseline"] = he["cpu_baseline"]
    if not args.headline_only:
        # the other half of the metric: causal prefill rows (the chunked-prefill
        # mix's 8 prefills alone), and the mix as one launch of both kinds
        if args.prefill_workload and args.prefill_workload != args.workload:
            r = measure(args.prefill_workload, args, dev, flush, "TFLOP/s" if cpu else None, fp8)
            line["prefill"] = entry(r, fp8, args.prefill_workload + sfx)
        if args.mixed_workload and args.mixed_workload != args.workload:
            r = measure(args.mixed_workload, args, dev, flush, "TFLOP/s" if cpu else None, fp8)
            line["mixed"] = mixed_entry(r, fp8, args.mixed_workload + sfx)
    if args.secondary:
        sec = {}
        for name in ("chunked_prefill_mix", "chunked_prefill_mix_prefill", "prefill_causal_8k",
                     "long_decode_d256", "cascade_prefix"):
            r = measure(name, args, dev, flush)
            w = r["wl"]
            ent = {"ms_per_step": round(r["ms_per_step"], 4),
                   "attn_avg_us": round(r["attn_mean_s"] * 1e6, 2),
                   "kernel": kernel_names(r, False),
                   "kv_GBps": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9, 1),
                   "hbm_frac": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9 / HBM_PEAK_GBS, 4)}
            if name == "cascade_prefix":
                # the host decision against both measured paths
                P, use = ops.pa_cascade_decide(
                    ops.make_params(w.B, w.H, w.Hkv, w.D, w.BS, w.num_blocks,
                                    w.block_table.shape[1], w.causal, w.scale),
                    w.cu_seqlens_q, w.k_lens, w.block_table)
                one = measure(name, args, dev, flush, single_pass=True)
                ent["single_pass_attn_avg_us"] = round(one["attn_mean_s"] * 1e6, 2)
                ent["cascade_decision"] = {"common_prefix_len": P, "use_cascade": use}
            if name.startswith("chunked_prefill_mix") or name.startswith("prefill_"):
                ent["attn_TFLOPs"] = round(r["flops"] / r["attn_mean_s"] / 1e12, 1)
                ent["mfma_frac"] = round(r["flops"] / r["attn_mean_s"] / 1e12 / BF16_PEAK_TFLOPS, 4)
            sec[name] = ent
        if not fp8:
            # the decision on a longer shared prefix (64 requests x 16384 shared
            # tokens): both paths measured next to it
            w = W.make("cascade_prefix_16k", materialise=False)
            P, use = ops.pa_cascade_decide(
                ops.make_params(w.B, w.H, w.Hkv, w.D, w.BS, w.num_blocks, w.block_table.shape[1],
                                w.causal, w.scale), w.cu_seqlens_q, w.k_lens, w.block_table)
            casc = measure("cascade_prefix_16k", args, dev, flush)
            one = measure("cascade_prefix_16k", args, dev, flush, single_pass=True)
            sec["cascade_prefix_16k"] = {"attn_avg_us": round(casc["attn_mean_s"] * 1e6, 2),
                                         "single_pass_attn_avg_us": round(one["attn_mean_s"] * 1e6, 2),
                                         "cascade_decision": {"common_prefix_len": P,
                                                              "use_cascade": use}}
        if not fp8:
            # decode with a 1024-key sliding window and per-head sinks
            r = measure("decode_llama8b", args, dev, flush, window=1024, sinks=True)
            sec["decode_llama8b_window1024_sinks"] = {
                "attn_avg_us": round(r["attn_mean_s"] * 1e6, 2),
                "kv_GBps": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9, 1),
                "hbm_frac": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9 / HBM_PEAK_GBS, 4)}
        if not fp8:
            r = measure("decode_llama8b", args, dev, flush, fp8=True)
            sec["decode_llama8b_fp8"] = {
                "ms_per_step": round(r["ms_per_step"], 4),
                "attn_avg_us": round(r["attn_mean_s"] * 1e6, 2),
                "kv_GBps": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9, 1),
                "hbm_frac": round(r["kv_bytes"] / r["attn_mean_s"] / 1e9 / HBM_PEAK_GBS, 4)}
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
