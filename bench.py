#!/usr/bin/env python3
"""Benchmark of the paged MLA decode hot path on one MI355X.

A step is one pass of the whole path over one batch: the split-KV plan
(mla_get_metadata), then mla_decode_with_kvcache, i.e. the split decode
kernel and the kernel that merges the partial results of split sequences
(launched as its two phases so that each kernel is timed on its own).  The default workload is the memory-bound decode:
b=64, s_q=1, h_q=16, h_kv=1, d_qk=576, dv=512, lengths uniform in [1, 4096]
(seeded), 64-token pages, shuffled block table over a 6000-page pool, bf16
N(0, 1) data.

Inputs are resident in HBM before timing starts.  Four copies of the cache
(each 442 MB) are used in rotation, so the 256 MB Infinity Cache cannot serve
a step from the previous one; the step reads its keys from HBM as a decode
over a fresh layer would.  A GPU sleep queued ahead of the timed steps lets
the host enqueue them all before the GPU reaches them, so the K steps run
back to back and the HIP events measure GPU time, not Python launch time.
Events sit only at the two ends of the timed region: an event between two
launches costs several microseconds of GPU time.  The duration of each
launch (plan, split decode, combine) comes from a second pass that enqueues
K launches of that kernel alone, back to back, between two events.

The default run also times the compute-bound workloads (near-ridge b=128
h_q=128 L=4096; MTP causal b=32 s_q=2 h_q=128; sparse top-k b=16 s_q=8 h_q=128
k=2048) and reports their bf16 TFLOPS and MFMA fraction under
`compute_bound`; --secondary adds the other workloads.

`traffic` is the HBM traffic of one decode launch measured with rocprofv3
counters (FETCH_SIZE and WRITE_SIZE, each calibrated against a plain device
copy of known size, see --calibrate-copy) and stored in
profiles/decode_<workload>_traffic.json together with the SHA-256 of the
decode kernels' sources it was taken on (mla_common.h, mla_decode_kernel.h,
mla_decode.hip, mla_decode_rows128.hip); it is reported only while those
sources are unchanged, else null.

Prints one JSON line (the last line of stdout).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
NCOPIES = 4


def algorithmic_work(w):
    """KV bytes (each key row of each latent head once, at its stored size: 1152
    bytes bf16, 656 packed FP8) and FLOPs (2 * (576 + 512) per query row and key)."""
    L = w.cache_seqlens.astype(np.int64)
    h_kv = w.kv.shape[2]
    KV_ROW_BYTES = w.kv.shape[3] * w.kv.itemsize
    d_qk = w.q.shape[3]
    if w.indices is not None:
        ok = (w.indices >= 0) & (w.indices < L[:, None, None])
        keys = int(ok.sum())
        if w.aux is not None:      # dual cache: the auxiliary keys join each token's key set
            idx2, L2 = w.aux[3], w.aux[2].astype(np.int64)
            keys += int(((idx2 >= 0) & (idx2 < L2[:, None, None])).sum())
        return keys * h_kv * KV_ROW_BYTES, keys * w.h_q * 2 * (d_qk + 512)
    kv = int(L.sum()) * h_kv * KV_ROW_BYTES
    if w.causal:
        qk = sum(w.h_q * max(int(l) - w.s_q + s + 1, 0) for l in L for s in range(w.s_q))
    else:
        qk = int(L.sum()) * w.s_q * w.h_q
    return kv, qk * 2 * (d_qk + 512)


def gpu_sleep_ms(torch, ms):
    """Queue a GPU spin of about `ms` milliseconds on the current stream."""
    if not hasattr(gpu_sleep_ms, "cycles_per_ms"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        gpu_sleep_ms.cycles_per_ms = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(gpu_sleep_ms.cycles_per_ms * ms))


def _to_dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda() if dtype is None else t.cuda().view(dtype)


def run_workload(torch, m, w, steps, warmup, ncopies=NCOPIES):
    q0 = _to_dev(torch, w.q.view(np.int16), torch.bfloat16)
    kv0 = _to_dev(torch, w.kv) if w.kv.dtype == np.uint8 else _to_dev(torch, w.kv.view(np.int16), torch.bfloat16)
    bt = _to_dev(torch, w.block_table.astype(np.int32))
    sl = _to_dev(torch, w.cache_seqlens.astype(np.int32))
    idx = _to_dev(torch, w.indices.astype(np.int32)) if w.indices is not None else None
    qs = [q0] + [q0.clone() for _ in range(ncopies - 1)]
    kvs = [kv0] + [kv0.clone() for _ in range(ncopies - 1)]
    h_kv = w.kv.shape[2]
    rows = w.s_q * w.h_q // h_kv
    aux = None
    topk2 = 0
    if w.aux is not None:
        kv2, bt2, sl2, idx2 = w.aux
        aux = (_to_dev(torch, kv2.view(np.int16), torch.bfloat16), _to_dev(torch, bt2.astype(np.int32)),
               _to_dev(torch, sl2.astype(np.int32)), _to_dev(torch, idx2.astype(np.int32)))
        topk2 = idx2.shape[2]
    fp8 = w.kv.dtype == np.uint8
    plan, ns = m.get_mla_metadata(sl, rows, h_kv, s_q=w.s_q, topk=w.topk, topk2=topk2, fp8=fp8)
    W = int(plan[0].item())                   # header word 0
    B = w.B
    o = torch.empty((B, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")
    ws_bytes = m.workspace_bytes(B, w.s_q, rows, h_kv, w.topk or 0, 512, W)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def plan_call(k):
        return m.get_mla_metadata(sl, rows, h_kv, s_q=w.s_q, topk=w.topk, topk2=topk2, fp8=fp8)

    def decode_call(k, p, n, phases):
        c = k % ncopies
        m.mla_decode_with_kvcache(qs[c], kvs[c], bt, sl, 512, p, n, causal=w.causal, indices=idx,
                                  out=(o, lse), workspace=ws, phases=phases, aux=aux)

    def step(k):
        p, n = plan_call(k)
        decode_call(k, p, n, 1)      # split decode kernel
        decode_call(k, p, n, 2)      # merge of split items

    def step_single(k):
        p, n = plan_call(k)
        decode_call(k, p, n, 4)      # split decode that merges split items itself

    def timed(fn, n):
        """GPU time of n calls of fn enqueued back to back (events at the two ends only)."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_sleep_ms(torch, 2.0 + 0.25 * n)   # host enqueues all calls meanwhile
        t0 = time.perf_counter()
        start.record()
        for k in range(n):
            fn(k)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end), time.perf_counter() - t0

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    # Timed region: K whole steps.
    total_ms, wall = timed(step, steps)
    single_ms, _ = timed(step_single, steps)
    # Each launch of the step on its own: K launches back to back on the
    # stream the library launches on, so the average is the launch duration
    # plus the gap between two launches.
    plan_total, _ = timed(plan_call, steps)
    dec_total, _ = timed(lambda k: decode_call(k, plan, ns, 1), steps)
    comb_total, _ = timed(lambda k: decode_call(k, plan, ns, 2), steps)
    fused_total, _ = timed(lambda k: decode_call(k, plan, ns, 4), steps)
    return dict(ms_per_step=total_ms / steps, ms_per_step_single=single_ms / steps,
                decode_single_ms=fused_total / steps, wall_s=wall, plan_ms=plan_total / steps,
                decode_ms=dec_total / steps, combine_ms=comb_total / steps, num_workers=W, o=o, lse=lse)


HERE = os.path.dirname(os.path.abspath(__file__))
DECODE_SRCS = tuple(os.path.join(HERE, "mla_paged_kv_get_amd", "csrc", f)
                    for f in ("mla_common.h", "mla_decode_kernel.h", "mla_decode.hip", "mla_decode_rows128.hip"))
PROFILES = os.path.join(HERE, "profiles")
COMPUTE_BOUND = ("near_ridge", "mtp_causal", "sparse_topk")
SECONDARY = ("grouped_heads", "sparse_prefill", "memory_bound_fp8", "sparse_topk_fp8", "dual_cache")


def source_sha256(paths=DECODE_SRCS):
    """Digest of the decode kernels' sources (counter runs are valid for one)."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key, workload):
    """HBM bytes per decode launch from the committed counter run of workload
    `key`, if it was taken on this workload and on the current kernel source;
    else None."""
    try:
        with open(os.path.join(PROFILES, f"decode_{key}_traffic.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256") != source_sha256():
        return None
    return t.get("traffic_bytes_per_launch")


def calibrate_copy(torch, mib, reps=10):
    """Plain device-to-device copies of `mib` MiB: the reference dispatches
    for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "reps": reps}), flush=True)


def cpu_baseline(w, budget_s=8.0):
    """The CPU oracle on the same workload, timed twice: with its BLAS pinned to
    one thread, then with every host core; each leg repeats the whole decode
    until about budget_s of wall time."""
    from oracle import mla_oracle as orc
    from threadpoolctl import threadpool_info, threadpool_limits

    kv_bytes, flops = algorithmic_work(w)

    def blas_threads():
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return max((i.get("num_threads") or 1) for i in infos) if infos else 1

    def leg():
        t0 = time.perf_counter()
        reps = 0
        while True:
            orc.decode(w.q, w.kv, w.block_table, w.cache_seqlens, 512, causal=w.causal,
                       indices=w.indices, aux=w.aux)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 50:
                return reps, el

    with threadpool_limits(limits=1, user_api="blas"):
        one = blas_threads()
        r1, e1 = leg()
    cores = blas_threads()
    rn, en = leg()
    return {"value": round(kv_bytes * rn / en / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 NumPy oracle, whole workload ({w.B} sequences) decoded {rn}x in {en:.1f} s "
                      f"with {cores} BLAS threads",
            "gflops": round(flops * rn / en / 1e9, 3),
            "one_thread": {"value": round(kv_bytes * r1 / e1 / 1e9, 4), "unit": "GB/s", "cores": one,
                           "gflops": round(flops * r1 / e1 / 1e9, 3),
                           "sample": f"the same, decoded {r1}x in {e1:.1f} s with {one} BLAS thread"},
            "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="memory_bound",
                    choices=["tiny", "memory_bound", "near_ridge", "mtp_causal", "sparse_topk",
                             "grouped_heads", "sparse_prefill", "memory_bound_fp8", "sparse_topk_fp8",
                             "dual_cache"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-compute-bound", action="store_true",
                    help="skip the near-ridge, MTP-causal and sparse top-k workloads")
    ap.add_argument("--secondary", action="store_true",
                    help="also time the grouped-heads, sparse-prefill, the two packed-FP8 and the "
                         "dual-cache workloads")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode shards over sequences with no exchange, "
              "and this build runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return
    import mla_paged_kv_get_amd as m
    from mla_paged_kv_get_amd import workloads as wl

    w = wl.NAMED[args.workload]()
    kv_bytes, flops = algorithmic_work(w)
    r = run_workload(torch, m, w, args.steps, args.warmup)
    dec_s = r["decode_ms"] / 1e3
    dc_s = (r["decode_ms"] + r["combine_ms"]) / 1e3      # decode + combine, the step without the plan
    achieved = kv_bytes / dec_s / 1e9
    step_s = r["ms_per_step"] / 1e3
    line = {
        "metric": "paged MLA decode: achieved KV HBM GB/s + bf16 TFLOPS (% of MI355X roofline)",
        "value": round(kv_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "s_q": w.s_q, "h_q": w.h_q, "h_kv": int(w.kv.shape[2]),
                   "d_qk": int(w.q.shape[3]), "dv": 512, "page": 64, "causal": bool(w.causal),
                   "topk": w.topk, "kv_bytes": kv_bytes, "flops": flops,
                   "num_workers": r["num_workers"], "kv_copies_rotated": NCOPIES},
        "tflops": round(flops / step_s / 1e12, 3),
        "step_breakdown_ms": {"plan": round(r["plan_ms"], 5), "decode": round(r["decode_ms"], 5),
                              "combine": round(r["combine_ms"], 5),
                              "single_launch_decode": round(r["decode_single_ms"], 5),
                              "single_launch_step": round(r["ms_per_step_single"], 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, w.name),
                     "frac_decode_plus_combine": round(kv_bytes / dc_s / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": "split decode kernel", "launch_ms": round(r["decode_ms"], 5),
                     "mfma_tflops": round(flops / dec_s / 1e12, 2),
                     "mfma_frac": round(flops / dec_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    def other(names, steps):
        out = {}
        for name in names:
            print(f"bench: timing {name}", file=sys.stderr, flush=True)
            w2 = wl.NAMED[name]()
            kb, fl = algorithmic_work(w2)
            r2 = run_workload(torch, m, w2, steps, 3)
            d2 = r2["decode_ms"] / 1e3
            dc2 = (r2["decode_ms"] + r2["combine_ms"]) / 1e3
            out[name] = {"workload": w2.name, "kv_bytes": kb, "flops": fl,
                         "decode_ms": round(r2["decode_ms"], 5), "combine_ms": round(r2["combine_ms"], 5),
                         "plan_ms": round(r2["plan_ms"], 5), "step_ms": round(r2["ms_per_step"], 5),
                         "num_workers": r2["num_workers"],
                         "TFLOPS": round(fl / d2 / 1e12, 1), "mfma_frac": round(fl / d2 / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "kv_GBps": round(kb / d2 / 1e9, 1), "hbm_frac": round(kb / d2 / 1e9 / HBM_PEAK_GBS, 4),
                         "mfma_frac_decode_plus_combine": round(fl / dc2 / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "hbm_frac_decode_plus_combine": round(kb / dc2 / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(name, w2.name)}
            del r2, w2
            torch.cuda.empty_cache()
        return out

    if not args.no_compute_bound and args.workload == "memory_bound":
        line["compute_bound"] = other(COMPUTE_BOUND, max(10, args.steps // 2))
    if args.secondary:
        line["secondary"] = other(SECONDARY, max(10, args.steps // 2))
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
