#!/usr/bin/env python3
"""Benchmark of paged-KV batch attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--warm-ms MS] [--only NAME] [--no-cpu-baseline]

A step is one run of the planned batch (every kernel the plan launches:
attention, and the split-KV merge when the plan split any KV) over inputs
already resident in HBM; the plan is made once beforehand, as a serving
engine plans a batch once and runs it for every layer.  Host planning time
is reported separately as plan_ms.

The JSON line's value is the causal paged prefill throughput on the
dense-vs-vector-sparse workload (B=16, L=1024, Hq=Hkv=32, D=128,
page_size=1, randomly permuted pages), the comparison the FlashInfer 0.2
release blog benchmarks.  The same run also reports the ragged dense
baseline, GQA append-prefill, long-context causal prefill (compute-bound)
and batch decode (HBM-bound) under "workloads".

Throughput uses algorithmic work only: prefill flops = 4 D Hq (visible
query-key pairs); decode bytes = every valid K/V row once + q + o + lse +
page ids.  Two input copies alternate between steps so that no step finds
its K/V left in the 256 MB last-level cache by the previous one.  Before the
timed steps, each workload runs at least W launches and at least --warm-ms
(default 300) of back-to-back launches: the GPU's clocks ramp up over the
first ~100 ms under load, and the timed steps measure the steady state.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "causal paged prefill TFLOP/s (D=128) and decode HBM GB/s, % of roofline"
KERNEL_SOURCES = ["prefill.hip", "decode.hip", "merge.hip", "device.h", "args.h", "planner.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "paged_kv_cache_plan_amd", "csrc", f) for f in KERNEL_SOURCES]
    paths.append(os.path.join(ROOT, "paged_kv_cache_plan_amd", "build.py"))  # compile flags
    for path in paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_flops(w) -> float:
    import paged_kv_cache_plan_amd as pka
    return 4.0 * w.head_dim * w.num_qo_heads * pka.visible_pairs(w.qo_lens, w.kv_lens, w.causal)


def decode_bytes(w) -> float:
    kv = sum(w.kv_lens) * 2 * w.num_kv_heads * w.head_dim * 2
    q = w.total_q * w.num_qo_heads * w.head_dim * 2
    o = q
    lse = w.total_q * w.num_qo_heads * 4
    idx = w.nnz_pages * 4
    return float(kv + q + o + lse + idx)


def make_plan(w, dev, ragged=False):
    import torch
    import paged_kv_cache_plan_amd as pka
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if ragged:
        plan = pka.Plan(w.qo_indptr, w.kv_token_indptr, None, None, w.num_qo_heads, w.num_kv_heads,
                        w.head_dim, 1, causal=w.causal, sm_scale=w.sm_scale, ragged=True, device=dev)
    else:
        plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                        w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                        num_pages=w.num_pages, device=dev)
    plan_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    return plan, plan_ms


WARM_MS = 300.0  # minimum back-to-back warm-up per workload (the GPU's clocks ramp up under load)


def time_launches(launch, steps, warmup):
    """Warm up (at least `warmup` launches and WARM_MS of back-to-back
    launches, so that the timed launches run at steady-state clocks), then
    time exactly `steps` launches bracketed by synchronisation.  Returns
    (total ms, per-launch ms list) from HIP events recorded on the stream the
    library launches on (torch's current stream)."""
    import torch
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), warmup
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        for _ in range(4):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start.record()
    for i in range(steps):
        evs[i][0].record()
        launch(i)
        evs[i][1].record()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end), [a.elapsed_time(b) for a, b in evs]


def bench_workload(name, w, dev, steps, warmup, ragged=False, copies=2):
    import torch
    plan, plan_ms = make_plan(w, dev, ragged)
    qs = [w.q] + [w.q.clone() for _ in range(copies - 1)]
    if ragged:
        ks = [w.k] + [w.k.clone() for _ in range(copies - 1)]
        vs = [w.v] + [w.v.clone() for _ in range(copies - 1)]
    else:
        pools = [w.paged_kv] + [w.paged_kv.clone() for _ in range(copies - 1)]
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.total_q, w.num_qo_heads), dtype=torch.float32, device=dev)

    def launch(i):
        c = i % copies
        if ragged:
            plan.run_ragged(qs[c], ks[c], vs[c], o, lse)
        else:
            plan.run(qs[c], pools[c], o, lse)

    total_ms, per = time_launches(launch, steps, warmup)
    info = plan.info
    plan.close()
    per_sorted = sorted(per)
    med = per_sorted[len(per) // 2]
    avg = sum(per) / len(per)
    res = {"ms_per_step": total_ms / steps, "launch_ms_avg": avg, "launch_ms_median": med,
           "launch_ms_min": per_sorted[0], "plan_ms": plan_ms, "units": info["num_units"],
           "merge_groups": info["num_merge_groups"], "kv_chunk": info["kv_chunk"],
           "kernel": "decode" if info["kernel"] == 1 else "prefill"}
    if info["kernel"] == 1:
        b = decode_bytes(w)
        res.update({"algorithmic_bytes": b, "GB_per_s": b / (avg * 1e-3) / 1e9,
                    "frac_of_hbm_peak": b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS})
    else:
        f = prefill_flops(w)
        res.update({"algorithmic_flops": f, "TFLOP_per_s": f / (avg * 1e-3) / 1e12,
                    "frac_of_bf16_peak": f / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
    del qs, o, lse
    if ragged:
        del ks, vs
    else:
        del pools
    torch.cuda.empty_cache()
    return res


def bench_append(w, dev, steps, warmup, copies=4, pools=2):
    """Paged-KV append of one batch: the batch-indices/positions launch and
    the copy launch, each timed with HIP events on the launch stream.  Four
    copies of the appended rows and two pools alternate, so the working set
    (~430 MB) exceeds the 256 MB MALL; every launch rewrites the same slots."""
    import torch
    import paged_kv_cache_plan_amd as pka
    ind, sl = w.append_indptr.to(dev), w.seq_lens.to(dev)
    kvi, kvp = w.kv_indices.to(dev), w.kv_indptr.to(dev)
    ks = [w.append_k] + [w.append_k.clone() for _ in range(copies - 1)]
    vs = [w.append_v] + [w.append_v.clone() for _ in range(copies - 1)]
    bi, pos = pka.get_batch_indices_positions(ind, sl, w.nnz)
    pls = [w.paged_kv] + [w.paged_kv.clone() for _ in range(pools - 1)]

    def idx_launch(i):
        pka.get_batch_indices_positions(ind, sl, w.nnz)

    def app_launch(i):
        c = i % copies
        pka.append_paged_kv(ks[c], vs[c], bi, pos, pls[i % pools], kvi, kvp)

    _, per_idx = time_launches(idx_launch, steps, warmup)
    total_ms, per = time_launches(app_launch, steps, warmup)
    avg = sum(per) / len(per)
    row = w.num_kv_heads * w.head_dim * 2
    b = w.nnz * (4 * row + 8)  # K and V rows read and written, plus the index pair
    return {"ms_per_step": total_ms / steps, "launch_ms_avg": avg, "launch_ms_min": min(per),
            "indices_launch_ms_avg": sum(per_idx) / len(per_idx), "tokens": w.nnz,
            "algorithmic_bytes": b, "GB_per_s": b / (avg * 1e-3) / 1e9,
            "frac_of_hbm_peak": b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, "kernel": "append"}
    # (the caller drops the workload afterwards; the copies go with this frame)


def _sub_batch(w, rs):
    """Page table and row indices of requests rs of w, as a batch of their own."""
    qo, kv, idx, last, rows = [0], [0], [], [], []
    for r in rs:
        a, b = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        rows += list(range(a, b))
        qo.append(qo[-1] + b - a)
        pa, pb = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        kv.append(kv[-1] + pb - pa)
        idx += w.kv_indices[pa:pb].tolist()
        last.append(int(w.kv_last_page_len[r]))
    return qo, kv, idx, last, rows


def bench_mixed(w, dev, steps, warmup, copies=2):
    """One chunked-prefill serving step (prefill chunks and decode requests in
    one batch), three ways, each timed with HIP events on the caller's stream:
    (a) PKA_MIXED_BATCH: the prefill and decode kernels side by side on a
    split of the compute units; (b) one ordinary plan, whose prefill kernel
    takes every row; (c) the prefill requests, then the decode requests, as
    two plans run one after the other."""
    import torch
    import paged_kv_cache_plan_amd as pka
    mk = lambda qo, kv, idx, last, **kw: pka.Plan(qo, kv, idx, last, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                                  w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                                                  num_pages=w.num_pages, device=dev, **kw)
    full = (w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len)
    t0 = time.perf_counter()
    plan_mixed = mk(*full, mixed=True)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan_whole = mk(*full)
    pre = [r for r in range(w.batch) if w.qo_lens[r] > 1]
    dec = [r for r in range(w.batch) if w.qo_lens[r] == 1]
    sp, sd = _sub_batch(w, pre), _sub_batch(w, dec)
    plan_p, plan_d = mk(*sp[:4]), mk(*sd[:4])
    qs = [w.q] + [w.q.clone() for _ in range(copies - 1)]
    pools = [w.paged_kv] + [w.paged_kv.clone() for _ in range(copies - 1)]
    q_p = [q[sp[4]] for q in qs]
    q_d = [q[sd[4]] for q in qs]
    H, D = w.num_qo_heads, w.head_dim
    o = torch.empty((w.total_q, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.total_q, H), dtype=torch.float32, device=dev)
    o_p, l_p = o[:len(sp[4])], lse[:len(sp[4])]
    o_d, l_d = o[len(sp[4]):], lse[len(sp[4]):]

    def run_mixed(i):
        plan_mixed.run(qs[i % copies], pools[i % copies], o, lse)

    def run_whole(i):
        plan_whole.run(qs[i % copies], pools[i % copies], o, lse)

    def run_seq(i):
        plan_p.run(q_p[i % copies], pools[i % copies], o_p, l_p)
        plan_d.run(q_d[i % copies], pools[i % copies], o_d, l_d)

    res = {"kernel": "mixed", "plan_ms": plan_ms, "requests_prefill": len(pre), "requests_decode": len(dec),
           "prefill_cus": plan_mixed.info["prefill_cus"], "decode_cus": plan_mixed.info["decode_cus"]}
    for name, fn in (("mixed", run_mixed), ("single_launch", run_whole), ("sequential", run_seq)):
        _, per = time_launches(fn, steps, warmup)
        res[f"{name}_ms_avg"] = sum(per) / len(per)
        res[f"{name}_ms_median"] = sorted(per)[len(per) // 2]
    for p in (plan_mixed, plan_whole, plan_p, plan_d):
        p.close()
    flop = 4.0 * D * H * pka.visible_pairs([w.qo_lens[r] for r in pre], [w.kv_lens[r] for r in pre], w.causal)
    kv_bytes = 4.0 * w.num_kv_heads * D * sum(w.kv_lens[r] for r in dec)
    t = res["mixed_ms_avg"] * 1e-3
    res.update({"prefill_flops": flop, "decode_kv_bytes": kv_bytes,
                "speedup_vs_sequential": res["sequential_ms_avg"] / res["mixed_ms_avg"],
                "speedup_vs_single_launch": res["single_launch_ms_avg"] / res["mixed_ms_avg"],
                "ms_per_step": res["mixed_ms_avg"]})
    del qs, pools, q_p, q_d, o, lse
    torch.cuda.empty_cache()
    return res


def bench_cascade(w, dev, steps, warmup, copies=2):
    """Batch decode over a long shared prefix, two ways, each timed with HIP
    events on the caller's stream: (a) one flat decode plan whose page table
    lists the prefix in every request; (b) the two-level cascade (level 0:
    all queries over the prefix, read once; level 1: each request over its
    suffix; then the state merge).  decode_bytes is what the flat form must
    read; cascade_unique_bytes the K/V the cascade reads once."""
    import torch
    import paged_kv_cache_plan_amd as pka
    flat = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale, num_pages=w.num_pages,
                    device=dev)
    t0 = time.perf_counter()
    casc = pka.Cascade(w.notes["levels"], w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                       causal=w.causal, sm_scale=w.sm_scale, num_pages=w.num_pages, device=dev)
    plan_ms = (time.perf_counter() - t0) * 1e3
    qs = [w.q] + [w.q.clone() for _ in range(copies - 1)]
    pools = [w.paged_kv] + [w.paged_kv.clone() for _ in range(copies - 1)]
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.total_q, w.num_qo_heads), dtype=torch.float32, device=dev)

    def run_flat(i):
        flat.run(qs[i % copies], pools[i % copies], o, lse)

    def run_cascade(i):
        casc.run(qs[i % copies], pools[i % copies])

    res = {"kernel": "cascade", "plan_ms": plan_ms, "requests": w.batch, "prefix": w.notes["prefix"],
           "levels": len(w.notes["levels"])}
    for name, fn in (("flat", run_flat), ("cascade", run_cascade)):
        _, per = time_launches(fn, steps, warmup)
        res[f"{name}_ms_avg"] = sum(per) / len(per)
        res[f"{name}_ms_median"] = sorted(per)[len(per) // 2]
    flat.close()
    casc.close()
    b = decode_bytes(w)
    row = 4.0 * w.num_kv_heads * w.head_dim
    unique = row * (w.notes["prefix"] + sum(w.notes["suffixes"]))
    res.update({"decode_bytes": b, "cascade_unique_bytes": unique,
                "flat_GB_per_s": b / (res["flat_ms_avg"] * 1e-3) / 1e9,
                "speedup": res["flat_ms_avg"] / res["cascade_ms_avg"], "ms_per_step": res["cascade_ms_avg"]})
    del qs, pools, o, lse
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, budget_s=10.0):
    """The CPU fp64 oracle, as it stands, on a bounded sample of the headline
    workload (the same inputs the GPU was timed on, copied to the host):
    whole requests (all heads, all rows), request after request and pass
    after pass over the batch, until ~budget_s seconds of CPU work."""
    import torch

    import oracle
    import paged_kv_cache_plan_amd as pka
    threads = torch.get_num_threads()
    w.q, w.paged_kv = w.q.cpu(), w.paged_kv.cpu()
    done, flops, t_total = 0, 0.0, 0.0
    while t_total < budget_s:
        r = done % w.batch
        q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        t0 = time.perf_counter()
        oracle.batch_attention_paged(w.q, w.paged_kv, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                     w.kv_last_page_len, True, w.sm_scale, rows=list(range(q0, q1)))
        t_total += time.perf_counter() - t0
        flops += 4.0 * w.head_dim * w.num_qo_heads * pka.visible_pairs([q1 - q0], [w.kv_lens[r]], True)
        done += 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} request runs ({done / w.batch:.1f} passes over the {w.batch} requests, all "
                      f"{w.num_qo_heads} heads, all rows) of the dense-vs-vector-sparse workload, paged "
                      f"page_size=1, fp64 torch CPU, {t_total:.1f} s", "os_cpu_count": os.cpu_count()}


def load_traffic():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None  # kernel changed since the counters were taken
    return t


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="minimum back-to-back warm-up per workload before timing (ms)")
    ap.add_argument("--only", default=None,
                    help="run one workload: dense_vs_sparse_paged, dense_vs_sparse_ragged, gqa_append, long_causal, batch_decode, append, mixed, cascade (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    WARM_MS = args.warm_ms
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_plan_amd as pka
    from paged_kv_cache_plan_amd import workloads as W
    pka.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4}))
        return

    prop = torch.cuda.get_device_properties(dev)
    sel = args.only
    results = {}

    def want(n):
        return sel is None or sel == n

    w2 = None
    if want("dense_vs_sparse_paged") or want("dense_vs_sparse_ragged"):
        w2 = W.dense_vs_sparse(device=dev)
        if want("dense_vs_sparse_paged"):
            results["dense_vs_sparse_paged_ps1"] = bench_workload("dense_vs_sparse_paged", w2, dev, args.steps, args.warmup)
            print(f"# dense_vs_sparse paged: {results['dense_vs_sparse_paged_ps1']}", file=sys.stderr, flush=True)
        if want("dense_vs_sparse_ragged"):
            results["dense_vs_sparse_ragged"] = bench_workload("dense_vs_sparse_ragged", w2, dev, args.steps, args.warmup,
                                                               ragged=True)
            print(f"# dense_vs_sparse ragged: {results['dense_vs_sparse_ragged']}", file=sys.stderr, flush=True)
        w2.k = w2.v = None
    if want("gqa_append"):
        w3 = W.gqa_append(device=dev)
        results["gqa_append"] = bench_workload("gqa_append", w3, dev, args.steps, args.warmup)
        print(f"# gqa_append: {results['gqa_append']}", file=sys.stderr, flush=True)
        del w3
    if want("long_causal"):
        w4 = W.long_causal(device=dev)
        results["long_causal"] = bench_workload("long_causal", w4, dev, args.steps, args.warmup)
        print(f"# long_causal: {results['long_causal']}", file=sys.stderr, flush=True)
        del w4
    if want("batch_decode"):
        w5 = W.batch_decode(device=dev)
        results["batch_decode"] = bench_workload("batch_decode", w5, dev, args.steps, args.warmup)
        print(f"# batch_decode: {results['batch_decode']}", file=sys.stderr, flush=True)
        del w5
    if want("append"):
        wa = W.chunk_append(device=dev)
        results["chunk_append"] = bench_append(wa, dev, args.steps, args.warmup)
        print(f"# append: {results['chunk_append']}", file=sys.stderr, flush=True)
        del wa
    torch.cuda.empty_cache()
    if want("mixed"):
        wm = W.mixed_batch(device=dev)
        results["mixed_batch"] = bench_mixed(wm, dev, args.steps, args.warmup)
        print(f"# mixed: {results['mixed_batch']}", file=sys.stderr, flush=True)
        del wm
        torch.cuda.empty_cache()
    if want("cascade"):
        wc = W.shared_prefix_decode(device=dev)
        results["shared_prefix_decode"] = bench_cascade(wc, dev, args.steps, args.warmup)
        print(f"# cascade: {results['shared_prefix_decode']}", file=sys.stderr, flush=True)
        del wc
        torch.cuda.empty_cache()

    if sel is not None:
        print(json.dumps({"only": sel, "results": results}))
        return

    main_r = results["dense_vs_sparse_paged_ps1"]
    rag = results["dense_vs_sparse_ragged"]
    traffic = load_traffic()
    roofline = {"bound": "mfma", "achieved": main_r["TFLOP_per_s"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": main_r["TFLOP_per_s"] / PEAK_BF16_TFLOPS,
                "traffic": traffic.get("dense_vs_sparse_paged_bytes_per_launch") if traffic else None,
                "kernel": "prefill_kernel<128, paged, causal>",
                "per_launch_flops": main_r["algorithmic_flops"], "avg_launch_ms": main_r["launch_ms_avg"]}
    line = {
        "metric": METRIC,
        "value": main_r["TFLOP_per_s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense_vs_vector_sparse causal paged prefill: B=16, L=1024, Hq=Hkv=32, "
                               "D=128, page_size=1, randomly permuted pages",
                   "batch": 16, "seq_len": 1024, "num_qo_heads": 32, "num_kv_heads": 32, "head_dim": 128,
                   "page_size": 1, "parallelism": "single GPU"},
        "roofline": roofline,
        "paged_over_ragged": main_r["TFLOP_per_s"] / rag["TFLOP_per_s"],
        "device": {"name": prop.name, "compute_units": prop.multi_processor_count,
                   "clock_khz": getattr(prop, "clock_rate", None)},
        "workloads": results,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w2)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
