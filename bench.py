#!/usr/bin/env python3
"""Benchmark of paged-KV batch attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--warm-ms MS] [--only NAME] [--no-cpu-baseline]

A step is one run of the planned batch (every kernel the plan launches:
attention, and the split-KV merge when the plan split any KV) over inputs
already resident in HBM; the plan is made once beforehand, as a serving
engine plans a batch once and runs it for every layer.  Host planning time
is reported separately as plan_ms.

The JSON line's value is the long-context causal paged prefill throughput
(B=2 requests of L=16384, Hq=32, Hkv=8, D=128, page_size=16, randomly
permuted pages), the compute-bound case, from the wall time of the timed
steps.  Its roofline is the bf16 MFMA peak.  Batch decode (B=256 single-token
queries over log-uniform KV lengths in [128, 32768], same heads, page_size
16), the HBM-bound case, is reported beside it with its own roofline against
HBM peak (``roofline_decode``).  The dense-vs-vector-sparse comparison the
FlashInfer 0.2 release blog benchmarks ("performance benchmark": causal,
head_dim 128, Gaussian inputs; here B=16, L=1024, Hq=Hkv=32, once ragged and
once paged with page_size 1), GQA append-prefill and the extra rows
(append, mixed batch, cascade) are under "workloads".

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
KERNEL_SOURCES = ["prefill_worker.h", "prefill.hip", "decode_worker.h", "decode.hip", "mixed.hip", "merge.hip",
                  "append.hip", "device.h", "args.h", "planner.h"]


def _code_only(text: str) -> str:
    """C++ source without its // comments and blank lines (the kernel sources
    have no block comments and no // inside strings)."""
    lines = (line.split("//", 1)[0].rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash() -> str:
    """Hash of the code behind the measured kernels: their sources without
    comments, and the build script (compile flags), so that an edit to a
    comment does not mark profiles/traffic.json as stale."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_plan_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    with open(os.path.join(ROOT, "paged_kv_cache_plan_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def visible_pairs(qo_lens, kv_lens, causal=True) -> int:
    """Number of (query, key) pairs the attention definition visits: with the
    bottom-right causal mask, row i of a request sees min(kv, max(0, i + kv -
    qo + 1)) keys; without it, all kv keys."""
    total = 0
    for q, k in zip(qo_lens, kv_lens):
        if not causal:
            total += q * k
            continue
        blind = max(0, q - k)  # rows with i + k - q + 1 <= 0 see no key
        n = q - blind          # rows that see at least one key: 1, 2, ... n + (k - q) keys
        if n:
            first = blind + k - q + 1
            total += n * first + n * (n - 1) // 2
    return total


def prefill_flops(w) -> float:
    return 4.0 * w.head_dim * w.num_qo_heads * visible_pairs(w.qo_lens, w.kv_lens, w.causal)


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


def plan_cost(w, dev, ragged=False, n=10):
    """Host time of Plan(...) (the library's plan call plus the binding's
    workspace allocation from torch's caching allocator): the first plan of
    the workload, then the median of n more create/destroy cycles, as a
    serving engine plans a new batch every step."""
    first = None
    times = []
    for i in range(n + 1):
        plan, ms = make_plan(w, dev, ragged)
        plan.close()
        if i == 0:
            first = ms
        else:
            times.append(ms)
    times.sort()
    return {"plan_ms": times[len(times) // 2], "plan_ms_first": first}


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
    cost = plan_cost(w, dev, ragged)
    per_sorted = sorted(per)
    med = per_sorted[len(per) // 2]
    avg = sum(per) / len(per)
    res = {"ms_per_step": total_ms / steps, "launch_ms_avg": avg, "launch_ms_median": med,
           "launch_ms_min": per_sorted[0], **cost, "units": info["num_units"],
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
    one batch), four ways, each timed with HIP events on the caller's stream:
    (a) PKA_MIXED_BATCH: one launch whose workgroups serve both kinds;
    (b) with PKA_MIXED_TWO_LAUNCHES: the prefill and decode kernels side by
    side on a split of the compute units; (c) one ordinary plan, whose
    prefill kernel takes every row; (d) the prefill requests, then the decode
    requests, as two plans run one after the other."""
    import torch
    import paged_kv_cache_plan_amd as pka
    mk = lambda qo, kv, idx, last, **kw: pka.Plan(qo, kv, idx, last, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                                  w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                                                  num_pages=w.num_pages, device=dev, **kw)
    full = (w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len)
    # plan cost as for the other workloads: the first plan, then the median
    # of 10 more create / destroy cycles (a serving engine plans every step)
    times = []
    for i in range(11):
        t0 = time.perf_counter()
        plan_mixed = mk(*full, mixed=True)
        times.append((time.perf_counter() - t0) * 1e3)
        if i < 10:
            plan_mixed.close()
    plan_ms_first = times[0]
    plan_ms = sorted(times[1:])[5]
    plan_two = mk(*full, mixed_two_launches=True)
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

    def run_two(i):
        plan_two.run(qs[i % copies], pools[i % copies], o, lse)

    def run_whole(i):
        plan_whole.run(qs[i % copies], pools[i % copies], o, lse)

    def run_seq(i):
        plan_p.run(q_p[i % copies], pools[i % copies], o_p, l_p)
        plan_d.run(q_d[i % copies], pools[i % copies], o_d, l_d)

    res = {"kernel": "mixed", "plan_ms": plan_ms, "plan_ms_first": plan_ms_first, "requests_prefill": len(pre), "requests_decode": len(dec),
           "prefill_cus": plan_mixed.info["prefill_cus"], "decode_cus": plan_mixed.info["decode_cus"]}
    for name, fn in (("mixed", run_mixed), ("two_launches", run_two), ("single_launch", run_whole),
                     ("sequential", run_seq)):
        _, per = time_launches(fn, steps, warmup)
        res[f"{name}_ms_avg"] = sum(per) / len(per)
        res[f"{name}_ms_median"] = sorted(per)[len(per) // 2]
    for p in (plan_mixed, plan_two, plan_whole, plan_p, plan_d):
        p.close()
    flop = 4.0 * D * H * visible_pairs([w.qo_lens[r] for r in pre], [w.kv_lens[r] for r in pre], w.causal)
    kv_bytes = 4.0 * w.num_kv_heads * D * sum(w.kv_lens[r] for r in dec)
    t = res["mixed_ms_avg"] * 1e-3
    res.update({"prefill_flops": flop, "decode_kv_bytes": kv_bytes,
                "speedup_vs_sequential": res["sequential_ms_avg"] / res["mixed_ms_avg"],
                "speedup_vs_single_launch": res["single_launch_ms_avg"] / res["mixed_ms_avg"],
                "speedup_vs_two_launches": res["two_launches_ms_avg"] / res["mixed_ms_avg"],
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
        casc.run(qs[i % copies], pools[i % copies], o, lse)

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


def _host_sub_batch(w, rs, kv_head):
    """Requests rs of workload w restricted to one KV head and its group of
    query heads, as host tensors: (q, pool, qo_indptr, kv_indptr, kv_indices,
    kv_last_page_len, qo_lens, kv_lens).  The pool keeps every page (so the
    page ids stay valid) but only the one KV head."""
    import torch
    G = w.num_qo_heads // w.num_kv_heads
    qo, kv, idx, last, rows = [0], [0], [], [], []
    for r in rs:
        a, b = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        rows.append((a, b))
        qo.append(qo[-1] + b - a)
        pa, pb = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        kv.append(kv[-1] + pb - pa)
        idx += w.kv_indices[pa:pb].tolist()
        last.append(int(w.kv_last_page_len[r]))
    heads = slice(kv_head * G, (kv_head + 1) * G)
    q = torch.cat([w.q[a:b, heads] for a, b in rows]).cpu()
    pool = w.paged_kv[:, :, :, kv_head:kv_head + 1].cpu()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32)
    return (q, pool, i32(qo), i32(kv), i32(idx), i32(last), [w.qo_lens[r] for r in rs],
            [w.kv_lens[r] for r in rs])


def cpu_baseline_prefill(sample, head_dim, sm_scale, budget_s=10.0):
    """The CPU fp64 oracle, as it stands, on a bounded sample of the
    long-context causal workload: whole requests (every row) for one KV head
    and its group of query heads, request after request, until at least
    budget_s seconds of CPU work.  Throughput is the sample's algorithmic
    flops over its time (the same per-pair count as the GPU figure)."""
    import torch

    import oracle
    q, pool, qo, kv, idx, last, qo_lens, kv_lens = sample
    G = q.shape[1]
    done, flops, t_total = 0, 0.0, 0.0
    while t_total < budget_s and done < 2 * len(qo_lens):
        r = done % len(qo_lens)
        a, b = int(qo[r]), int(qo[r + 1])
        pa, pb = int(kv[r]), int(kv[r + 1])
        t0 = time.perf_counter()
        oracle.batch_attention_paged(q[a:b], pool, torch.tensor([0, b - a], dtype=torch.int32),
                                     torch.tensor([0, pb - pa], dtype=torch.int32), idx[pa:pb], last[r:r + 1],
                                     True, sm_scale)
        t_total += time.perf_counter() - t0
        flops += 4.0 * head_dim * G * visible_pairs([qo_lens[r]], [kv_lens[r]], True)
        done += 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "os_cpu_count": os.cpu_count(), "nproc": _nproc(),
            "sample": f"{done} whole request(s) of the long-context causal workload (L={qo_lens[0]}, every "
                      f"row) for one KV head and its {G} query heads, fp64 torch CPU, {t_total:.1f} s; "
                      f"throughput = the sample's algorithmic flops / its time"}


def cpu_baseline_decode(w_host, budget_s=30.0):
    """The CPU fp64 oracle on the batch-decode workload: requests in batch
    order, all heads, until the whole batch is done or budget_s has passed;
    throughput is the algorithmic bytes of the requests done over their time."""
    import torch

    import oracle
    q, pool = w_host["q"], w_host["pool"]
    qo_indptr, kv_indptr, kv_indices, last = (w_host[k] for k in ("qo_indptr", "kv_indptr", "kv_indices", "last"))
    kv_lens, Hq, Hkv, D = w_host["kv_lens"], q.shape[1], pool.shape[3], q.shape[2]
    B = len(kv_lens)
    done, nbytes, t_total = 0, 0.0, 0.0
    chunk = 16
    while done < B and t_total < budget_s:
        rs = list(range(done, min(B, done + chunk)))
        a, b = int(qo_indptr[rs[0]]), int(qo_indptr[rs[-1] + 1])
        t0 = time.perf_counter()
        oracle.batch_attention_paged(q, pool, qo_indptr, kv_indptr, kv_indices, last, True, None,
                                     rows=list(range(a, b)))
        t_total += time.perf_counter() - t0
        nbytes += sum(kv_lens[r] * 2 * Hkv * D * 2 + Hq * D * 4 + Hq * 4 for r in rs)
        nbytes += 4 * (int(kv_indptr[rs[-1] + 1]) - int(kv_indptr[rs[0]]))
        done = rs[-1] + 1
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "nproc": _nproc(),
            "sample": f"{done} of the {B} batch-decode requests (all heads), fp64 torch CPU, {t_total:.1f} s; "
                      f"throughput = their algorithmic bytes / their time"}


def _nproc():
    import subprocess
    try:
        return int(subprocess.run(["nproc"], capture_output=True, text=True, timeout=10).stdout.strip())
    except Exception:
        return None


def peak_clock_mhz():
    """The device's peak shader clock (hipDeviceGetAttribute, ClockRate)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:  # hipDeviceAttributeClockRate (kHz)
            return v.value / 1000.0
    except OSError:
        pass
    return None


def clock_under_load(launch, n):
    """The shader clock rocm-smi reports while n launches run back to back
    (queued first, so that the GPU is busy while rocm-smi reads it)."""
    import re
    import subprocess

    import torch
    torch.cuda.synchronize()
    for i in range(n):
        launch(i)
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30).stdout
        m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", out)
        mhz = float(m.group(1)) if m else None
    except Exception:
        mhz = None
    torch.cuda.synchronize()
    return mhz


TRAFFIC_WORKLOADS = ["dense_vs_sparse_paged", "long_causal", "batch_decode", "append"]
COPY_CALIBRATION_BYTES = 1 << 30  # --copy-calibration copies 2^28 floats


def _counter_means(path):
    """Mean counter value (KiB) per kernel over the dispatches of one
    rocprofv3 --pmc CSV (one counter per run)."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def _short_kernel(name):
    n = name.replace("void ", "").replace("pka::(anonymous namespace)::", "")
    return n.split("(pka::")[0]


def summarize_traffic(prof_dir):
    """profiles/traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (directories pmc_<COUNTER>_<workload> and pmc_<COUNTER>_calib under
    prof_dir): each counter is scaled by what it reads for a plain copy of
    known size, and a workload's bytes per launch sum its attention kernels."""
    import glob

    def means(counter, tag):
        files = glob.glob(os.path.join(prof_dir, f"pmc_{counter}_{tag}", "*counter_collection.csv"))
        return _counter_means(files[0]) if files else {}

    factors = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [v for k, v in means(counter, "calib").items() if "copyBuffer" in k or "copy" in k.lower()]
        factors[counter] = (COPY_CALIBRATION_BYTES / 1024) / copy[0]
    out = {"kernel_source_hash": kernel_source_hash(), "fetch_factor": factors["FETCH_SIZE"],
           "write_factor": factors["WRITE_SIZE"], "detail": {}}
    lines = []
    for w in TRAFFIC_WORKLOADS:
        fetch, write = means("FETCH_SIZE", w), means("WRITE_SIZE", w)
        det, total = {}, 0.0
        for k in sorted(set(fetch) | set(write)):
            fb = fetch.get(k, 0.0) * 1024 * factors["FETCH_SIZE"]
            wb = write.get(k, 0.0) * 1024 * factors["WRITE_SIZE"]
            det[_short_kernel(k)] = {"fetch_bytes": fb, "write_bytes": wb}
            total += fb + wb
            lines.append(f"{w:22s} {_short_kernel(k)[:34]:34s} fetch {fetch.get(k, 0.0):12.1f} KiB -> {fb / 1e6:9.1f} MB"
                         f"   write {write.get(k, 0.0):11.1f} KiB -> {wb / 1e6:8.1f} MB")
        out["detail"][w] = det
        out[w] = total
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    return out, lines


def summarize_trace(csv_path, pattern):
    """avg/min/max duration of the kernels matching `pattern` in a rocprofv3
    --kernel-trace --stats kernel_stats.csv."""
    import csv
    import re
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if re.search(pattern, r["Name"]):
                rows.append((_short_kernel(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                             float(r["MaxNs"])))
    return rows


def load_traffic():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None  # kernel changed since the counters were taken
    return t


def roofline_entry(res, bound, kernel, traffic_key, traffic, clock_mhz, peak_mhz):
    """Roofline of a workload's attention kernel: algorithmic work per launch
    over its average launch time (HIP events on the launch stream)."""
    if bound == "mfma":
        achieved, peak, unit, work = res["TFLOP_per_s"], PEAK_BF16_TFLOPS, "TFLOP/s", res["algorithmic_flops"]
    else:
        achieved, peak, unit, work = res["GB_per_s"], PEAK_HBM_GBS, "GB/s", res["algorithmic_bytes"]
    e = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "traffic": traffic.get(traffic_key) if traffic else None, "kernel": kernel,
         "per_launch_work": work, "avg_launch_ms": res["launch_ms_avg"],
         "clock_mhz_under_load": clock_mhz, "peak_clock_mhz": peak_mhz}
    if bound == "mfma" and clock_mhz and peak_mhz:
        # the MFMA peak scales with the shader clock; HBM's does not
        e["frac_at_measured_clock"] = achieved / (peak * clock_mhz / peak_mhz)
    return e


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="minimum back-to-back warm-up per workload before timing (ms)")
    ap.add_argument("--only", default=None,
                    help="run one workload: dense_vs_sparse_paged, dense_vs_sparse_ragged, gqa_append, long_causal, "
                         "batch_decode, append, mixed, cascade (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the rocm-smi clock reading")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-traffic", metavar="DIR", default=None,
                    help="write profiles/traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR (no GPU)")
    args = ap.parse_args()
    if args.summarize_traffic:
        out, lines = summarize_traffic(args.summarize_traffic)
        print("fetch factor %.4f, write factor %.4f" % (out["fetch_factor"], out["write_factor"]))
        print("\n".join(lines))
        return
    WARM_MS = args.warm_ms
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_plan_amd as pka
    from inputs import workloads as W
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
    host = {}
    clock = None

    def want(n):
        return sel is None or sel == n

    def log(name, r):
        print(f"# {name}: {r}", file=sys.stderr, flush=True)

    if want("long_causal"):
        w4 = W.long_causal(device=dev)
        results["long_causal"] = bench_workload("long_causal", w4, dev, args.steps, args.warmup)
        log("long_causal", results["long_causal"])
        if sel is None and not args.no_clock:
            plan, _ = make_plan(w4, dev)
            o = torch.empty((w4.total_q, w4.num_qo_heads, w4.head_dim), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((w4.total_q, w4.num_qo_heads), dtype=torch.float32, device=dev)
            clock = clock_under_load(lambda i: plan.run(w4.q, w4.paged_kv, o, lse), 300)
            plan.close()
            del o, lse
        if sel is None and not args.no_cpu_baseline:
            host["long_causal"] = _host_sub_batch(w4, [0, 1], 0)
        del w4
        torch.cuda.empty_cache()
    if want("batch_decode"):
        w5 = W.batch_decode(device=dev)
        results["batch_decode"] = bench_workload("batch_decode", w5, dev, args.steps, args.warmup)
        log("batch_decode", results["batch_decode"])
        if sel is None and not args.no_cpu_baseline:
            host["batch_decode"] = {"q": w5.q.cpu(), "pool": w5.paged_kv.cpu(), "qo_indptr": w5.qo_indptr,
                                    "kv_indptr": w5.kv_indptr, "kv_indices": w5.kv_indices,
                                    "last": w5.kv_last_page_len, "kv_lens": list(w5.kv_lens)}
        del w5
        torch.cuda.empty_cache()
    if want("dense_vs_sparse_paged") or want("dense_vs_sparse_ragged"):
        w2 = W.dense_vs_sparse(device=dev)
        if want("dense_vs_sparse_paged"):
            results["dense_vs_sparse_paged_ps1"] = bench_workload("dense_vs_sparse_paged", w2, dev, args.steps,
                                                                  args.warmup)
            log("dense_vs_sparse paged", results["dense_vs_sparse_paged_ps1"])
        if want("dense_vs_sparse_ragged"):
            results["dense_vs_sparse_ragged"] = bench_workload("dense_vs_sparse_ragged", w2, dev, args.steps,
                                                               args.warmup, ragged=True)
            log("dense_vs_sparse ragged", results["dense_vs_sparse_ragged"])
        del w2
        torch.cuda.empty_cache()
    if want("gqa_append"):
        w3 = W.gqa_append(device=dev)
        results["gqa_append"] = bench_workload("gqa_append", w3, dev, args.steps, args.warmup)
        log("gqa_append", results["gqa_append"])
        del w3
        torch.cuda.empty_cache()
    if want("append"):
        wa = W.chunk_append(device=dev)
        results["chunk_append"] = bench_append(wa, dev, args.steps, args.warmup)
        log("append", results["chunk_append"])
        del wa
        torch.cuda.empty_cache()
    if want("mixed"):
        wm = W.mixed_batch(device=dev)
        results["mixed_batch"] = bench_mixed(wm, dev, args.steps, args.warmup)
        log("mixed", results["mixed_batch"])
        del wm
        torch.cuda.empty_cache()
    if want("cascade"):
        wc = W.shared_prefix_decode(device=dev)
        results["shared_prefix_decode"] = bench_cascade(wc, dev, args.steps, args.warmup)
        log("cascade", results["shared_prefix_decode"])
        del wc
        torch.cuda.empty_cache()

    if sel is not None:
        print(json.dumps({"only": sel, "results": results}))
        return

    c4 = results["long_causal"]
    c5 = results["batch_decode"]
    paged, rag = results["dense_vs_sparse_paged_ps1"], results["dense_vs_sparse_ragged"]
    traffic = load_traffic()
    peak_mhz = peak_clock_mhz()
    value = c4["algorithmic_flops"] / (c4["ms_per_step"] * 1e-3) / 1e12
    roofline = roofline_entry(c4, "mfma", "prefill_kernel<128, paged (page_size 16), causal>", "long_causal",
                              traffic, clock, peak_mhz)
    roofline_decode = roofline_entry(c5, "hbm", "decode_kernel<128, paged (page_size 16)> + split merge",
                                     "batch_decode", traffic, None, peak_mhz)
    decode_value = c5["algorithmic_bytes"] / (c5["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": c4["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long-context causal paged prefill: B=2 requests of L=16384, Hq=32, Hkv=8, "
                               "D=128, page_size=16, randomly permuted pages",
                   "batch": 2, "seq_len": 16384, "num_qo_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                   "page_size": 16, "parallelism": "single GPU"},
        "roofline": roofline,
        "decode": {"workload": "batch decode: B=256 single-token queries, KV lengths log-uniform in "
                               "[128, 32768], Hq=32, Hkv=8, D=128, page_size=16, split-KV + merge",
                   "value": decode_value, "unit": "GB/s", "ms_per_step": c5["ms_per_step"]},
        "roofline_decode": roofline_decode,
        "paged_over_ragged": paged["TFLOP_per_s"] / rag["TFLOP_per_s"],
        "gates": {"long_causal_ge_50pct_bf16_peak": value / PEAK_BF16_TFLOPS >= 0.50,
                  "batch_decode_ge_70pct_hbm_peak": decode_value / PEAK_HBM_GBS >= 0.70,
                  "page_size_1_within_10pct_of_ragged": paged["TFLOP_per_s"] / rag["TFLOP_per_s"] >= 0.90},
        "device": {"name": prop.name, "compute_units": prop.multi_processor_count, "peak_clock_mhz": peak_mhz,
                   "clock_mhz_under_load": clock},
        "workloads": results,
    }
    if not args.no_cpu_baseline:
        import torch as _t
        _t.set_num_threads(min(os.cpu_count() or 1, 16))
        line["cpu_baseline"] = cpu_baseline_prefill(host.pop("long_causal"), 128, 1.0 / (128 ** 0.5))
        line["cpu_baseline_decode"] = cpu_baseline_decode(host.pop("batch_decode"))
    print(json.dumps(line))


if __name__ == "__main__":
    main()
