"""GPU parity of mixed prefill + decode batches (PKA_MIXED_BATCH).

By default a mixed batch runs as one launch whose workgroups serve both
kinds (the decode worker with the prefill workgroup's waves, 8 at D=128):
* every row against the CPU oracle (tolerance);
* without split KV, its prefill rows bit-identical to the prefill kernel
  (the same worker code), and at D=64, where the wave counts agree, its
  decode rows to the decode kernel;
* repeated runs bit for bit (the queues' counters reset after every run),
  fp32 output, ragged K/V, and the full-size chunked-prefill serving step
  on sampled prefill rows and every decode row.

With PKA_MIXED_TWO_LAUNCHES the prefill launch and the decode launch run side
by side on a split of the compute units and write disjoint output rows:
* every row against the CPU oracle;
* without split KV, bit-identical to each kernel run on its own: the prefill
  rows to an ordinary plan of the whole batch (whose prefill kernel takes
  every row), the decode rows to a plan of the decode requests alone;
* the full-size serving step, ragged K/V, fp32 output, and repeated runs
  (the plan's side stream and events are reused) bit for bit."""
import random
import time

import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged, sample_rows

pytestmark = pytest.mark.gpu


def _mixed(seed, D=128, ps=16, ragged=False):
    rng = random.Random(500 + seed)
    B = rng.randint(6, 40)
    Hkv = rng.choice([1, 2, 8])
    G = rng.choice([1, 3, 4, 6, 8])
    qo = [rng.choice([1, 1, 1, 0, rng.randint(2, 400)]) for _ in range(B)]
    i, j = rng.sample(range(B), 2)
    qo[i], qo[j] = rng.randint(2, 400), 1
    kv = [max(q, rng.choice([rng.randint(1, 60), rng.randint(60, 2500)])) for q in qo]
    return W.build("mixed", 500 + seed, qo, kv, Hkv * G, Hkv, D, ps, causal=True, pool_slack=0.2,
                   ragged=ragged, poison=not ragged)


def _plan(w, **kw):
    return pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=cuda(), **kw)


def _run(w, **kw):
    plan = _plan(w, **kw)
    o, lse = plan.run(w.q.to(cuda()), w.paged_kv.to(cuda()))
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o.cpu(), lse.cpu(), info


def _decode_alone(w, **kw):
    """The decode requests as a batch of their own (compacted rows and page
    table), through an ordinary plan; returns their rows and outputs."""
    dec = [r for r in range(w.batch) if w.qo_lens[r] == 1]
    rows = [int(w.qo_indptr[r]) for r in dec]
    kv_ptr, idx, last = [0], [], []
    for r in dec:
        a, b = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        kv_ptr.append(kv_ptr[-1] + b - a)
        idx += w.kv_indices[a:b].tolist()
        last.append(int(w.kv_last_page_len[r]))
    plan = pka.Plan(list(range(len(dec) + 1)), kv_ptr, idx, last, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    w.page_size, causal=w.causal, sm_scale=w.sm_scale, num_pages=w.num_pages, device=cuda(),
                    **kw)
    assert plan.info["kernel"] == pka.PKA_KERNEL_DECODE
    o, lse = plan.run(w.q[rows].to(cuda()), w.paged_kv.to(cuda()))
    torch.cuda.synchronize()
    plan.close()
    return rows, o.cpu(), lse.cpu()


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


@pytest.mark.parametrize("seed,D,ps", [(0, 128, 16), (1, 128, 1), (2, 64, 4), (3, 128, 3)])
def test_two_launches_match_oracle_and_each_kernel(seed, D, ps):
    w = _mixed(seed, D, ps)
    o, lse, info = _run(w, mixed_two_launches=True)
    assert info["kernel"] == pka.PKA_KERNEL_MIXED
    compare(o.float(), lse, *oracle_paged(w), f"mixed seed {seed}")
    # no split: each kernel's rows equal that kernel run on its own
    o1, l1, info1 = _run(w, mixed_two_launches=True, disable_split_kv=True)
    assert info1["kernel"] == pka.PKA_KERNEL_MIXED and info1["num_merge_groups"] == 0
    op, lp, infop = _run(w, disable_split_kv=True)
    assert infop["kernel"] == pka.PKA_KERNEL_PREFILL
    pre = [row for r in range(w.batch) if w.qo_lens[r] > 1
           for row in range(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1]))]
    assert torch.equal(_bits(o1[pre]), _bits(op[pre])) and torch.equal(_bits(l1[pre]), _bits(lp[pre]))
    rows, od, ld = _decode_alone(w, disable_split_kv=True)
    assert torch.equal(_bits(o1[rows]), _bits(od)) and torch.equal(_bits(l1[rows]), _bits(ld))


def test_two_launches_repeat_and_fp32():
    w = _mixed(4)
    plan = _plan(w, mixed_two_launches=True, out_fp32=True)
    q, pool = w.q.to(cuda()), w.paged_kv.to(cuda())
    outs = []
    for _ in range(3):
        o, lse = plan.run(q, pool)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    plan.close()
    assert outs[0][0].dtype == torch.float32
    for o, lse in outs[1:]:
        assert torch.equal(_bits(o), _bits(outs[0][0])) and torch.equal(_bits(lse), _bits(outs[0][1]))
    compare(outs[0][0], outs[0][1], *oracle_paged(w), "mixed fp32")


def test_two_launches_ragged():
    w = _mixed(5, ps=1, ragged=True)
    plan = pka.Plan(w.qo_indptr, w.kv_token_indptr, None, None, w.num_qo_heads, w.num_kv_heads, w.head_dim, 1,
                    causal=w.causal, sm_scale=w.sm_scale, ragged=True, device=cuda(), mixed_two_launches=True)
    assert plan.info["kernel"] == pka.PKA_KERNEL_MIXED
    o, lse = plan.run_ragged(w.q.to(cuda()), w.k.to(cuda()), w.v.to(cuda()))
    torch.cuda.synchronize()
    plan.close()
    compare(o.float().cpu(), lse.cpu(), *oracle_paged(w), "mixed ragged")


def test_two_launches_full_size():
    """The chunked-prefill serving step the benchmark runs (4 prefill chunks,
    prefix 1024..8192, chunk 512..2048, and 192 decode requests) as two
    launches: sampled prefill rows (with every request's first and last row)
    and every decode row against the oracle."""
    w = W.mixed_batch(device=cuda())
    plan = _plan(w, mixed_two_launches=True)
    info = plan.info
    assert info["kernel"] == pka.PKA_KERNEL_MIXED
    assert info["prefill_cus"] + info["decode_cus"] == 256
    o, lse = plan.run(w.q, w.paged_kv)
    torch.cuda.synchronize()
    plan.close()
    o, lse = o.float().cpu(), lse.cpu()
    dec = [int(w.qo_indptr[r]) for r in range(w.batch) if w.qo_lens[r] == 1]
    ends = [x for r in range(w.batch) if w.qo_lens[r] > 1 for x in (int(w.qo_indptr[r]), int(w.qo_indptr[r + 1]) - 1)]
    rows = sample_rows(w.total_q, 512, 31, must=dec + ends)
    wc = W.Workload(**{**w.__dict__, "q": w.q.cpu(), "paged_kv": w.paged_kv.cpu()})
    t0 = time.time()
    ref_o, ref_l = oracle_paged(wc, rows=rows)
    print(f"mixed_batch: oracle on {len(rows)} rows in {time.time() - t0:.1f} s "
          f"(prefill cus {info['prefill_cus']}, decode cus {info['decode_cus']})", flush=True)
    idx = torch.as_tensor(rows)
    err = compare(o[idx], lse[idx], ref_o, ref_l, "mixed_batch")
    print(f"mixed_batch: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)


@pytest.mark.parametrize("seed,D,ps", [(0, 128, 16), (1, 128, 1), (2, 64, 4), (3, 128, 3), (6, 64, 16)])
def test_one_grid_matches_oracle_and_kernels(seed, D, ps):
    w = _mixed(seed, D, ps)
    print(f"one grid: seed {seed} D {D} ps {ps} batch {w.batch}", flush=True)
    o, lse, info = _run(w, mixed=True)
    assert info["kernel"] == pka.PKA_KERNEL_MIXED and info["decode_cus"] + info["prefill_cus"] == 256
    compare(o.float(), lse, *oracle_paged(w), f"one grid seed {seed}")
    o1, l1, info1 = _run(w, mixed=True, disable_split_kv=True)
    assert info1["num_merge_groups"] == 0
    op, lp, _ = _run(w, disable_split_kv=True)
    pre = [row for r in range(w.batch) if w.qo_lens[r] > 1
           for row in range(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1]))]
    assert torch.equal(_bits(o1[pre]), _bits(op[pre])) and torch.equal(_bits(l1[pre]), _bits(lp[pre]))
    if D == 64:
        rows, od, ld = _decode_alone(w, disable_split_kv=True)
        assert torch.equal(_bits(o1[rows]), _bits(od)) and torch.equal(_bits(l1[rows]), _bits(ld))


def test_one_grid_repeat_and_fp32():
    """Repeated runs of one plan are bit-identical: the last workgroup of each
    worker resets its queue counters for the next run."""
    w = _mixed(7)
    plan = _plan(w, mixed=True, out_fp32=True)
    q, pool = w.q.to(cuda()), w.paged_kv.to(cuda())
    outs = []
    for _ in range(4):
        o, lse = plan.run(q, pool)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    plan.close()
    for o, lse in outs[1:]:
        assert torch.equal(_bits(o), _bits(outs[0][0])) and torch.equal(_bits(lse), _bits(outs[0][1]))
    compare(outs[0][0], outs[0][1], *oracle_paged(w), "one grid fp32")


def test_one_grid_ragged():
    w = _mixed(8, ps=1, ragged=True)
    plan = pka.Plan(w.qo_indptr, w.kv_token_indptr, None, None, w.num_qo_heads, w.num_kv_heads, w.head_dim, 1,
                    causal=w.causal, sm_scale=w.sm_scale, ragged=True, device=cuda(), mixed=True)
    assert plan.info["kernel"] == pka.PKA_KERNEL_MIXED
    o, lse = plan.run_ragged(w.q.to(cuda()), w.k.to(cuda()), w.v.to(cuda()))
    torch.cuda.synchronize()
    plan.close()
    compare(o.float().cpu(), lse.cpu(), *oracle_paged(w), "one grid ragged")


@pytest.mark.parametrize("D", [128, 64])
def test_one_grid_full_size(D):
    """The chunked-prefill serving step as the benchmark runs it (and at
    head_dim 64, where the decode worker keeps its 4 waves), in one launch:
    sampled prefill rows (with every request's first and last row) and every
    decode row against the oracle."""
    w = W.mixed_batch(device=cuda(), head_dim=D)
    plan = _plan(w, mixed=True)
    assert plan.info["kernel"] == pka.PKA_KERNEL_MIXED
    o, lse = plan.run(w.q, w.paged_kv)
    torch.cuda.synchronize()
    plan.close()
    o, lse = o.float().cpu(), lse.cpu()
    dec = [int(w.qo_indptr[r]) for r in range(w.batch) if w.qo_lens[r] == 1]
    ends = [x for r in range(w.batch) if w.qo_lens[r] > 1 for x in (int(w.qo_indptr[r]), int(w.qo_indptr[r + 1]) - 1)]
    rows = sample_rows(w.total_q, 512, 37 + D, must=dec + ends)
    wc = W.Workload(**{**w.__dict__, "q": w.q.cpu(), "paged_kv": w.paged_kv.cpu()})
    ref_o, ref_l = oracle_paged(wc, rows=rows)
    idx = torch.as_tensor(rows)
    err = compare(o[idx], lse[idx], ref_o, ref_l, f"one grid mixed_batch D{D}")
    print(f"one grid mixed_batch D{D}: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)


def _subset(w, reqs):
    """Requests reqs of w as a batch of their own over w's pool: the index
    arrays and the rows of q (and of the whole batch's outputs) they cover."""
    qo, kv, idx, last, rows = [0], [0], [], [], []
    for r in reqs:
        a, b = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        qo.append(qo[-1] + int(w.qo_lens[r]))
        kv.append(kv[-1] + b - a)
        idx += w.kv_indices[a:b].tolist()
        last.append(int(w.kv_last_page_len[r]))
        rows += list(range(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])))
    return qo, kv, idx, last, rows


@pytest.mark.parametrize("kw", [{"mixed": True}, {"mixed_two_launches": True}], ids=["one_grid", "two_launches"])
def test_mixed_plan_update_across_kinds(kw):
    """One mixed-batch plan updated from a mixed batch to a decode-only batch,
    a prefill-only batch and another mixed batch of the same pool: every run
    against the oracle rows of its requests."""
    w = _mixed(9)
    ref_o, ref_l = oracle_paged(w)
    pre = [r for r in range(w.batch) if w.qo_lens[r] > 1]
    dec = [r for r in range(w.batch) if w.qo_lens[r] == 1]
    batches = [list(range(w.batch)), dec, pre, pre[: max(1, len(pre) // 2)] + dec[::2]]
    plan = None
    q_all, pool = w.q.to(cuda()), w.paged_kv.to(cuda())
    for i, reqs in enumerate(batches):
        qo, kv, idx, last, rows = _subset(w, reqs)
        print(f"update {i}: {len(reqs)} requests, {len(rows)} rows", flush=True)
        if plan is None:
            plan = pka.Plan(qo, kv, idx, last, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            causal=w.causal, sm_scale=w.sm_scale, num_pages=w.num_pages, device=cuda(),
                            int_ws_bytes=1 << 22, float_ws_bytes=1 << 26, **kw)
        else:
            plan.update(qo, kv, idx, last)
        kinds = {pka.PKA_KERNEL_PREFILL, pka.PKA_KERNEL_DECODE} if i in (1, 2) else {pka.PKA_KERNEL_MIXED}
        assert plan.info["kernel"] in kinds
        o, lse = plan.run(q_all[rows], pool)
        torch.cuda.synchronize()
        idx_t = torch.as_tensor(rows)
        compare(o.float().cpu(), lse.cpu(), ref_o[idx_t], ref_l[idx_t], f"update {i}")
    plan.close()


@pytest.mark.parametrize("kw", [{"mixed": True}, {"mixed_two_launches": True}], ids=["one_grid", "two_launches"])
@pytest.mark.parametrize("D,ps", [(128, 16), (64, 3)])
def test_mixed_edge_requests(kw, D, ps):
    """Mixed batches holding the edge cases of both kinds: a decode request
    with no key, causal prefill rows that see no key (qo_len > kv_len), an
    empty request, single-key requests, and one long chunk (split KV)."""
    qo = [1, 5, 0, 1, 300, 1, 2, 1]
    kv = [0, 3, 10, 1, 2000, 3000, 1, 17]
    w = W.build("mixed_edges", 777 + D + ps, qo, kv, 8, 2, D, ps, causal=True, pool_slack=0.3)
    o, lse, info = _run(w, **kw)
    assert info["kernel"] == pka.PKA_KERNEL_MIXED
    compare(o.float(), lse, *oracle_paged(w), f"mixed edges {kw} D{D} ps{ps}")
