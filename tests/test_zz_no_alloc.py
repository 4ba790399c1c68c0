"""pka_run_noalloc (partial states in the library's static device scratch)
against pka_run (partial states in the plan's float workspace), through the
C ABI: the same kernels, so bit-identical outputs, and both within tolerance
of the CPU oracle.  Two calls in a row on one GPU, the second with a smaller
batch, so the second reads a scratch the first left behind; plus a plan
whose partial states exceed the scratch, which must be refused.  A mixed
prefill + decode batch goes through the same entry point (in one launch, and
as two launches)."""
import os

import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged

pytestmark = pytest.mark.gpu


def _both(w, **kw):
    dev = cuda()
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale, num_pages=w.num_pages,
                    device=dev, **kw)
    q, pool = w.q.to(dev), w.paged_kv.to(dev)
    shape = (w.total_q, w.num_qo_heads, w.head_dim)
    o1 = torch.full(shape, 7.0, dtype=torch.bfloat16, device=dev)
    l1 = torch.full(shape[:2], 7.0, dtype=torch.float32, device=dev)
    o2, l2 = o1.clone(), l1.clone()
    plan.run(q, pool, o1, l1)
    plan.run_noalloc(q, pool, o2, l2)
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o1.cpu(), l1.cpu(), o2.cpu(), l2.cpu(), info


CASES = [
    # decode with split KV (merge groups), then a smaller decode batch
    ("decode", lambda: W.batch_decode(seed=301, batch=48, kv_log2_range=(6.0, 13.0), kv_clamp=(1, 8192)),
     lambda: W.batch_decode(seed=302, batch=7, kv_log2_range=(4.0, 11.0), kv_clamp=(1, 2048))),
    # prefill with split KV (few row blocks), then a smaller one
    ("prefill", lambda: W.gqa_append(seed=303, batch=2, prefix_range=(3000, 6000), chunk_range=(100, 300)),
     lambda: W.gqa_append(seed=304, batch=1, prefix_range=(500, 900), chunk_range=(20, 60))),
    # a mixed prefill + decode batch (its decode requests split KV), then a smaller one
    ("mixed", lambda: W.mixed_batch(seed=306, num_prefill=2, num_decode=24, prefix_range=(500, 2000),
                                    chunk_range=(100, 300)),
     lambda: W.mixed_batch(seed=307, num_prefill=1, num_decode=8, prefix_range=(100, 400), chunk_range=(20, 60))),
]
PLAN_KW = {"decode": {}, "prefill": {}, "mixed": {"mixed": True}, "mixed_two_launches": {"mixed_two_launches": True}}
CASES.append(("mixed_two_launches", CASES[2][1], CASES[2][2]))


@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_run_twice(name, big, small):
    for i, make in enumerate((big, small)):
        w = make()
        print(f"noalloc {name} call {i}: batch={w.batch} total_q={w.total_q}", flush=True)
        o1, l1, o2, l2, info = _both(w, **PLAN_KW[name])
        assert info["num_merge_groups"] > 0, "the case must split KV"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (name, i)
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), (name, i)
        compare(o2.float(), l2, *oracle_paged(w), f"noalloc {name} {i}")


def test_noalloc_rejects_plans_beyond_the_scratch(monkeypatch):
    # tiny forced chunks: the partial states of this decode batch need more
    # than the 64 MiB the static scratch holds
    monkeypatch.setenv("PKA_KV_CHUNK", "32")
    w = W.batch_decode(seed=305, batch=64, kv_log2_range=(13.0, 14.0), kv_clamp=(8192, 16384))
    dev = cuda()
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, causal=True, num_pages=w.num_pages, device=dev)
    assert plan.info["float_ws_bytes"] > (64 << 20)
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    with pytest.raises(pka.PkaError) as e:
        plan.run_noalloc(w.q.to(dev), w.paged_kv.to(dev), o)
    assert e.value.code == pka.PKA_ERR_WORKSPACE and "scratch" in str(e.value)
    plan.close()
