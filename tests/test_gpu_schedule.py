"""Persistent scheduling of the prefill kernel: a worker takes units from
its own XCD's queue and, once that is empty, from the other queues; the
launch's last worker resets every queue's counter for the next run.  Runs of
one plan back to back, with another plan's runs in between, must each cover
every unit exactly once: bit-identical outputs, within tolerance of the
oracle."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged

pytestmark = pytest.mark.gpu


def _plan(w):
    return pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=cuda())


# uneven queues: one long request over few KV heads leaves most queues short
# or empty, so their workers go on to the other queues; and many equal groups
@pytest.mark.parametrize("qo,kv,Hkv,ps", [([1500, 90, 70], [3000, 90, 70], 2, 16),
                                          ([300] * 40, [300] * 40, 8, 1)])
def test_repeated_runs_cover_every_unit_once(qo, kv, Hkv, ps):
    dev = cuda()
    w = W.build("sched", 91, qo, kv, 4 * Hkv, Hkv, 128, ps, causal=True, pool_slack=0.05)
    w2 = W.build("sched_other", 92, [64] * 6, [200] * 6, 8, 2, 128, 16, causal=True)
    plan, other = _plan(w), _plan(w2)
    assert plan.info["kernel"] == pka.PKA_KERNEL_PREFILL and plan.info["num_queues"] > 1
    q, pool = w.q.to(dev), w.paged_kv.to(dev)
    q2, pool2 = w2.q.to(dev), w2.paged_kv.to(dev)
    outs = []
    for i in range(8):
        o, lse = plan.run(q, pool)
        other.run(q2, pool2)
        outs.append((o, lse))
        if i % 3 == 2:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    o0, l0 = outs[0]
    for i, (o, lse) in enumerate(outs[1:], 1):
        assert torch.equal(o, o0) and torch.equal(lse, l0), f"run {i} differs from run 0"
    plan.close()
    other.close()
    compare(o0.float().cpu(), l0.cpu(), *oracle_paged(w), f"repeated runs qo={qo[:3]} Hkv={Hkv}")
