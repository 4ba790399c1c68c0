"""Graph replay across batches: a run of a PKA_GRAPH_STABLE plan is captured
into a HIP graph once; for each later batch the plan is updated in place
(pka_plan_update) and the same graph is replayed.  Every replay must equal
an eager run of an ordinary plan of that batch bit for bit, and the oracle
within tolerance; replays alternate with eager work and synchronisations."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged

pytestmark = pytest.mark.gpu


def _eager(w):
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=cuda())
    o, lse = plan.run(w.q.to(cuda()), w.paged_kv.to(cuda()))
    torch.cuda.synchronize()
    plan.close()
    return o.cpu(), lse.cpu()


def _replay_batches(ws):
    dev = cuda()
    w0 = ws[0]
    flags = pka.PKA_GRAPH_STABLE
    sizes = [pka.workspace_size(w.qo_indptr, w.kv_indptr, w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads,
                                w.head_dim, w.page_size, w.causal, flags) for w in ws]
    plan = pka.Plan(w0.qo_indptr, w0.kv_indptr, w0.kv_indices, w0.kv_last_page_len, w0.num_qo_heads,
                    w0.num_kv_heads, w0.head_dim, w0.page_size, causal=w0.causal, sm_scale=w0.sm_scale,
                    num_pages=w0.num_pages, device=dev, graph_stable=True,
                    int_ws_bytes=max(a for a, _ in sizes), float_ws_bytes=max(b for _, b in sizes))
    max_q = max(w.total_q for w in ws)
    q_buf = torch.zeros((max_q, w0.num_qo_heads, w0.head_dim), dtype=torch.bfloat16, device=dev)
    pool_buf = torch.zeros_like(w0.paged_kv, device=dev)
    o_buf = torch.zeros((max_q, w0.num_qo_heads, w0.head_dim), dtype=torch.bfloat16, device=dev)
    lse_buf = torch.zeros((max_q, w0.num_qo_heads), dtype=torch.float32, device=dev)

    def load(w):
        q_buf[:w.total_q].copy_(w.q.to(dev))
        pool_buf.copy_(w.paged_kv.to(dev))

    load(w0)
    plan.run(q_buf, pool_buf, o_buf, lse_buf)  # warm-up, eager
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(q_buf, pool_buf, o_buf, lse_buf)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, w in enumerate(ws):
            load(w)
            plan.update(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len)
            g.replay()
            torch.cuda.synchronize()
            o, lse = o_buf[:w.total_q].cpu(), lse_buf[:w.total_q].cpu()
            eo, el = _eager(w)  # eager work between replays
            assert torch.equal(o.view(torch.int16), eo.view(torch.int16)), (rep, i)
            assert torch.equal(lse.view(torch.int32), el.view(torch.int32)), (rep, i)
            if rep == 0:
                compare(o.float(), lse, *oracle_paged(w), f"graph replay {i}")
    plan.close()


def test_graph_replay_prefill_batches():
    """Append-prefill batches of different sizes (one with split KV)."""
    ws = [W.gqa_append(seed=80 + i, batch=b, prefix_range=(40, 900), chunk_range=(5, 200), num_pages=2400)
          for i, b in enumerate([3, 6, 1])]
    ws.append(W.long_causal(seed=84, batch=1, length=1500, num_pages=2400))
    _replay_batches(ws)


def test_graph_replay_decode_batches():
    """Decode batches of different sizes and lengths (split KV + merge)."""
    ws = [W.batch_decode(seed=90 + i, batch=b, kv_log2_range=(4.0, 12.0), kv_clamp=(1, 4096), num_pages=12000)
          for i, b in enumerate([16, 40, 5])]
    _replay_batches(ws)


def test_graph_stable_update_rejects_kind_change():
    dev = cuda()
    wp = W.gqa_append(seed=95, batch=2, prefix_range=(40, 90), chunk_range=(5, 20), num_pages=400)
    wd = W.batch_decode(seed=96, batch=4, kv_log2_range=(4.0, 8.0), kv_clamp=(1, 256), num_pages=400)
    plan = pka.Plan(wp.qo_indptr, wp.kv_indptr, wp.kv_indices, wp.kv_last_page_len, wp.num_qo_heads,
                    wp.num_kv_heads, wp.head_dim, wp.page_size, causal=True, num_pages=400, device=dev,
                    graph_stable=True, int_ws_bytes=1 << 20, float_ws_bytes=1 << 20)
    with pytest.raises(pka.PkaError):
        plan.update(wd.qo_indptr, wd.kv_indptr, wd.kv_indices, wd.kv_last_page_len)
    plan.close()


@pytest.mark.parametrize("decode", [False, True])
def test_graph_replay_head_dim_64_group_6(decode):
    """D=64, six query heads per KV head, page_size 4: batches of different
    sizes replayed through one captured graph."""
    if decode:
        kvs = [[3, 500, 77, 1200, 9], [64, 65], [2000, 1, 333]]
        qos = [[1] * len(k) for k in kvs]
    else:
        qos = [[30, 7, 100], [1, 64], [200]]
        kvs = [[60, 7, 300], [40, 64], [900]]
    ws = [W.build(f"graph_g6_{decode}_{i}", 97 + i, qo, kv, 12, 2, 64, 4, causal=True, num_pages=1200)
          for i, (qo, kv) in enumerate(zip(qos, kvs))]
    _replay_batches(ws)
