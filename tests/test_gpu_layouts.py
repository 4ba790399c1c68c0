"""Strided KV layouts (pka_run_paged_strided): the same logical pages stored
as NHD views, HND pages, separate K and V pools, and pages spaced apart in a
larger buffer.  Only the addresses change, so every layout must give the
standard NHD run's o and lse bit for bit; the standard run is checked against
the oracle."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged

pytestmark = pytest.mark.gpu


def _layouts(pool):
    """(name, k_view, v_view) [num_pages, ps, Hkv, D] views of the same values."""
    P, _, ps, Hkv, D = pool.shape
    out = [("nhd_views", pool[:, 0], pool[:, 1])]
    hnd = pool.permute(0, 1, 3, 2, 4).contiguous()  # [P, 2, Hkv, ps, D]
    out.append(("hnd", hnd[:, 0].permute(0, 2, 1, 3), hnd[:, 1].permute(0, 2, 1, 3)))
    out.append(("split", pool[:, 0].contiguous(), pool[:, 1].contiguous()))
    half = ps * Hkv * D
    pad = 64
    store = torch.full((P, 2 * half + pad), float("nan"), dtype=pool.dtype, device=pool.device)
    store[:, :2 * half] = pool.reshape(P, 2 * half)
    st = (2 * half + pad, Hkv * D, D, 1)
    out.append(("padded", store.as_strided((P, ps, Hkv, D), st, 0), store.as_strided((P, ps, Hkv, D), st, half)))
    return out


def _plan(w):
    return pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=cuda())


def _check_layouts(w, what):
    dev = cuda()
    plan = _plan(w)
    q, pool = w.q.to(dev), w.paged_kv.to(dev)
    o0, l0 = plan.run(q, pool)
    torch.cuda.synchronize()
    compare(o0.float().cpu(), l0.cpu(), *oracle_paged(w), what)
    for name, k, v in _layouts(pool):
        o, l = plan.run_strided(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), (what, name)
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32)), (what, name)
    plan.close()


@pytest.mark.parametrize("ps", [1, 3, 16])
def test_prefill_layouts(ps):
    w = W.gqa_append(seed=60 + ps, batch=3, prefix_range=(40, 300), chunk_range=(5, 130), page_size=ps)
    _check_layouts(w, f"prefill ps={ps}")


@pytest.mark.parametrize("ps", [3, 16])
def test_decode_layouts(ps):
    w = W.batch_decode(seed=70 + ps, batch=12, kv_log2_range=(4.0, 11.0), kv_clamp=(1, 2048), page_size=ps)
    _check_layouts(w, f"decode ps={ps}")


@pytest.mark.parametrize("decode", [False, True])
def test_layouts_head_dim_64_group_6(decode):
    """Head strides at D=64 with six query heads per KV head."""
    qo = [1] * 9 if decode else [20, 1, 77, 6]
    kv = [3, 40, 129, 1, 300, 64, 65, 2, 17] if decode else [20, 33, 200, 6]
    w = W.build(f"layouts_g6_{decode}", 75 + decode, qo, kv, 12, 2, 64, 4, causal=True, pool_slack=0.1)
    _check_layouts(w, f"D=64 G=6 decode={decode}")


def test_strided_rejects_bad_strides():
    w = W.tiny()
    dev = cuda()
    plan = _plan(w)
    pool = w.paged_kv.to(dev)
    k = pool[:, 0]
    bad = k.as_strided(k.shape, (k.stride(0), k.stride(1), 4, 1))  # head stride not a multiple of 8
    with pytest.raises(pka.PkaError):
        plan.run_strided(w.q.to(dev), bad, bad)
    plan.close()


def test_layouts_head_dim_64_three_per_cu():
    """A D=64 batch of long units (three workgroups per CU, the build made
    for three) through every layout."""
    w = W.gqa_append(seed=79, batch=32, prefix_range=(2000, 4000), chunk_range=(16, 64), page_size=16, head_dim=64)
    plan = _plan(w)
    assert plan.info["num_workers"] > 2 * 256, plan.info["num_workers"]
    plan.close()
    _check_layouts(w, "D=64 three per CU")
