"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the CPU oracle on the same seeded inputs."""
import math

import torch

import oracle
import paged_kv_cache_plan_amd as pka

# Tolerances stated for bf16 inputs with fp32 accumulation.
O_TOL = 2e-2
LSE_TOL = 1e-2


def cuda():
    return torch.device("cuda", 0)


def run_paged(w, rows=None, **kw):
    dev = cuda()
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=dev, **kw)
    q = w.q.to(dev)
    pool = w.paged_kv.to(dev)
    o, lse = plan.run(q, pool)
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o.float().cpu(), lse.cpu(), info


def run_ragged(w, **kw):
    dev = cuda()
    plan = pka.Plan(w.qo_indptr, w.kv_token_indptr, None, None, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, 1, causal=w.causal, sm_scale=w.sm_scale, ragged=True, device=dev, **kw)
    o, lse = plan.run_ragged(w.q.to(dev), w.k.to(dev), w.v.to(dev))
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o.float().cpu(), lse.cpu(), info


def oracle_paged(w, rows=None):
    return oracle.batch_attention_paged(w.q, w.paged_kv, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                        w.kv_last_page_len, w.causal, w.sm_scale, rows=rows)


def compare(o, lse, ref_o, ref_lse, what=""):
    """Element-wise parity with the fp64 oracle: max |dO| <= 2e-2 and
    max |dlse| <= 1e-2; rows that see no key must be exactly (0, -inf)."""
    assert o.shape == ref_o.shape and lse.shape == ref_lse.shape, (o.shape, ref_o.shape)
    assert torch.isfinite(o).all(), f"{what}: non-finite O"
    empty = torch.isneginf(ref_lse)
    assert torch.equal(torch.isneginf(lse), empty), f"{what}: -inf lse pattern differs"
    assert not torch.isnan(lse).any(), f"{what}: NaN lse"
    if empty.any():
        assert (o[empty] == 0).all(), f"{what}: rows without keys must be 0"
    err_o = (o.double() - ref_o).abs().max().item() if o.numel() else 0.0
    fin = ~empty
    err_l = (lse.double()[fin] - ref_lse[fin]).abs().max().item() if fin.any() else 0.0
    assert err_o <= O_TOL, f"{what}: max |dO| = {err_o}"
    assert err_l <= LSE_TOL, f"{what}: max |dlse| = {err_l}"
    return err_o, err_l


def sample_rows(total_q, n, seed, must=()):
    g = torch.Generator().manual_seed(seed)
    rows = set(int(x) for x in torch.randint(0, total_q, (n,), generator=g))
    rows.update(int(m) for m in must if 0 <= m < total_q)
    return sorted(rows)
