"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times (same seeded inputs drawn on the GPU, same plans): the HIP
path against the CPU fp64 oracle on sampled query rows (every head of each
sampled row), plus the rows where the causal mask is extreme.  Decode is
checked on every row."""
import time

import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged, sample_rows

pytestmark = pytest.mark.gpu


def _plan(w, ragged=False):
    if ragged:
        return pka.Plan(w.qo_indptr, w.kv_token_indptr, None, None, w.num_qo_heads, w.num_kv_heads,
                        w.head_dim, 1, causal=w.causal, sm_scale=w.sm_scale, ragged=True,
                        device=cuda())
    return pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=cuda())


def _run_paged(w):
    plan = _plan(w)
    o, lse = plan.run(w.q, w.paged_kv)
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o.float().cpu(), lse.cpu(), info


def _boundary_rows(w):
    """First and last query row of every request."""
    rows = []
    for r in range(w.batch):
        a, b = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        if b > a:
            rows += [a, b - 1]
    return rows


def _check_sampled(w, o, lse, n, seed, what, extra=()):
    rows = sample_rows(w.total_q, n, seed, must=list(_boundary_rows(w)) + list(extra))
    wc = _to_cpu(w)
    t0 = time.time()
    ref_o, ref_l = oracle_paged(wc, rows=rows)
    print(f"{what}: oracle on {len(rows)} rows x {w.num_qo_heads} heads in {time.time() - t0:.1f} s",
          flush=True)
    idx = torch.as_tensor(rows)
    err = compare(o[idx], lse[idx], ref_o, ref_l, what)
    print(f"{what}: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)
    return err


class _Cpu:
    pass


def _to_cpu(w):
    c = _Cpu()
    for k in ("qo_indptr", "kv_indptr", "kv_indices", "kv_last_page_len", "causal", "sm_scale"):
        setattr(c, k, getattr(w, k))
    c.q = w.q.cpu()
    c.paged_kv = w.paged_kv.cpu()
    return c


def test_dense_vs_vector_sparse_full():
    """B=16, L=1024, Hq=Hkv=32, D=128, causal; page_size=1 permuted pool and
    the dense ragged K/V that filled it: the two runs agree on every row and
    both match the oracle on sampled rows."""
    w = W.dense_vs_sparse(device=cuda())
    o_p, l_p, info = _run_paged(w)
    plan = _plan(w, ragged=True)
    o_r, l_r = plan.run_ragged(w.q, w.k, w.v)
    torch.cuda.synchronize()
    plan.close()
    o_r, l_r = o_r.float().cpu(), l_r.cpu()
    assert info["num_queues"] > 1 and info["num_merge_groups"] == 0
    d_o = (o_p - o_r).abs().max().item()
    d_l = (l_p - l_r).abs().max().item()
    assert d_o <= 2e-2 and d_l <= 1e-2, (d_o, d_l)
    print(f"dense_vs_sparse: paged vs ragged on every row: max |dO| {d_o:.2e}, max |dlse| {d_l:.2e}", flush=True)
    _check_sampled(w, o_p, l_p, 2048, 21, "dense_vs_sparse paged")
    _check_sampled(w, o_r, l_r, 512, 24, "dense_vs_sparse ragged")


def test_gqa_append_full():
    """B=32 append chunks over prefixes in [512, 8192], Hq=32, Hkv=8, ps=16."""
    w = W.gqa_append(device=cuda())
    o, lse, _ = _run_paged(w)
    _check_sampled(w, o, lse, 2048, 22, "gqa_append")


def test_long_causal_full():
    """B=2, L=16384, Hq=32, Hkv=8, ps=16: 4096 sampled rows plus rows 0 and
    L-1 of both requests (the first row sees one key, the last all)."""
    w = W.long_causal(device=cuda())
    o, lse, _ = _run_paged(w)
    assert torch.isfinite(o).all()
    _check_sampled(w, o, lse, 4096, 23, "long_causal")


def test_batch_decode_full():
    """B=256 single-token queries, KV lengths log-uniform in [128, 32768],
    split-KV plus merge: every row."""
    w = W.batch_decode(device=cuda())
    o, lse, info = _run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE and info["num_merge_groups"] > 0
    wc = _to_cpu(w)
    t0 = time.time()
    ref_o, ref_l = oracle_paged(wc)
    print(f"batch_decode: oracle on all {w.total_q} rows in {time.time() - t0:.1f} s", flush=True)
    err = compare(o, lse, ref_o, ref_l, "batch_decode")
    print(f"batch_decode: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)


def test_very_long_kv():
    """KV far past the benchmark sizes: decode rows over 131072, 3 and 4096
    keys (many split chunks per row, so large merge groups), and an
    append chunk of 200 queries over a 100000-token prefix, on sampled rows."""
    w = W.build("long_kv_decode", 31, [1, 1, 1], [131072, 3, 4096], 32, 8, 128, 16, causal=True,
                pool_slack=0.01, device=cuda())
    o, lse, info = _run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE and info["num_merge_groups"] > 0
    ref_o, ref_l = oracle_paged(_to_cpu(w))
    compare(o, lse, ref_o, ref_l, "long kv decode")
    del w
    w = W.build("long_kv_append", 32, [200], [100200], 32, 8, 128, 16, causal=True, pool_slack=0.01,
                device=cuda())
    o, lse, info = _run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_PREFILL
    _check_sampled(w, o, lse, 48, 24, "long kv append")
