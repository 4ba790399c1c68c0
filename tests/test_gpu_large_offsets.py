"""Pages past the first 4 GiB of the pool: K/V byte offsets that need 64
bits.  A small causal GQA batch is run twice through the C ABI, once on its
own pool and once with its pages moved past byte 2^32 of a larger pool whose
first 4 GiB hold NaN, so that an offset wrapped to 32 bits would show as NaN
or as a different result; the two runs must agree bit for bit, and with the
oracle."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged

pytestmark = pytest.mark.gpu


def _run(w, pool, kv_indices, num_pages, dev):
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=num_pages, device=dev)
    o, lse = plan.run(w.q.to(dev), pool)
    torch.cuda.synchronize()
    kernel = plan.info["kernel"]
    plan.close()
    return o.cpu(), lse.cpu(), kernel


@pytest.mark.parametrize("ps", [16, 1, 3])
@pytest.mark.parametrize("decode", [False, True])
def test_pages_past_4gib(ps, decode):
    dev = cuda()
    qo = [1, 1, 1] if decode else [300, 77, 1]
    w = W.build(f"past4g_{ps}_{decode}", 400 + ps, qo, [700, 1200, 65], 8, 2, 128, ps, causal=True)
    page_bytes = 2 * ps * w.num_kv_heads * w.head_dim * 2
    shift = (1 << 32) // page_bytes + 1  # the first page that starts past byte 2^32
    print(f"ps={ps} decode={decode}: pages moved by {shift} ({shift * page_bytes / 2**30:.2f} GiB)", flush=True)
    big = torch.empty((shift + w.num_pages,) + tuple(w.paged_kv.shape[1:]), dtype=torch.bfloat16, device=dev)
    big[:shift].fill_(float("nan"))
    big[shift:] = w.paged_kv.to(dev)
    o_big, l_big, k_big = _run(w, big, w.kv_indices + shift, shift + w.num_pages, dev)
    del big
    torch.cuda.empty_cache()
    o, lse, k = _run(w, w.paged_kv.to(dev), w.kv_indices, w.num_pages, dev)
    assert k_big == k == (pka.PKA_KERNEL_DECODE if decode else pka.PKA_KERNEL_PREFILL)
    assert torch.equal(o_big.view(torch.int16), o.view(torch.int16)) and torch.equal(l_big, lse)
    compare(o.float(), lse, *oracle_paged(w), f"ps={ps} decode={decode}")
