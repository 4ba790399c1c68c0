"""CPU pins of the seeded input generator against the oracle's own reading
of the page table (no GPU).

The generator builds flat page tables from drawn lengths (each request's
last_page_len = kv_len - (npages - 1) * page_size) and, for the
dense-vs-sparse comparison, scatters dense ragged K/V rows into a
page_size-1 pool.  Both steps must agree with how the oracle reads a page
table (FlashInfer 0.2 release blog, "flexible block sparsity and vector
sparsity"; flashinfer-trace discussion #15, "Notes on fa3_gqa_prefill_v1"):

* oracle.kv_lengths of every generated table equals the drawn lengths;
* gathering every request back through oracle.gather_paged_kv gives the
  dense K/V bit for bit (dense-vs-sparse) and never touches a poisoned slot;
* the poison covers exactly the slots no request references;
* the two-level cascade tables of the shared-prefix workload read the same
  keys, in the same order, as its flat table.
"""
import pytest
import torch

import oracle
from inputs import workloads as W


def _referenced(w):
    """bool [num_pages, page_size]: the (page, slot) pairs some request reads."""
    used = torch.zeros((w.num_pages, w.page_size), dtype=torch.bool)
    for r in range(w.batch):
        a = int(w.kv_indptr[r])
        for t in range(w.kv_lens[r]):
            used[int(w.kv_indices[a + t // w.page_size]), t % w.page_size] = True
    return used


def _check_table(w):
    assert oracle.kv_lengths(w.kv_indptr, w.kv_last_page_len, w.page_size) == list(w.kv_lens)
    assert int(w.kv_indices.min()) >= 0 and int(w.kv_indices.max()) < w.num_pages
    for r in range(w.batch):
        K, V = oracle.gather_paged_kv(w.paged_kv, w.kv_indptr, w.kv_indices, w.kv_last_page_len,
                                      w.page_size, r)
        assert K.shape[0] == w.kv_lens[r]
        assert not K.isnan().any() and not V.isnan().any(), f"request {r} reads a poisoned slot"
    if w.poisoned:
        used = _referenced(w)
        nan = w.paged_kv.isnan().flatten(3).all(-1)  # [pages, 2, ps]: the whole slot is NaN
        assert torch.equal(nan[:, 0], ~used) and torch.equal(nan[:, 1], ~used)


SMALL = {
    "tiny": lambda: W.tiny(),
    "gqa_append": lambda: W.gqa_append(batch=5, prefix_range=(20, 90), chunk_range=(3, 40), heads=4,
                                       kv_heads=2, head_dim=8, page_size=16),
    "gqa_append_ps3": lambda: W.gqa_append(batch=4, prefix_range=(1, 30), chunk_range=(1, 20), heads=2,
                                           kv_heads=1, head_dim=8, page_size=3),
    "long_causal": lambda: W.long_causal(batch=2, length=77, heads=4, kv_heads=2, head_dim=8),
    "batch_decode": lambda: W.batch_decode(batch=9, kv_log2_range=(1.0, 7.0), kv_clamp=(1, 128), heads=4,
                                           kv_heads=2, head_dim=8),
    "mixed_batch": lambda: W.mixed_batch(num_prefill=2, num_decode=5, prefix_range=(5, 40),
                                         chunk_range=(2, 30), kv_log2_range=(1.0, 6.0), kv_clamp=(1, 64),
                                         heads=4, kv_heads=2, head_dim=8),
    "p5_shape": lambda: W.p5_shape(max_len=150),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_page_table_round_trip(name):
    _check_table(SMALL[name]())


def test_full_size_tables_match_drawn_lengths():
    # the full-size recipes' tables (values drawn at a tiny head size, the
    # lengths and page tables exactly as benchmarked)
    for w in (W.gqa_append(heads=1, kv_heads=1, head_dim=8, poison=False),
              W.batch_decode(heads=1, kv_heads=1, head_dim=8, poison=False),
              W.long_causal(heads=1, kv_heads=1, head_dim=8, poison=False)):
        assert oracle.kv_lengths(w.kv_indptr, w.kv_last_page_len, w.page_size) == list(w.kv_lens)
        assert len(set(w.kv_indices.tolist())) == w.nnz_pages  # every page owned once
        assert int(w.kv_indices.max()) < w.num_pages


@pytest.mark.parametrize("batch,length,ps_pool", [(3, 37, None), (2, 64, None)])
def test_dense_vs_sparse_scatter_is_exact(batch, length, ps_pool):
    w = W.dense_vs_sparse(batch=batch, length=length, heads=2, head_dim=16)
    assert w.page_size == 1
    assert oracle.kv_lengths(w.kv_indptr, w.kv_last_page_len, 1) == [length] * batch
    for r in range(batch):
        Kp, Vp = oracle.gather_paged_kv(w.paged_kv, w.kv_indptr, w.kv_indices, w.kv_last_page_len, 1, r)
        Kd, Vd = oracle.gather_ragged_kv(w.k, w.v, w.kv_token_indptr, r)
        assert torch.equal(Kp, Kd) and torch.equal(Vp, Vd)
    # the pages really are permuted (a scatter that ignored the table would
    # still pass the equality above only by luck)
    assert w.kv_indices.tolist() != list(range(w.nnz_pages))


def test_shared_prefix_levels_read_the_flat_keys():
    w = W.shared_prefix_decode(batch=5, prefix=48, suffix_range=(1, 40), heads=4, kv_heads=2, head_dim=8)
    (qo0, kv0, idx0, last0), (qo1, kv1, idx1, last1) = w.notes["levels"]
    assert qo0.tolist() == [0, w.batch]
    K0, V0 = oracle.gather_paged_kv(w.paged_kv, kv0, idx0, last0, w.page_size, 0)
    assert K0.shape[0] == w.notes["prefix"]
    for r in range(w.batch):
        K, V = oracle.gather_paged_kv(w.paged_kv, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.page_size, r)
        K1, V1 = oracle.gather_paged_kv(w.paged_kv, kv1, idx1, last1, w.page_size, r)
        assert torch.equal(K, torch.cat([K0, K1])) and torch.equal(V, torch.cat([V0, V1]))
        assert not K.isnan().any()
    assert oracle.kv_lengths(w.kv_indptr, w.kv_last_page_len, w.page_size) == list(w.kv_lens)


def test_append_tables_cover_lengths_after_the_append():
    a = W.chunk_append(batch=6, prefix_range=(3, 50), chunk_range=(1, 20), num_kv_heads=2, head_dim=8,
                       page_size=16)
    assert oracle.kv_lengths(a.kv_indptr, a.kv_last_page_len, a.page_size) == a.seq_lens.tolist()
    assert a.seq_lens.tolist() == [p + n for p, n in zip(a.prior_lens, a.append_lens)]
    assert a.append_indptr.tolist()[-1] == sum(a.append_lens)
