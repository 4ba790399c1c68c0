"""Pins of the append oracle (oracle/append.py), CPU only.

* a hand-worked fixture (tests/golden/append_by_hand.txt);
* the round trip through the attention oracle's gather, an independent
  reading of the same page table: after an append, each request's last n
  tokens read back as the appended rows and every other pool element is
  unchanged;
* appending a batch at once equals appending its tokens one decode step at a
  time;
* planted mistakes (off-by-one position, page and slot swapped) are caught.
"""
import os

import pytest
import torch

import oracle
from oracle import append as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "append_by_hand.txt")


def _fixture():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        d[k.strip()] = v.split()
    ints = lambda k: [int(x) for x in d[k]]
    pairs = lambda k: [tuple(int(y) for y in x.split(",")) for x in d[k]]
    return d, ints, pairs


def test_golden_positions_and_slots():
    d, ints, pairs = _fixture()
    b, p = A.batch_indices_positions(ints("append_indptr"), ints("seq_lens"))
    assert b.tolist() == ints("batch_indices") and p.tolist() == ints("positions")
    b2, p2 = A.batch_indices_positions(ints("decode_append_indptr"), ints("seq_lens"))
    assert b2.tolist() == ints("decode_batch_indices") and p2.tolist() == ints("decode_positions")
    ps, npg = int(d["page_size"][0]), int(d["num_pages"][0])
    Hkv, D = 2, 3
    pool = torch.zeros((npg, 2, ps, Hkv, D), dtype=torch.float64)
    for name, (bi, po) in (("page_slot", (b, p)), ("decode_page_slot", (b2, p2))):
        n = bi.numel()
        k = torch.arange(1, n * Hkv * D + 1, dtype=torch.float64).reshape(n, Hkv, D)
        out = A.append_paged_kv(pool, k, -k, bi, po, ints("kv_indices"), ints("kv_indptr"))
        changed = sorted({(pg, sl) for pg, _, sl in (out != pool).any(-1).any(-1).nonzero().tolist()})
        assert changed == sorted(pairs(name)), name
        for i, (pg, sl) in enumerate(pairs(name)):
            assert torch.equal(out[pg, 0, sl], k[i]) and torch.equal(out[pg, 1, sl], -k[i])


def _random_append(seed, ps, B=5, Hkv=2, D=4):
    g = torch.Generator().manual_seed(seed)
    n_app = torch.randint(0, 6, (B,), generator=g).tolist()
    prior = torch.randint(0, 11, (B,), generator=g).tolist()
    seq = [a + b for a, b in zip(n_app, prior)]
    npages = [(L + ps - 1) // ps for L in seq]
    nnz_pages = sum(npages)
    num_pages = nnz_pages + 3
    perm = torch.randperm(num_pages, generator=g)[:nnz_pages].to(torch.int32)
    kv_indptr = [0]
    for n in npages:
        kv_indptr.append(kv_indptr[-1] + n)
    last = [0 if L == 0 else L - (n - 1) * ps for L, n in zip(seq, npages)]
    pool = torch.randn((num_pages, 2, ps, Hkv, D), generator=g, dtype=torch.float64)
    app_indptr = [0]
    for n in n_app:
        app_indptr.append(app_indptr[-1] + n)
    nnz = app_indptr[-1]
    k = torch.randn((nnz, Hkv, D), generator=g, dtype=torch.float64)
    v = torch.randn((nnz, Hkv, D), generator=g, dtype=torch.float64)
    return dict(pool=pool, k=k, v=v, seq=seq, n_app=n_app, prior=prior, kv_indptr=kv_indptr,
                kv_indices=perm, last=last, app_indptr=app_indptr, ps=ps)


@pytest.mark.parametrize("ps", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_through_gather(ps, seed):
    c = _random_append(seed, ps)
    b, p = A.batch_indices_positions(c["app_indptr"], c["seq"])
    out = A.append_paged_kv(c["pool"], c["k"], c["v"], b, p, c["kv_indices"], c["kv_indptr"])
    touched = torch.zeros(c["pool"].shape[:3], dtype=torch.bool)
    for r in range(len(c["seq"])):
        K0, V0 = oracle.gather_paged_kv(c["pool"], c["kv_indptr"], c["kv_indices"], c["last"], ps, r)
        K1, V1 = oracle.gather_paged_kv(out, c["kv_indptr"], c["kv_indices"], c["last"], ps, r)
        n, m = c["n_app"][r], c["prior"][r]
        a = c["app_indptr"][r]
        assert torch.equal(K1[:m], K0[:m]) and torch.equal(V1[:m], V0[:m])
        assert torch.equal(K1[m:], c["k"][a:a + n]) and torch.equal(V1[m:], c["v"][a:a + n])
        for t in range(m, m + n):
            pg = int(c["kv_indices"][c["kv_indptr"][r] + t // ps])
            touched[pg, :, t % ps] = True
    assert torch.equal(out[~touched], c["pool"][~touched])


def test_batched_equals_one_step_at_a_time():
    c = _random_append(7, 4, B=4)
    b, p = A.batch_indices_positions(c["app_indptr"], c["seq"])
    once = A.append_paged_kv(c["pool"], c["k"], c["v"], b, p, c["kv_indices"], c["kv_indptr"])
    pool = c["pool"]
    lens = list(c["prior"])
    step = 0
    while any(lens[r] < c["seq"][r] for r in range(len(lens))):
        live = [r for r in range(len(lens)) if lens[r] < c["seq"][r]]
        rows = [c["app_indptr"][r] + (lens[r] - c["prior"][r]) for r in live]
        indptr = [0]
        for r in range(len(lens)):
            indptr.append(indptr[-1] + (1 if r in live else 0))
        new_lens = [lens[r] + (1 if r in live else 0) for r in range(len(lens))]
        bb, pp = A.batch_indices_positions(indptr, new_lens)
        pool = A.append_paged_kv(pool, c["k"][rows], c["v"][rows], bb, pp, c["kv_indices"], c["kv_indptr"])
        lens = new_lens
        step += 1
    assert step > 1 and torch.equal(pool, once)


def test_planted_mistakes_are_caught():
    d, ints, pairs = _fixture()
    b, p = A.batch_indices_positions(ints("append_indptr"), ints("seq_lens"))
    assert (p + 1).tolist() != ints("positions")  # off-by-one position
    c = _random_append(3, 4)
    bi, po = A.batch_indices_positions(c["app_indptr"], c["seq"])
    ps = c["ps"]

    def swapped(pool, k, v, bi, po, idx, indptr):  # page and slot roles exchanged
        out = pool.clone()
        for i in range(k.shape[0]):
            r, q = int(bi[i]), int(po[i])
            page = int(idx[int(indptr[r]) + q % ps]) if int(indptr[r]) + q % ps < len(idx) else 0
            out[page, 0, (q // ps) % ps] = k[i]
            out[page, 1, (q // ps) % ps] = v[i]
        return out
    good = A.append_paged_kv(c["pool"], c["k"], c["v"], bi, po, c["kv_indices"], c["kv_indptr"])
    bad = swapped(c["pool"], c["k"], c["v"], bi, po, c["kv_indices"], c["kv_indptr"])
    assert not torch.equal(good, bad)
