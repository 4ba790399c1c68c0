"""GPU parity of the paged-KV append (pka_get_batch_indices_positions and
pka_append_paged_kv, through the C ABI) against the CPU oracle in
oracle/append.py.  Both are index work and copies, so every comparison is
bit-exact: the batch indices and positions, and the whole pool after the
append (touched and untouched slots alike)."""
import pytest
import torch

from oracle import append as A
import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import cuda

pytestmark = pytest.mark.gpu


def _gpu_append(w, bi=None, pos=None):
    dev = cuda()
    if bi is None:
        bi, pos = pka.get_batch_indices_positions(w.append_indptr.to(dev), w.seq_lens.to(dev), w.nnz)
    pool = w.paged_kv.to(dev).clone()
    pka.append_paged_kv(w.append_k.to(dev), w.append_v.to(dev), bi.to(dev), pos.to(dev), pool,
                        w.kv_indices.to(dev), w.kv_indptr.to(dev))
    torch.cuda.synchronize()
    return bi.cpu(), pos.cpu(), pool.cpu()


def _oracle(w, bi=None, pos=None):
    if bi is None:
        bi, pos = A.batch_indices_positions(w.append_indptr, w.seq_lens)
    pool = A.append_paged_kv(w.paged_kv.cpu(), w.append_k.cpu(), w.append_v.cpu(), bi, pos,
                             w.kv_indices, w.kv_indptr)
    return bi, pos, pool


def _check(w):
    bi, pos, pool = _gpu_append(w)
    rb, rp, rpool = _oracle(w)
    assert torch.equal(bi, rb) and torch.equal(pos, rp)
    assert torch.equal(pool.view(torch.int16), rpool.view(torch.int16))


@pytest.mark.parametrize("ps", [1, 3, 4, 16, 128])
@pytest.mark.parametrize("D,Hkv", [(128, 8), (64, 1), (128, 2)])
def test_append_matches_oracle(ps, D, Hkv):
    g = torch.Generator().manual_seed(100 + ps + D + Hkv)
    B = 9
    prior = torch.randint(0, 300, (B,), generator=g).tolist()
    n = torch.randint(0, 70, (B,), generator=g).tolist()
    n[2] = 0  # a request that appends nothing
    prior[4] = 0  # a request whose cache starts empty
    w = W.build_append("t", 200 + ps, prior, n, Hkv, D, ps, gen=g)
    _check(w)


def test_chunk_append_full_size():
    """B=32 chunks U{64..1024} appended behind prefixes U{512..8192}, Hkv=8,
    D=128, page_size=16: the whole pool bit-exact."""
    w = W.chunk_append(device=cuda())
    _check(w)


def test_decode_step_append():
    """One token per request for B=256 (lengths log-uniform, clamped to 4096)."""
    w = W.decode_append(kv_clamp=(128, 4096), device=cuda())
    _check(w)


def test_append_skips_invalid_entries():
    """Entries whose request, position or page id is out of range write
    nothing; the rest are written as usual."""
    g = torch.Generator().manual_seed(5)
    w = W.build_append("t", 5, [10, 40, 0], [5, 3, 4], 2, 64, 4, gen=g)
    bi, pos = A.batch_indices_positions(w.append_indptr, w.seq_lens)
    bi, pos = bi.clone(), pos.clone()
    bad = {0: (bi[0].item(), -1),                      # negative position
           3: (bi[3].item(), int(w.seq_lens[bi[3]]) + 16),  # past the request's pages
           6: (7, pos[6].item()),                      # no such request
           7: (-1, pos[7].item())}
    for i, (b_, p_) in bad.items():
        bi[i], pos[i] = b_, p_
    idx = w.kv_indices.clone()
    idx[int(w.kv_indptr[2])] = w.num_pages + 5  # request 2's first page id is outside the pool
    w.kv_indices = idx
    _, _, pool = _gpu_append(w, bi, pos)
    keep = [i for i in range(w.nnz) if i not in bad and int(bi[i]) != 2]
    ref = A.append_paged_kv(w.paged_kv, w.append_k[keep], w.append_v[keep], bi[keep], pos[keep],
                            w.kv_indices, w.kv_indptr)
    assert torch.equal(pool.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("batch", [1, 4096, 5000])
def test_batch_indices_positions_many_requests(batch):
    """One request, and thousands of requests (a binary search over
    append_indptr per token), with empty requests: indices and positions
    bit-exact."""
    dev = cuda()
    g = torch.Generator().manual_seed(batch)
    n = torch.randint(0, 4, (batch,), generator=g)
    n[::7] = 0
    if batch == 1:
        n[0] = 3
    indptr = torch.zeros(batch + 1, dtype=torch.int32)
    indptr[1:] = torch.cumsum(n, 0).to(torch.int32)
    seq = (n + torch.randint(0, 50, (batch,), generator=g)).to(torch.int32)
    bi, pos = pka.get_batch_indices_positions(indptr.to(dev), seq.to(dev), int(indptr[-1]))
    rb, rp = A.batch_indices_positions(indptr, seq)
    assert torch.equal(bi.cpu(), rb) and torch.equal(pos.cpu(), rp)


def test_append_nothing():
    g = torch.Generator().manual_seed(6)
    w = W.build_append("t", 6, [5, 9], [0, 0], 1, 128, 16, gen=g)
    bi, pos, pool = _gpu_append(w)
    assert bi.numel() == 0 and torch.equal(pool.view(torch.int16), w.paged_kv.view(torch.int16))
