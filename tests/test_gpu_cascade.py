"""Cascade attention (pka.Cascade over pka_cascade_create / pka_cascade_run:
one plan per level, the levels' states merged on the GPU) against the oracle
run on the concatenation of each request's keys, level 0 first, with the
bottom-right causal mask over the whole length -- the recursive-attention
identity says the two agree."""
import pytest
import torch

import oracle
import paged_kv_cache_plan_amd as pka
from tests.gpu_common import compare, cuda

pytestmark = pytest.mark.gpu


def _pages(n_tokens, ps, free):
    n = (n_tokens + ps - 1) // ps
    ids, free[:] = free[:n], free[n:]
    last = 0 if n_tokens == 0 else n_tokens - (n - 1) * ps
    return ids, last


def _build(seed, groups_per_level, level_lens, qo_lens, ps=16, Hq=8, Hkv=2, D=128):
    """groups_per_level[l]: list of request-index lists (contiguous, covering
    all requests); level_lens[l][g]: key count of group g at level l (the last
    level has one group per request)."""
    g = torch.Generator().manual_seed(seed)
    B = len(qo_lens)
    total_tokens = sum(sum(x) for x in level_lens)
    num_pages = sum((t + ps - 1) // ps for lens in level_lens for t in lens) + 8
    free = torch.randperm(num_pages, generator=g).tolist()
    pool = torch.randn((num_pages, 2, ps, Hkv, D), generator=g).to(torch.bfloat16)
    qo_indptr_req = [0]
    for n in qo_lens:
        qo_indptr_req.append(qo_indptr_req[-1] + n)
    total_q = qo_indptr_req[-1]
    q = torch.randn((total_q, Hq, D), generator=g).to(torch.bfloat16)
    levels, level_tables = [], []
    for groups, lens in zip(groups_per_level, level_lens):
        qo = [0]
        kvp, kvi, last = [0], [], []
        for members, n_tok in zip(groups, lens):
            qo.append(qo_indptr_req[members[-1] + 1])
            ids, l_ = _pages(n_tok, ps, free)
            kvi += ids
            kvp.append(len(kvi))
            last.append(l_)
        t = (torch.tensor(qo, dtype=torch.int32), torch.tensor(kvp, dtype=torch.int32),
             torch.tensor(kvi, dtype=torch.int32), torch.tensor(last, dtype=torch.int32))
        levels.append(t)
        level_tables.append((groups, t))
    return pool, q, levels, level_tables, torch.tensor(qo_indptr_req, dtype=torch.int32), num_pages, (Hq, Hkv, D, ps)


def _oracle(pool, q, level_tables, qo_indptr, causal, ps):
    def kv_source(r):
        Ks, Vs = [], []
        for groups, (qo, kvp, kvi, last) in level_tables:
            gi = next(i for i, m in enumerate(groups) if r in m)
            K, V = oracle.gather_paged_kv(pool, kvp, kvi, last, ps, gi)
            Ks.append(K)
            Vs.append(V)
        return torch.cat(Ks), torch.cat(Vs)
    return oracle.batch_attention(q, qo_indptr, kv_source, pool.shape[3], causal)


@pytest.mark.parametrize("qo", ["prefill", "decode"])
def test_two_level_shared_prefix(qo):
    B = 5
    qo_lens = [1] * B if qo == "decode" else [37, 1, 90, 64, 5]
    own = [70, 3, 130, 64, 18]
    own = [max(o, n) for o, n in zip(own, qo_lens)]
    groups = [[list(range(B))], [[r] for r in range(B)]]
    pool, q, levels, tables, qo_indptr, num_pages, (Hq, Hkv, D, ps) = _build(1, groups, [[300], own], qo_lens)
    dev = cuda()
    c = pka.Cascade(levels, Hq, Hkv, D, ps, causal=True, num_pages=num_pages, device=dev)
    o, lse = c.run(q.to(dev), pool.to(dev))
    torch.cuda.synchronize()
    c.close()
    compare(o.float().cpu(), lse.cpu(), *_oracle(pool, q, tables, qo_indptr, True, ps), f"cascade-2 {qo}")


def test_three_levels_uneven_pages():
    """Level 0 shared by all, level 1 by two groups, level 2 per request;
    key counts not multiples of the page size at every level."""
    B = 4
    qo_lens = [20, 33, 7, 50]
    groups = [[[0, 1, 2, 3]], [[0, 1], [2, 3]], [[0], [1], [2], [3]]]
    lens = [[45], [19, 100], [20, 40, 9, 77]]
    pool, q, levels, tables, qo_indptr, num_pages, (Hq, Hkv, D, ps) = _build(2, groups, lens, qo_lens)
    dev = cuda()
    c = pka.Cascade(levels, Hq, Hkv, D, ps, causal=True, num_pages=num_pages, out_fp32=True, device=dev)
    o, lse = c.run(q.to(dev), pool.to(dev))
    torch.cuda.synchronize()
    c.close()
    compare(o.cpu(), lse.cpu(), *_oracle(pool, q, tables, qo_indptr, True, ps), "cascade-3")


def test_merge_states_levels():
    g = torch.Generator().manual_seed(3)
    S, n, H, D = 3, 41, 4, 64
    v = torch.randn((S, n, H, D), generator=g)
    s = torch.randn((S, n, H), generator=g) * 4
    s[1, 5] = float("-inf")
    s[:, 7, 2] = float("-inf")
    dev = cuda()
    vo, so = pka.merge_states_levels(v.to(dev), s.to(dev), out_fp32=True)
    ro, rs = oracle.merge_states(v.permute(1, 0, 2, 3).double(), s.permute(1, 0, 2).double())
    compare(vo.cpu(), so.cpu(), ro, rs, "merge levels")


def test_shared_prefix_decode_full_size():
    """The benchmarked shared-prefix decode (64 requests over one 16384-token
    prefix plus their own 128..1024-token suffixes, Hq=32, Hkv=8, D=128,
    page_size=16), drawn on the GPU as bench.py draws it: the two-level
    cascade and the flat decode plan both match the oracle on every row."""
    from inputs import workloads as W
    from tests.gpu_common import oracle_paged, run_paged
    dev = cuda()
    w = W.shared_prefix_decode(device=dev)
    c = pka.Cascade(w.notes["levels"], w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, causal=True,
                    sm_scale=w.sm_scale, num_pages=w.num_pages, device=dev)
    o, lse = c.run(w.q, w.paged_kv)
    torch.cuda.synchronize()
    c.close()
    fo, fl, info = run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE
    w.q, w.paged_kv = w.q.cpu(), w.paged_kv.cpu()
    ref_o, ref_l = oracle_paged(w)
    compare(o.float().cpu(), lse.cpu(), ref_o, ref_l, "shared-prefix cascade")
    compare(fo, fl, ref_o, ref_l, "shared-prefix flat")


@pytest.mark.parametrize("qo", ["prefill", "decode"])
def test_cascade_head_dim_64_group_3(qo):
    """Two levels at D=64, three query heads per KV head, page_size 3: the
    shared level's key count and every request's own keys end mid-page."""
    B = 4
    qo_lens = [1] * B if qo == "decode" else [9, 1, 40, 17]
    own = [max(o, n) for o, n in zip([22, 5, 61, 17], qo_lens)]
    groups = [[list(range(B))], [[r] for r in range(B)]]
    pool, q, levels, tables, qo_indptr, num_pages, (Hq, Hkv, D, ps) = _build(
        3, groups, [[100], own], qo_lens, ps=3, Hq=6, Hkv=2, D=64)
    dev = cuda()
    c = pka.Cascade(levels, Hq, Hkv, D, ps, causal=True, num_pages=num_pages, device=dev)
    o, lse = c.run(q.to(dev), pool.to(dev))
    torch.cuda.synchronize()
    c.close()
    compare(o.float().cpu(), lse.cpu(), *_oracle(pool, q, tables, qo_indptr, True, ps), f"cascade D=64 G=3 {qo}")


def _random_cascade(seed):
    g = torch.Generator().manual_seed(4000 + seed)
    pick = lambda xs: xs[int(torch.randint(0, len(xs), (1,), generator=g))]
    B = int(torch.randint(2, 7, (1,), generator=g))
    decode = seed % 3 == 0
    qo_lens = [1] * B if decode else [int(torch.randint(1, 60, (1,), generator=g)) for _ in range(B)]
    causal = bool(torch.rand(1, generator=g) < 0.7)
    groups = [[list(range(B))]]
    lens = [[int(torch.randint(0, 400, (1,), generator=g))]]
    if torch.rand(1, generator=g) < 0.5:  # a middle level over contiguous groups of requests
        cuts = sorted(set(int(c) for c in torch.randint(1, B, (int(torch.randint(0, 3, (1,), generator=g)),),
                                                        generator=g).tolist()))
        bounds = [0] + cuts + [B]
        groups.append([list(range(a, b)) for a, b in zip(bounds, bounds[1:])])
        lens.append([int(torch.randint(0, 150, (1,), generator=g)) for _ in groups[-1]])
    if seed % 4 == 2:  # an empty shared level
        lens[0][0] = 0
    if len(lens) > 1 and seed % 5 == 1:  # an empty group in the middle level
        lens[1][0] = 0
    groups.append([[r] for r in range(B)])
    own = [int(torch.randint(0, 200, (1,), generator=g)) for _ in range(B)]
    if causal:  # the last level holds at least each request's query rows
        own = [max(o, n) for o, n in zip(own, qo_lens)]
    lens.append(own)
    shape = dict(ps=pick([1, 3, 16]), Hq=0, Hkv=pick([1, 2]), D=pick([64, 128]))
    shape["Hq"] = shape["Hkv"] * pick([1, 3, 4])
    return groups, lens, qo_lens, causal, shape, bool(torch.rand(1, generator=g) < 0.3)


@pytest.mark.parametrize("seed", range(12))
def test_random_cascade(seed):
    """Seeded random cascades: two or three levels, random group splits,
    empty levels, decode or prefill rows, causal or not, page sizes 1, 3
    and 16, D=64 and 128, bf16 or fp32 output."""
    groups, lens, qo_lens, causal, shape, fp32 = _random_cascade(seed)
    print(f"case {seed}: groups={groups} lens={lens} qo={qo_lens} causal={causal} {shape} fp32={fp32}", flush=True)
    pool, q, levels, tables, qo_indptr, num_pages, (Hq, Hkv, D, ps) = _build(50 + seed, groups, lens, qo_lens,
                                                                             **shape)
    dev = cuda()
    c = pka.Cascade(levels, Hq, Hkv, D, ps, causal=causal, num_pages=num_pages, out_fp32=fp32, device=dev)
    o, lse = c.run(q.to(dev), pool.to(dev))
    torch.cuda.synchronize()
    c.close()
    compare(o.float().cpu(), lse.cpu(), *_oracle(pool, q, tables, qo_indptr, causal, ps), f"random cascade {seed}")
