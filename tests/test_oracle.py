"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent fact: hand-worked values (tests/golden), a pure-Python brute
force, a library routine (torch's scaled_dot_product_attention and
logsumexp), closed forms, invariances fixed by the pages, or the
recursive-attention identity.  ``test_pins_catch_planted_mistakes`` plants
plausible mistakes in the oracle (on the CPU, via monkeypatch) and checks that
at least one pin fails for each.
"""
import math
import os
import random

import pytest
import torch

import oracle
from oracle import attention as A
from inputs import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN2 = math.log(2.0)


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def _tiny_random(seed, B=None, causal=True, ps=None, G=None):
    """A random tiny paged workload (B <= 3, L <= 9, D <= 8, ps in {1,2,3})."""
    rng = random.Random(seed)
    B = B or rng.randint(1, 3)
    ps = ps or rng.choice([1, 2, 3])
    G = G or rng.choice([1, 2])
    Hkv = rng.choice([1, 2])
    D = rng.choice([2, 4, 8])
    qo, kv = [], []
    for _ in range(B):
        k = rng.randint(0, 9)
        q = rng.randint(0, 9) if not causal else rng.randint(0, max(k, 1))
        qo.append(q)
        kv.append(k)
    return W.build("rand", seed, qo, kv, Hkv * G, Hkv, D, ps, causal=causal,
                   pool_slack=0.5, poison=True)


def _oracle_paged(w, rows=None, sm_scale=None):
    return oracle.batch_attention_paged(w.q, w.paged_kv, w.qo_indptr, w.kv_indptr,
                                        w.kv_indices, w.kv_last_page_len, w.causal,
                                        sm_scale if sm_scale is not None else w.sm_scale,
                                        rows=rows)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_golden_page_table():
    g = _read_golden("page_table_ps4.txt")
    ps = int(g["page_size"][0])
    npool = int(g["num_pages"][0])
    indptr = torch.tensor([int(x) for x in g["kv_indptr"]], dtype=torch.int32)
    idx = torch.tensor([int(x) for x in g["kv_indices"]], dtype=torch.int32)
    last = torch.tensor([int(x) for x in g["kv_last_page_len"]], dtype=torch.int32)
    assert oracle.kv_lengths(indptr, last, ps) == [int(x) for x in g["kv_len"]]
    # a pool whose K value at (page, slot) encodes the address
    pool = torch.zeros((npool, 2, ps, 1, 1), dtype=torch.float64)
    for p in range(npool):
        for s in range(ps):
            pool[p, 0, s, 0, 0] = 100 * p + s
            pool[p, 1, s, 0, 0] = -(100 * p + s)
    for r in range(2):
        K, V = oracle.gather_paged_kv(pool, indptr, idx, last, ps, r)
        want = [tuple(int(x) for x in e.split(",")) for e in g[f"request{r}"]]
        assert K[:, 0, 0].tolist() == [100 * p + s for p, s in want]
        assert V[:, 0, 0].tolist() == [-(100 * p + s) for p, s in want]


def pin_golden_attention():
    g = _read_golden("attention_by_hand.txt")
    q = torch.tensor([float(x) for x in g["q"]], dtype=torch.float64).view(2, 1, 2)
    k = torch.tensor([float(x) for x in g["k"]], dtype=torch.float64).view(3, 1, 2)
    v = torch.tensor([float(x) for x in g["v"]], dtype=torch.float64).view(3, 1, 2)
    o, lse = oracle.batch_attention_ragged(q, k, v, [0, 2], [0, 3], causal=True, sm_scale=1.0)
    want_o = torch.tensor([float(x) for x in g["o"]], dtype=torch.float64).view(2, 1, 2)
    want_l = torch.tensor([float(x) for x in g["lse2"]], dtype=torch.float64).view(2, 1)
    assert torch.allclose(o, want_o, atol=1e-13, rtol=0), (o, want_o)
    assert torch.allclose(lse, want_l, atol=1e-13, rtol=0), (lse, want_l)


def pin_golden_merge():
    g = _read_golden("merge_by_hand.txt")
    s = torch.tensor([float(x) for x in g["lse"]], dtype=torch.float64).view(1, 3, 1)
    v = torch.tensor([float(x) for x in g["o"]], dtype=torch.float64).view(1, 3, 1, 2)
    vo, so = oracle.merge_states(v, s)
    want = torch.tensor([float(x) for x in g["o_merged"]], dtype=torch.float64)
    assert torch.allclose(vo[0, 0], want, atol=1e-14, rtol=0), vo
    assert abs(float(so[0, 0]) - float(g["lse_merged"][0])) < 1e-14, so


def brute_force(w, sm_scale=None):
    """Softmax attention straight from the definition with scalar loops,
    math.exp and math.fsum, reading each key through the page table."""
    q = w.q.to(torch.float64).tolist()
    pool = w.paged_kv.to(torch.float64).tolist()
    qo_indptr = w.qo_indptr.tolist()
    kv_indptr = w.kv_indptr.tolist()
    kv_indices = w.kv_indices.tolist()
    last = w.kv_last_page_len.tolist()
    ps = w.page_size
    Hq, Hkv, D = w.num_qo_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = w.sm_scale if sm_scale is None else sm_scale
    o = [[[0.0] * D for _ in range(Hq)] for _ in range(len(q))]
    lse = [[float("-inf")] * Hq for _ in range(len(q))]
    for r in range(w.batch):
        npg = kv_indptr[r + 1] - kv_indptr[r]
        kv_len = 0 if npg == 0 else (npg - 1) * ps + last[r]
        qo_len = qo_indptr[r + 1] - qo_indptr[r]
        for i in range(qo_len):
            row = qo_indptr[r] + i
            for h in range(Hq):
                hk = h // G
                logits, vals = [], []
                for j in range(kv_len):
                    if w.causal and j > i + kv_len - qo_len:
                        continue
                    page = kv_indices[kv_indptr[r] + j // ps]
                    slot = j % ps
                    kk = pool[page][0][slot][hk]
                    logits.append(scale * math.fsum(q[row][h][d] * kk[d] for d in range(D)))
                    vals.append(pool[page][1][slot][hk])
                if not logits:
                    continue
                m = max(logits)
                e = [math.exp(s - m) for s in logits]
                Z = math.fsum(e)
                for d in range(D):
                    o[row][h][d] = math.fsum(a * vv[d] for a, vv in zip(e, vals)) / Z
                lse[row][h] = (m + math.log(Z)) / math.log(2.0)
    n = len(q)
    return (torch.tensor(o, dtype=torch.float64).reshape(n, Hq, D),
            torch.tensor(lse, dtype=torch.float64).reshape(n, Hq))


def _close(a, b, tol):
    fin = torch.isfinite(b)
    assert torch.equal(torch.isfinite(a), fin) and torch.equal(a[~fin], b[~fin]), (a, b)
    err = (a[fin] - b[fin]).abs().max().item() if fin.any() else 0.0
    assert err <= tol, err


def pin_brute_force():
    ws = [W.tiny()] + [_tiny_random(s) for s in range(12)] + \
         [_tiny_random(100 + s, causal=False) for s in range(4)]
    for w in ws:
        o, lse = _oracle_paged(w)
        bo, bl = brute_force(w)
        _close(o, bo, 1e-12)
        _close(lse, bl, 1e-12)


def pin_library_sdpa():
    """torch's scaled_dot_product_attention (fp64, CPU, explicit bottom-right
    boolean mask) and logsumexp, per request, on append-shaped inputs."""
    ws = [W.gqa_append(batch=3, prefix_range=(5, 40), chunk_range=(3, 17), head_dim=32,
                       heads=8, kv_heads=2, page_size=4),
          W.p5_shape(batch=2, max_len=50)]
    for w in ws:
        o, lse = _oracle_paged(w)
        Hq, Hkv = w.num_qo_heads, w.num_kv_heads
        G = Hq // Hkv
        for r in range(w.batch):
            q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
            qo_len, kv_len = q1 - q0, w.kv_lens[r]
            # dense K/V of the request straight from the pool, page by page
            pages = w.kv_indices[int(w.kv_indptr[r]):int(w.kv_indptr[r + 1])].long()
            K = w.paged_kv[pages, 0].reshape(-1, Hkv, w.head_dim)[:kv_len].double()
            V = w.paged_kv[pages, 1].reshape(-1, Hkv, w.head_dim)[:kv_len].double()
            Kq = K.repeat_interleave(G, dim=1).transpose(0, 1)   # [Hq, kv, D]
            Vq = V.repeat_interleave(G, dim=1).transpose(0, 1)
            Q = w.q[q0:q1].double().transpose(0, 1)               # [Hq, qo, D]
            mask = torch.ones(qo_len, kv_len, dtype=torch.bool).tril(diagonal=kv_len - qo_len)
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q, Kq, Vq, attn_mask=mask, scale=w.sm_scale)
            logits = (Q @ Kq.transpose(1, 2)) * w.sm_scale
            logits = logits.masked_fill(~mask, float("-inf"))
            ref_lse = torch.logsumexp(logits, dim=-1) / LN2
            _close(o[q0:q1].transpose(0, 1), ref, 1e-12)
            _close(lse[q0:q1].transpose(0, 1), ref_lse, 1e-12)


def pin_causal_closed_forms():
    w = W.tiny(lens=(13, 21))
    o, lse = _oracle_paged(w)
    G = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        q0 = int(w.qo_indptr[r])
        K, V = oracle.gather_paged_kv(w.paged_kv, w.kv_indptr, w.kv_indices,
                                      w.kv_last_page_len, w.page_size, r)
        for h in range(w.num_qo_heads):
            # qo_len == kv_len: query 0 sees only key 0
            assert torch.equal(o[q0, h], V[0, h // G]), (r, h)
            s00 = w.sm_scale * float((w.q[q0, h].double() * K[0, h // G]).sum())
            assert abs(float(lse[q0, h]) - s00 / LN2) < 1e-12
    # the last row of a causal request sees every key: non-causal result
    wn = W.tiny(lens=(13, 21), causal=False)
    on, ln = _oracle_paged(wn)
    for r in range(w.batch):
        last = int(w.qo_indptr[r + 1]) - 1
        _close(o[last], on[last], 1e-12)
        _close(lse[last], ln[last], 1e-12)


def pin_zero_keys_mean():
    """K = 0: every visible logit is 0, so lse2 = log2(#visible) (to rounding) and o is
    the mean of the visible V rows (a cumulative mean along the diagonal)."""
    w = W.gqa_append(batch=2, prefix_range=(3, 9), chunk_range=(2, 6), head_dim=8,
                     heads=4, kv_heads=2, page_size=3)
    w.paged_kv[:, 0] = torch.where(w.paged_kv[:, 0].isnan(), w.paged_kv[:, 0],
                                   torch.zeros_like(w.paged_kv[:, 0]))
    o, lse = _oracle_paged(w)
    G = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        q0 = int(w.qo_indptr[r])
        qo_len, kv_len = w.qo_lens[r], w.kv_lens[r]
        prefix = kv_len - qo_len
        pages = w.kv_indices[int(w.kv_indptr[r]):int(w.kv_indptr[r + 1])].long()
        V = w.paged_kv[pages, 1].reshape(-1, w.num_kv_heads, w.head_dim)[:kv_len].double()
        csum = V.cumsum(0)
        for i in range(qo_len):
            n_vis = prefix + i + 1
            for h in range(w.num_qo_heads):
                assert abs(float(lse[q0 + i, h]) - math.log2(n_vis)) < 1e-14
                mean = csum[n_vis - 1, h // G] / n_vis
                assert (o[q0 + i, h] - mean).abs().max() < 1e-12


def pin_constant_values_and_single_key():
    w = W.p5_shape(batch=2, max_len=30)
    c = torch.linspace(-2, 2, w.head_dim, dtype=torch.float64).to(torch.bfloat16)
    w.paged_kv[:, 1] = torch.where(w.paged_kv[:, 1].isnan(), w.paged_kv[:, 1],
                                   c.expand_as(w.paged_kv[:, 1]))
    o, _ = _oracle_paged(w)
    assert (o - c.double()).abs().max() < 1e-13
    # one key: o = v and lse2 = s / ln 2
    w1 = W.build("one", 9, [1], [1], 4, 2, 16, 4, causal=True, pool_slack=1.0)
    o1, l1 = _oracle_paged(w1)
    page = int(w1.kv_indices[0])
    for h in range(4):
        kk = w1.paged_kv[page, 0, 0, h // 2].double()
        vv = w1.paged_kv[page, 1, 0, h // 2].double()
        assert torch.equal(o1[0, h], vv)
        s = w1.sm_scale * float((w1.q[0, h].double() * kk).sum())
        assert abs(float(l1[0, h]) - s / LN2) < 1e-12


def pin_gqa_equals_repeated_mha():
    w = W.gqa_append(batch=2, prefix_range=(4, 20), chunk_range=(2, 9), head_dim=16,
                     heads=8, kv_heads=2, page_size=2)
    o, lse = _oracle_paged(w)
    G = w.num_qo_heads // w.num_kv_heads
    pool = w.paged_kv.repeat_interleave(G, dim=3)      # [P, 2, ps, Hq, D]
    om, lm = oracle.batch_attention_paged(w.q, pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                          w.kv_last_page_len, True, w.sm_scale)
    _close(o, om, 0.0)
    _close(lse, lm, 0.0)


def pin_page_size_and_permutation_invariance():
    """page_size sets only the block width of the gather: the same K/V stored
    with page_size 1, 4 or 16 under random permutations, or as dense ragged
    tensors, gives bit-identical fp64 results."""
    base = W.dense_vs_sparse(batch=3, length=37, heads=2, head_dim=16)
    ref = oracle.batch_attention_ragged(base.q, base.k, base.v, base.qo_indptr,
                                        base.kv_token_indptr, True, base.sm_scale)
    for ps, seed in [(1, 11), (4, 12), (16, 13), (5, 14)]:
        g = torch.Generator().manual_seed(seed)
        kv_indptr, kv_indices, last = W.page_table_for(base.kv_lens, ps,
                                                       sum((L + ps - 1) // ps for L in base.kv_lens) + 7, g)
        pool = torch.full((int(kv_indptr[-1]) + 7, 2, ps, 2, 16), float("nan"), dtype=torch.bfloat16)
        for r in range(base.batch):
            t0 = int(base.kv_token_indptr[r])
            for t in range(base.kv_lens[r]):
                p = int(kv_indices[int(kv_indptr[r]) + t // ps])
                pool[p, 0, t % ps] = base.k[t0 + t]
                pool[p, 1, t % ps] = base.v[t0 + t]
        got = oracle.batch_attention_paged(base.q, pool, base.qo_indptr, kv_indptr, kv_indices,
                                           last, True, base.sm_scale)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), ps


def pin_recursive_merge_identity():
    """Merging the states of a partition of the visible keys equals attending
    to all of them, for every split point (empty parts included) and for
    random multi-way splits merged at once and pairwise."""
    rng = random.Random(7)
    w = W.gqa_append(batch=2, prefix_range=(3, 12), chunk_range=(2, 7), head_dim=8,
                     heads=2, kv_heads=1, page_size=2)
    for r in range(w.batch):
        q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        K, V = oracle.gather_paged_kv(w.paged_kv, w.kv_indptr, w.kv_indices,
                                      w.kv_last_page_len, w.page_size, r)
        L = K.shape[0]
        rows = torch.arange(q1 - q0)
        vis = oracle.visibility(q1 - q0, L, True, rows)
        qr = w.q[q0:q1, 0].double()
        full_o, full_l = oracle.attention_state(qr, K[:, 0], V[:, 0], vis, w.sm_scale)
        j = torch.arange(L)
        for m in range(L + 1):
            a = oracle.attention_state(qr, K[:, 0], V[:, 0], vis & (j < m)[None], w.sm_scale)
            b = oracle.attention_state(qr, K[:, 0], V[:, 0], vis & (j >= m)[None], w.sm_scale)
            vo, so = oracle.merge_states(torch.stack([a[0], b[0]], 1)[:, :, None],
                                         torch.stack([a[1], b[1]], 1)[:, :, None])
            _close(vo[:, 0], full_o, 1e-12)
            _close(so[:, 0], full_l, 1e-12)
        for _ in range(5):
            cuts = sorted(rng.sample(range(L + 1), min(3, L + 1)))
            bounds = [0] + cuts + [L]
            parts = [oracle.attention_state(qr, K[:, 0], V[:, 0],
                                            vis & ((j >= lo) & (j < hi))[None], w.sm_scale)
                     for lo, hi in zip(bounds[:-1], bounds[1:])]
            vo, so = oracle.merge_states(torch.stack([p[0] for p in parts], 1)[:, :, None],
                                         torch.stack([p[1] for p in parts], 1)[:, :, None])
            _close(vo[:, 0], full_o, 1e-12)
            _close(so[:, 0], full_l, 1e-12)
            acc = parts[0]
            for p in parts[1:]:
                mo, ml = oracle.merge_states(torch.stack([acc[0], p[0]], 1)[:, :, None],
                                             torch.stack([acc[1], p[1]], 1)[:, :, None])
                acc = (mo[:, 0], ml[:, 0])
            _close(acc[0], full_o, 1e-12)
            _close(acc[1], full_l, 1e-12)


def pin_sampled_rows():
    """batch_attention(rows=R) returns exactly the rows R of the whole-batch
    result, in R's order, for paged and ragged sources: R is unsorted, spans
    several requests, repeats a row, and includes rows that see no key (a
    qo_len > kv_len request and a kv_len 0 request) next to a qo_len 0
    request."""
    #          qo  kv
    # req 0:    5   9    rows 0..4
    # req 1:    0   4    (no rows)
    # req 2:    6   3    rows 5..10; rows 5..7 see no key (qo > kv)
    # req 3:    4   0    rows 11..14; no key at all
    # req 4:    3   7    rows 15..17
    w = W.build("rows", 11, [5, 0, 6, 4, 3], [9, 4, 3, 0, 7], 4, 2, 8, 3, causal=True, pool_slack=0.5,
                ragged=True)
    R = [16, 12, 0, 7, 5, 14, 3, 10, 9, 1, 13, 6, 3, 17, 2]
    for src in ("paged", "ragged"):
        if src == "paged":
            run = lambda rows: _oracle_paged(w, rows=rows)
        else:
            run = lambda rows: oracle.batch_attention_ragged(w.q, w.k, w.v, w.qo_indptr, w.kv_token_indptr,
                                                             True, w.sm_scale, rows=rows)
        full_o, full_l = run(None)
        o, l = run(R)
        assert torch.equal(o, full_o[R]) and torch.equal(l, full_l[R]), src
        assert torch.isneginf(full_l[5:8]).all() and torch.isneginf(full_l[11:15]).all()
        assert torch.isfinite(full_l[8:11]).all() and torch.isfinite(full_l[15:18]).all()
    # one row alone, as the sampled full-size checks pick them
    for r in (0, 9, 17):
        o, l = _oracle_paged(w, rows=[r])
        full_o, full_l = _oracle_paged(w)
        assert torch.equal(o[0], full_o[r]) and torch.equal(l[0], full_l[r])


PINS = [pin_golden_page_table, pin_golden_attention, pin_golden_merge, pin_brute_force,
        pin_library_sdpa, pin_causal_closed_forms, pin_zero_keys_mean,
        pin_constant_values_and_single_key, pin_gqa_equals_repeated_mha,
        pin_page_size_and_permutation_invariance, pin_recursive_merge_identity, pin_sampled_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_outputs_free_of_poison():
    w = W.tiny()
    assert w.paged_kv.isnan().any()
    o, lse = _oracle_paged(w)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_empty_and_fully_masked_rows():
    # kv_len = 0 request, qo_len = 0 request, and causal qo_len > kv_len rows
    w = W.build("edge", 3, [3, 0, 4], [0, 5, 2], 2, 1, 8, 2, causal=True, pool_slack=0.5)
    o, lse = _oracle_paged(w)
    assert torch.equal(o[0:3], torch.zeros_like(o[0:3]))
    assert torch.isneginf(lse[0:3]).all()
    # request 2: qo 4, kv 2 -> rows 0, 1 see nothing; rows 2, 3 see 1 and 2 keys
    assert torch.isneginf(lse[3:5]).all() and torch.isfinite(lse[5:7]).all()


def test_merge_properties():
    g = torch.Generator().manual_seed(0)
    v = torch.randn(5, 4, 3, 8, generator=g, dtype=torch.float64)
    s = torch.randn(5, 4, 3, generator=g, dtype=torch.float64) * 3
    s[0, :, 0] = float("-inf")
    s[1, 2, 1] = float("-inf")
    vo, so = oracle.merge_states(v, s)
    perm = torch.tensor([2, 0, 3, 1])
    vp, sp = oracle.merge_states(v[:, perm], s[:, perm])
    _close(vo, vp, 1e-13)
    _close(so, sp, 1e-13)
    assert torch.equal(vo[0, 0], torch.zeros(8, dtype=torch.float64))
    assert torch.isneginf(so[0, 0])
    v1, s1 = oracle.merge_states(v[:, :1], s[:, :1])
    fin = torch.isfinite(s[:, 0])
    assert (v1[fin] - v[:, 0][fin]).abs().max() < 1e-13
    assert torch.equal(s1[fin], s[:, 0][fin])


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------

def _wrong_kv_head(h, group):
    return h % max(1, group)


def _wrong_visibility_top_left(qo_len, kv_len, causal, rows):
    j = torch.arange(kv_len)
    if not causal:
        return torch.ones((rows.numel(), kv_len), dtype=torch.bool)
    return j[None, :] <= rows[:, None]


def _wrong_visibility_strict(qo_len, kv_len, causal, rows):
    j = torch.arange(kv_len)
    if not causal:
        return torch.ones((rows.numel(), kv_len), dtype=torch.bool)
    return j[None, :] < (rows[:, None] + (kv_len - qo_len))


def _wrong_token_location(t, page_size):
    return t % page_size, t // page_size


def _wrong_kv_len(npages, last_page_len, page_size):
    return npages * page_size if npages else 0


def _wrong_merge_natural(v, s):
    # weights e^(s - M) instead of 2^(s - M)
    vo, so = _ORIG_MERGE(v, s * math.log2(math.e))
    return vo, so / math.log2(math.e)


_ORIG_MERGE = A.merge_states


def _attention_state_natural_lse(q_rows, K, V, vis, sm_scale):
    o, lse2 = _ORIG_STATE(q_rows, K, V, vis, sm_scale)
    return o, lse2 * LN2


def _attention_state_no_scale(q_rows, K, V, vis, sm_scale):
    return _ORIG_STATE(q_rows, K, V, vis, 1.0)


def _attention_state_transposed_v(q_rows, K, V, vis, sm_scale):
    o, lse = _ORIG_STATE(q_rows, K, V, vis, sm_scale)
    return o.flip(-1), lse


def _batch_attention_global_local(q, qo_indptr, kv_source, num_kv_heads, causal, sm_scale=None, rows=None):
    """batch_attention with one planted slip: a selected row's local index
    is taken as its global row number (local = sel[pick], not sel[pick] - q0)."""
    total_q, Hq, D = q.shape
    G = Hq // num_kv_heads
    scale = (1.0 / math.sqrt(D)) if (sm_scale is None or sm_scale <= 0) else float(sm_scale)
    sel = torch.arange(total_q) if rows is None else torch.as_tensor(rows, dtype=torch.long)
    o_out = torch.zeros((sel.numel(), Hq, D), dtype=torch.float64)
    lse_out = torch.full((sel.numel(), Hq), float("-inf"), dtype=torch.float64)
    for r in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        pick = ((sel >= q0) & (sel < q1)).nonzero().flatten()
        if pick.numel() == 0:
            continue
        local = sel[pick]
        K, V = kv_source(r)
        vis = A.visibility(q1 - q0, K.shape[0], causal, local)
        for h in range(Hq):
            hk = A.kv_head_of(h, G)
            o, lse = A.attention_state(q[q0 + local.clamp(max=q1 - q0 - 1), h].to(torch.float64),
                                       K[:, hk], V[:, hk], vis, scale)
            o_out[pick, h] = o
            lse_out[pick, h] = lse
    return o_out, lse_out


def _batch_attention_sorted_rows(q, qo_indptr, kv_source, num_kv_heads, causal, sm_scale=None, rows=None):
    """batch_attention with the sampled rows returned in sorted order, not in
    the order asked for (a slip only the sampled-row path can make)."""
    rows = None if rows is None else sorted(int(r) for r in rows)
    return _ORIG_BATCH(q, qo_indptr, kv_source, num_kv_heads, causal, sm_scale, rows)


_ORIG_BATCH = A.batch_attention


_ORIG_STATE = A.attention_state

MISTAKES = {
    "gqa_head_modulo": ("kv_head_of", _wrong_kv_head),
    "causal_top_left": ("visibility", _wrong_visibility_top_left),
    "causal_off_by_one": ("visibility", _wrong_visibility_strict),
    "page_slot_swapped": ("token_location", _wrong_token_location),
    "kv_len_ignores_last_page": ("kv_len_of", _wrong_kv_len),
    "merge_natural_base": ("merge_states", _wrong_merge_natural),
    "lse_natural_log": ("attention_state", _attention_state_natural_lse),
    "sm_scale_dropped": ("attention_state", _attention_state_no_scale),
    "value_dim_reversed": ("attention_state", _attention_state_transposed_v),
    "sampled_rows_global_index": ("batch_attention", _batch_attention_global_local),
    "sampled_rows_sorted": ("batch_attention", _batch_attention_sorted_rows),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, bad = MISTAKES[name]
    monkeypatch.setattr(A, attr, bad)
    monkeypatch.setattr(oracle, attr, bad, raising=False)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
        except Exception:  # a planted mistake may also break shapes
            failed.append(pin.__name__)
    assert failed, f"no pin caught planted mistake {name}"
