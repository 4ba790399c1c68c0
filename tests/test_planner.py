"""CPU tests of the host planner and the C ABI (no GPU needed).

* every symbol include/pka.h declares is exported by libpka.so;
* coverage: every visible (request, query head, query row, key) lies in
  exactly one work unit, and no unit reads a key at or past kv_len;
* merge groups and partial rows are consistent;
* the plan is deterministic and its bytes equal a Python re-statement of the
  planning rule (tiling, split choice, ordering, image layout);
* invalid inputs return error codes with a message, never abort.
"""
import ctypes
import os
import random
import re

import pytest
import torch

import bench
import paged_kv_cache_plan_amd as pka
from inputs import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Planner constants (paged_kv_cache_plan_amd/csrc/planner.h).
BLOCK_KEYS, DECODE_TILE, DECODE_MAX_G = 64, 32, 16


def block_rows(D):
    """Packed query rows per prefill block: 32 per wave, 8 waves at D=128, 4 at D=64."""
    return 256 if D == 128 else 128


def wg_per_cu(D):
    return 1 if D == 128 else 2


# At D=64 a batch whose units average at least this many keys times the group
# size is planned for three prefill workgroups per CU (not graph-stable plans
# or mixed sub-plans).
LONG_UNIT_KEYS, WG_PER_CU_LONG64 = 2048, 3
NUM_CUS, NUM_XCDS, QUEUE_WINDOW, QUEUE_TAIL_SLOTS = 256, 8, 2, 2
UNIT_WORDS, REQ_WORDS, MERGE_WORDS = 16, 8, 8


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "pka.h")).read()
    declared = set(re.findall(r"\b(pka_[a-z_]+)\s*\(", header))
    assert declared == set(pka.EXPORTED), declared ^ set(pka.EXPORTED)
    lib = pka.load_library()
    for name in sorted(declared):
        assert hasattr(lib, name), name


# ---------------------------------------------------------------------------
# Python re-statement of the planning rule
# ---------------------------------------------------------------------------

def _cdiv(a, b):
    return -(-a // b)


def restate_plan(qo_indptr, kv_indptr, kv_indices, last, Hq, Hkv, ps, causal, flags, ragged=False, D=128,
                 num_cus=NUM_CUS, qo_begin=None, kv_begin=None, workers=0):
    B = len(qo_indptr) - 1
    G = Hq // Hkv
    qo_len = [qo_indptr[r + 1] - qo_indptr[r] for r in range(B)]
    if ragged:
        kv_len = [kv_indptr[r + 1] - kv_indptr[r] for r in range(B)]
    else:
        kv_len = [0 if kv_indptr[r + 1] == kv_indptr[r] else
                  (kv_indptr[r + 1] - kv_indptr[r] - 1) * ps + last[r] for r in range(B)]
    decode = B > 0 and max(qo_len) <= 1 and G <= DECODE_MAX_G
    blocks = []
    if decode:
        rows_per = G
        for r in range(B):
            if qo_len[r]:
                blocks += [(r, hk, 0, G, kv_len[r]) for hk in range(Hkv)]
    else:
        rows_per = block_rows(D)
        for r in range(B):
            if not qo_len[r]:
                continue
            rows = qo_len[r] * G
            for hk in range(Hkv):
                for r0 in range(0, rows, rows_per):
                    r1 = min(rows, r0 + rows_per)
                    hi = kv_len[r]
                    if causal:
                        hi = max(0, min(hi, (r1 - 1) // G + kv_len[r] - qo_len[r] + 1))
                    blocks.append((r, hk, r0, r1, hi))
    chunk = 0
    if not (flags & pka.PKA_DISABLE_SPLIT_KV) and blocks:
        if decode:
            keys = sum(b[4] for b in blocks)
            chunk = _cdiv(keys, num_cus * 8)
            chunk = min(16384, max(256, _cdiv(chunk, 128) * 128))
        elif len(blocks) < 2 * num_cus:
            tiles = sum(_cdiv(b[4], BLOCK_KEYS) for b in blocks)
            chunk = max(8, _cdiv(tiles, 4 * num_cus)) * BLOCK_KEYS
    units, merge, partial, any_split = [], [], 0, False
    for (r, hk, r0, r1, hi) in blocks:
        n = _cdiv(hi, chunk) if (chunk and hi > chunk) else 1
        nrows = r1 - r0
        base = -1
        if n > 1:
            any_split = True
            base = partial
            partial += n * nrows
            merge.append([r, hk, r0, r1, base, n, 0, 0])
        for s_ in range(n):
            lo = s_ * chunk if n > 1 else 0
            up = min(hi, lo + chunk) if n > 1 else hi
            # words 8-11 repeat the request's row offset, qo_len, KV base and kv_len
            req_words = [qo_indptr[r] if qo_begin is None else qo_begin[r], qo_len[r],
                         kv_begin[r] if (ragged and kv_begin is not None) else kv_indptr[r], kv_len[r]]
            units.append(([r, hk, r0, r1, lo, up, base + s_ * nrows if n > 1 else -1, 0] + req_words + [0] * 4,
                          (up - lo) * nrows + 1, len(units)))
    key = lambda u: (-u[1], u[2])
    fixed = bool(flags & pka.PKA_GRAPH_STABLE)
    wgs = 2 if decode else wg_per_cu(D)
    if (not decode and D == 64 and not fixed and workers <= 0 and qo_begin is None and units
            and sum(u[0][5] - u[0][4] for u in units) * G >= LONG_UNIT_KEYS * len(units)):
        wgs = WG_PER_CU_LONG64
    bounds = [0]  # queue q holds units bounds[q] .. bounds[q + 1]
    if decode or (len(units) <= NUM_XCDS and not fixed):
        units.sort(key=key)
        order = [u[0] for u in units]
        bounds.append(len(order))
    else:
        grps, i = [], 0
        while i < len(units):
            j = i
            while j < len(units) and units[j][0][:2] == units[i][0][:2]:
                j += 1
            grps.append((sum(u[1] for u in units[i:j]), i, j))
            i = j
        gorder = sorted(range(len(grps)), key=lambda g: (-grps[g][0], g))
        queues, load = [[] for _ in range(NUM_XCDS)], [0] * NUM_XCDS
        for g in gorder:
            x = min(range(NUM_XCDS), key=lambda k: (load[k], k))
            load[x] += grps[g][0]
            queues[x].append(units[grps[g][1]:grps[g][2]])
        # windows of QUEUE_WINDOW groups, units longest-first inside a window
        # (ties: group order, then planning order)
        queues = [[u for i in range(0, len(gs), QUEUE_WINDOW)
                   for u in sorted([v for g in gs[i:i + QUEUE_WINDOW] for v in g],
                                   key=lambda v: -v[1])]
                  for gs in queues]
        # the last QUEUE_TAIL_SLOTS units per worker slot of a queue run
        # longest-first across its groups (stable: ties keep queue order)
        tail = QUEUE_TAIL_SLOTS * max(1, num_cus * wgs // NUM_XCDS)
        queues = [q[:max(0, len(q) - tail)] + sorted(q[max(0, len(q) - tail):], key=lambda v: -v[1])
                  for q in queues]
        queues = [[u[0] for u in q] for q in queues]
        order = []
        for q in queues:
            order += q
            bounds.append(len(order))
    nq = len(bounds) - 1
    longest = max(bounds[q + 1] - bounds[q] for q in range(nq))
    # workers > 0: exactly that many, evenly over the queues (a one-grid mixed launch)
    slots = workers if workers > 0 else num_cus * wgs
    per_queue = max(1, slots // nq) if (fixed or workers > 0) else max(1, min(longest, max(1, slots // nq)))
    workers = nq * per_queue
    align = lambda w: _cdiv(w, 64) * 64
    nnz = 0 if ragged else kv_indptr[B]
    off_units = 64
    off_req = off_units + align(len(order) * UNIT_WORDS)
    off_merge = off_req + align(B * REQ_WORDS)
    off_sched = off_merge + align(len(merge) * MERGE_WORDS)
    off_idx = off_sched + align(nq * 64)
    total = off_idx + align(max(nnz, 1))
    img = [0] * total
    part_lse = _cdiv(partial * D * 4, 256) * 256 // 4
    # slices of the largest merge group: whole 256-item blocks of rows * D / 4, at most 32
    max_rows = max((m[3] - m[2] for m in merge), default=0)
    merge_slices = 1 if max_rows == 0 else min(32, _cdiv(max_rows * (D // 4), 256))
    hdr = [0x31414b50, 1 if decode else 0, len(order), len(merge), B, nnz, off_units, off_req,
           off_merge, off_idx, partial, rows_per, chunk if any_split else 0, flags, off_sched, nq, workers,
           part_lse, merge_slices]
    img[:len(hdr)] = hdr
    for q in range(nq):  # counters (words 0, 1) start at zero
        img[off_sched + 64 * q + 32: off_sched + 64 * q + 35] = [bounds[q], bounds[q + 1], per_queue]
    for i, u in enumerate(order):
        img[off_units + UNIT_WORDS * i: off_units + UNIT_WORDS * (i + 1)] = u
    dense = 0
    for r in range(B):
        img[off_req + 8 * r: off_req + 8 * r + 5] = [
            qo_indptr[r] if qo_begin is None else qo_begin[r], qo_len[r],
            kv_begin[r] if (ragged and kv_begin is not None) else kv_indptr[r], kv_len[r], dense]
        dense += kv_len[r]
    for g, m in enumerate(merge):
        img[off_merge + 8 * g: off_merge + 8 * g + 8] = m
    if nnz:
        img[off_idx: off_idx + nnz] = list(kv_indices)
    return img


# Compute-unit split of a mixed batch (planner.h: rates in flop and bytes per
# ns, per compute unit, and the decode total).
PREFILL_FLOP_PER_CU_NS, DECODE_BYTE_PER_CU_NS, DECODE_BYTE_PER_NS = 3500.0, 30.0, 6300.0


def restate_mixed_cus(flop, nbytes, num_cus=NUM_CUS, step=NUM_XCDS):
    best, best_t = step, None
    for p in range(step, num_cus - step + 1, step):
        t = max(flop / (PREFILL_FLOP_PER_CU_NS * p),
                nbytes / min(DECODE_BYTE_PER_NS, DECODE_BYTE_PER_CU_NS * (num_cus - p)))
        if best_t is None or t <= best_t:
            best, best_t = p, t
    return best


def restate_mixed(qo_indptr, kv_indptr, kv_indices, last, Hq, Hkv, ps, causal, flags, ragged=False, D=128):
    """The image of a PKA_MIXED_BATCH plan: a 64-word header, then the
    prefill sub-batch's image, then the decode sub-batch's; each sub-batch is
    planned as an ordinary batch over its own requests (in batch order) with
    the whole batch's row offsets, on its share of the compute units."""
    B = len(qo_indptr) - 1
    qo_len = [qo_indptr[r + 1] - qo_indptr[r] for r in range(B)]
    pre = [r for r in range(B) if qo_len[r] > 1]
    dec = [r for r in range(B) if qo_len[r] == 1]
    plain = flags & ~(pka.PKA_MIXED_BATCH | pka.PKA_MIXED_TWO_LAUNCHES)
    one_grid = not (flags & pka.PKA_MIXED_TWO_LAUNCHES)
    if not pre or not dec or Hq // Hkv > DECODE_MAX_G:
        return restate_plan(qo_indptr, kv_indptr, kv_indices, last, Hq, Hkv, ps, causal, plain, ragged, D)

    def kv_len(r):
        span = kv_indptr[r + 1] - kv_indptr[r]
        return span if ragged else (0 if span == 0 else (span - 1) * ps + last[r])

    def sub(rs, cus, workers=0):
        qi, ki, idx = [0], [0], []
        for r in rs:
            qi.append(qi[-1] + qo_len[r])
            ki.append(ki[-1] + kv_indptr[r + 1] - kv_indptr[r])
            if not ragged:
                idx += kv_indices[kv_indptr[r]:kv_indptr[r + 1]]
        return restate_plan(qi, ki, idx, None if ragged else [last[r] for r in rs], Hq, Hkv, ps, causal, plain,
                            ragged, D, num_cus=cus, qo_begin=[qo_indptr[r] for r in rs],
                            kv_begin=[kv_indptr[r] for r in rs], workers=workers)

    flop = sum(4.0 * D * Hq * bench.visible_pairs([qo_len[r]], [kv_len(r)], causal) for r in pre)
    nbytes = sum(4.0 * Hkv * D * kv_len(r) for r in dec)
    pcus = restate_mixed_cus(flop, nbytes)
    dcus = NUM_CUS - pcus
    if one_grid:
        # one launch: both sides on the whole chip, the decode side with the
        # prefill side's worker count (header word 16); the split only says
        # which workgroup slots of each XCD start with decode
        ip = sub(pre, NUM_CUS, workers=NUM_CUS * wg_per_cu(D))
        idc = sub(dec, NUM_CUS, workers=ip[16])
        first_decode = dcus // NUM_XCDS * wg_per_cu(D)
    else:
        ip, idc = sub(pre, pcus), sub(dec, dcus)
        first_decode = 0
    align = lambda w: _cdiv(w, 64) * 64
    off_d = 64 + align(len(ip))
    partial, part_lse = ip[10], ip[17]
    float_ws_p = max(256, part_lse * 4 + _cdiv(partial * 4, 256) * 256)  # at least 256 bytes
    hdr = [0x4d414b50, 2, 64, off_d, _cdiv(float_ws_p, 256) * 256 // 4, pcus, dcus, B,
           0 if ragged else kv_indptr[B], int(one_grid), first_decode]
    img = hdr + [0] * (64 - len(hdr)) + ip + [0] * (off_d - 64 - len(ip)) + idc
    return img


def _image(w, flags=0, causal=None):
    causal = w.causal if causal is None else causal
    return pka.plan_host_image(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                               w.num_kv_heads, w.head_dim, w.page_size, causal, w.num_pages, flags)


def _unpack(img):
    h = img[:16].tolist()
    n_units, n_merge, B = h[2], h[3], h[4]
    units = img[h[6]: h[6] + UNIT_WORDS * n_units].view(-1, UNIT_WORDS).tolist() if n_units else []
    req = img[h[7]: h[7] + 8 * B].view(-1, 8).tolist() if B else []
    merge = img[h[8]: h[8] + 8 * n_merge].view(-1, 8).tolist() if n_merge else []
    idx = img[h[9]: h[9] + h[5]].tolist()
    return h, units, req, merge, idx


def _random_batch(seed):
    rng = random.Random(seed)
    B = rng.randint(1, 6)
    Hkv = rng.choice([1, 2, 4])
    G = rng.choice([1, 2, 4, 8])
    ps = rng.choice([1, 2, 3, 4, 16, 64])
    decode = rng.random() < 0.3
    qo, kv = [], []
    for _ in range(B):
        k = rng.choice([0, rng.randint(1, 40), rng.randint(40, 3000)])
        q = (1 if rng.random() < 0.9 else 0) if decode else rng.choice([0, rng.randint(1, 70), rng.randint(1, 600)])
        qo.append(q)
        kv.append(k)
    causal = rng.random() < 0.7
    return W.build("rand", seed, qo, kv, Hkv * G, Hkv, 64, ps, causal=causal, pool_slack=0.3,
                   poison=False)


CASES = [("seed", s) for s in range(40)]


@pytest.mark.parametrize("kind,seed", CASES)
@pytest.mark.parametrize("flags", [0, pka.PKA_DISABLE_SPLIT_KV])
def test_coverage_and_restatement(kind, seed, flags):
    w = _random_batch(seed)
    img, info = _image(w, flags)
    img2, _ = _image(w, flags)
    assert torch.equal(img, img2), "planning must be deterministic"
    want = restate_plan(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                        w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size,
                        w.causal, flags, D=w.head_dim)
    assert img.tolist() == want
    h, units, req, merge, idx = _unpack(img)
    assert idx == w.kv_indices.tolist()
    G = w.num_qo_heads // w.num_kv_heads
    covered = {}
    for u in units:
        r, hk, r0, r1, lo, hi, prow = u[:7]
        assert u[8:12] == req[r][:4]  # the request words repeated in the unit
        assert r0 < r1
        assert 0 <= lo <= hi <= w.kv_lens[r]
        for p in range(r0, r1):
            covered.setdefault((r, hk, p), []).append((lo, hi))
    for r in range(w.batch):
        qo, kv = w.qo_lens[r], w.kv_lens[r]
        for hk in range(w.num_kv_heads):
            for p in range(qo * G):
                i = p // G
                vis_hi = kv if not w.causal else max(0, min(kv, i + kv - qo + 1))
                ranges = sorted(covered.get((r, hk, p), []))
                assert ranges, (r, hk, p)
                # disjoint, contiguous from 0, covering every visible key
                pos = 0
                for lo, hi in ranges:
                    assert lo == pos, (r, hk, p, ranges)
                    pos = hi
                assert pos >= vis_hi, (r, hk, p, ranges, vis_hi)
    if flags & pka.PKA_DISABLE_SPLIT_KV:
        assert h[3] == 0 and all(u[6] == -1 for u in units)
    # partial rows: each split group's units write disjoint rows in one block
    seen = set()
    for g in merge:
        r, hk, r0, r1, base, n = g[:6]
        nrows = r1 - r0
        parts = sorted(u[6] for u in units if u[0] == r and u[1] == hk and u[2] == r0 and u[6] >= 0)
        assert parts == [base + s * nrows for s in range(n)]
        rows = set(range(base, base + n * nrows))
        assert not rows & seen
        seen |= rows
    assert info["num_partial_rows"] == len(seen)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("dense_vs_sparse", dict(batch=3, length=300, heads=4)),
    ("gqa_append", dict(batch=5, prefix_range=(10, 900), chunk_range=(1, 200))),
    ("batch_decode", dict(batch=20)),
    ("p5_shape", {}),
])
def test_named_workloads_restatement(name, kw):
    w = W.make(name, **kw)
    img, info = _image(w)
    want = restate_plan(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                        w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size,
                        w.causal, 0, D=w.head_dim)
    assert img.tolist() == want
    a, b = pka.workspace_size(w.qo_indptr, w.kv_indptr, w.kv_last_page_len, w.num_qo_heads,
                              w.num_kv_heads, w.head_dim, w.page_size, w.causal)
    assert a == info["int_ws_bytes"] and b == info["float_ws_bytes"]


@pytest.mark.parametrize("long_units", [True, False])
@pytest.mark.parametrize("flags", [0, pka.PKA_GRAPH_STABLE])
def test_head_dim_64_workgroups_per_cu(long_units, flags):
    """At D=64 a batch of long units (keys per unit times the group size at
    least 2048 on average) is planned for three prefill workgroups per CU, one
    of short units for two; graph-stable plans always for two.  The image
    matches the restatement."""
    if long_units:
        w = W.gqa_append(seed=21, batch=32, prefix_range=(2000, 4000), chunk_range=(64, 300), head_dim=64)
    else:
        w = W.gqa_append(seed=22, batch=32, prefix_range=(40, 400), chunk_range=(64, 300), head_dim=64)
    img, info = _image(w, flags=flags)
    want = restate_plan(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                        w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size,
                        w.causal, flags, D=64)
    assert img.tolist() == want
    three = long_units and not flags
    _, units, _, _, _ = _unpack(img)
    mean_keys = sum(u[5] - u[4] for u in units) / len(units)
    assert (mean_keys * (w.num_qo_heads // w.num_kv_heads) >= LONG_UNIT_KEYS) == long_units
    if flags:
        assert info["num_workers"] == NUM_CUS * 2
    else:
        assert info["num_workers"] <= NUM_CUS * (3 if three else 2)
        if three:
            assert info["num_workers"] > NUM_CUS * 2 or len(units) <= NUM_CUS * 2


def test_ragged_restatement():
    w = W.dense_vs_sparse(batch=3, length=200, heads=2, head_dim=64)
    img, info = pka.plan_host_image(w.qo_indptr, w.kv_token_indptr, None, None, 2, 2, 64, 1, True,
                                    0, pka.PKA_RAGGED_KV)
    want = restate_plan(w.qo_indptr.tolist(), w.kv_token_indptr.tolist(), [], None, 2, 2, 1, True,
                        pka.PKA_RAGGED_KV, ragged=True, D=64)
    assert img.tolist() == want


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("dense_vs_sparse", dict(batch=3, length=300, heads=4)),
    ("gqa_append", dict(batch=5, prefix_range=(10, 900), chunk_range=(1, 200))),
])
def test_prefill_queues(name, kw):
    """Persistent prefill: the queue records partition the unit array, each
    (request, kv head) sits in one queue, counters start at zero and the
    launch size is queues x workers per queue."""
    w = W.make(name, **kw)
    img, info = _image(w)
    h = img[:32].tolist()
    off_sched, nq, workers = h[14], h[15], h[16]
    assert info["kernel"] == pka.PKA_KERNEL_PREFILL
    assert info["num_queues"] == nq >= 1 and info["num_workers"] == workers
    _, units, _, _, _ = _unpack(img)
    recs = [img[off_sched + 64 * q: off_sched + 64 * (q + 1)].tolist() for q in range(nq)]
    assert all(r[0] == 0 and r[1] == 0 for r in recs)
    assert recs[0][32] == 0 and recs[-1][33] == len(units)
    assert all(recs[q][33] == recs[q + 1][32] for q in range(nq - 1))
    per = recs[0][34]
    assert all(r[34] == per for r in recs) and workers == nq * per
    assert per <= max(r[33] - r[32] for r in recs)
    assert workers <= NUM_CUS * wg_per_cu(w.head_dim)
    home = {}
    for q, r in enumerate(recs):
        for u in units[r[32]:r[33]]:
            assert home.setdefault((u[0], u[1]), q) == q


def test_decode_single_queue():
    """Decode: one queue over every unit, longest first; at most two workers per CU."""
    w = W.batch_decode(batch=20)
    img, info = _image(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE
    h = img[:32].tolist()
    off_sched, nq, workers = h[14], h[15], h[16]
    assert nq == 1 and info["num_queues"] == 1
    rec = img[off_sched: off_sched + 64].tolist()
    assert rec[0] == 0 and rec[1] == 0 and rec[32] == 0 and rec[33] == info["num_units"]
    assert workers == rec[34] == min(info["num_units"], 2 * NUM_CUS) == info["num_workers"]


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("gqa_append", dict(batch=3, prefix_range=(10, 90),
                                                                       chunk_range=(1, 20))),
                                     ("batch_decode", dict(batch=5))])
def test_graph_stable_launch_shape(name, kw):
    """With PKA_GRAPH_STABLE the queue count and worker count depend only on
    the kernel kind and head_dim, never on the batch."""
    w = W.make(name, **kw)
    img, info = _image(w, flags=pka.PKA_GRAPH_STABLE)
    want = restate_plan(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                        w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size,
                        w.causal, pka.PKA_GRAPH_STABLE, D=w.head_dim)
    assert img.tolist() == want
    if info["kernel"] == pka.PKA_KERNEL_DECODE:
        assert info["num_queues"] == 1 and info["num_workers"] == 2 * NUM_CUS
    else:
        assert info["num_queues"] == NUM_XCDS and info["num_workers"] == NUM_CUS * wg_per_cu(w.head_dim)


def test_visible_pairs_brute():
    rng = random.Random(3)
    for _ in range(200):
        q, k = rng.randint(0, 30), rng.randint(0, 30)
        for causal in (True, False):
            brute = sum(1 for i in range(q) for j in range(k) if not causal or j <= i + k - q)
            assert bench.visible_pairs([q], [k], causal) == brute


# ---------------------------------------------------------------------------
# Error handling
# ---------------------------------------------------------------------------

def _expect(code, fn):
    with pytest.raises(pka.PkaError) as e:
        fn()
    assert e.value.code == code, str(e.value)
    assert str(e.value)


def test_errors():
    ok = dict(qo_indptr=[0, 3, 5], kv_indptr=[0, 2, 3], kv_indices=[4, 1, 0], kv_last_page_len=[2, 1],
              num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=4, causal=True, num_pages=8)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return pka.plan_host_image(**a)

    call()  # the baseline is valid
    E_ARG, E_UNS = pka.PKA_ERR_INVALID_ARG, pka.PKA_ERR_UNSUPPORTED
    _expect(E_ARG, lambda: call(qo_indptr=[0, 3, 2]))            # decreasing
    _expect(E_ARG, lambda: call(qo_indptr=[1, 3, 5]))            # does not start at 0
    _expect(E_ARG, lambda: call(kv_indptr=[0, 3, 2]))
    _expect(E_ARG, lambda: call(kv_indices=[4, 1, 8]))           # page id out of the pool
    _expect(E_ARG, lambda: call(kv_indices=[4, -1, 0]))
    _expect(E_ARG, lambda: call(kv_last_page_len=[0, 1]))        # a used page holds >= 1 slot
    _expect(E_ARG, lambda: call(kv_last_page_len=[5, 1]))        # > page_size
    _expect(E_ARG, lambda: call(kv_indptr=[0, 2, 2], kv_indices=[4, 1], kv_last_page_len=[2, 3]))  # empty but last != 0
    _expect(E_UNS, lambda: call(num_qo_heads=3))                  # Hq % Hkv
    _expect(E_UNS, lambda: call(head_dim=96))
    _expect(E_UNS, lambda: call(page_size=0))
    _expect(E_UNS, lambda: call(page_size=129))
    _expect(E_ARG, lambda: call(num_kv_heads=0))
    _expect(E_ARG, lambda: call(flags=0x80))
    # nnz_pages mismatch and null arrays through the raw ABI
    L = pka.load_library()
    i32 = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    info = pka.PlanInfo()
    rc = L.pka_plan_host_image(i32([0, 3, 5]), i32([0, 2, 3]), i32([4, 1, 0]), i32([2, 1]), 2, 2, 8, 4, 2, 64,
                               4, 1, 0, None, 0, ctypes.byref(info))
    assert rc == E_ARG and b"nnz" in L.pka_last_error()
    rc = L.pka_plan_host_image(None, i32([0, 2, 3]), i32([4, 1, 0]), i32([2, 1]), 2, 3, 8, 4, 2, 64, 4, 1, 0,
                               None, 0, ctypes.byref(info))
    assert rc == E_ARG
    rc = L.pka_plan_host_image(i32([0, 3, 5]), i32([0, 2, 3]), None, i32([2, 1]), 2, 3, 8, 4, 2, 64, 4, 1, 0,
                               None, 0, ctypes.byref(info))
    assert rc == E_ARG


def test_run_errors_without_a_gpu():
    """run / merge_states / debug_gather reject a bad plan or sizes, and
    pka_plan_create a too-small workspace, before any HIP call."""
    L = pka.load_library()
    E_ARG = pka.PKA_ERR_INVALID_ARG
    assert L.pka_run(None, None, None, None, None, None) == E_ARG
    assert L.pka_run_ragged(None, None, None, None, None, None, None) == E_ARG
    assert L.pka_debug_gather(None, None, None, None, None) == E_ARG
    assert L.pka_merge_states(None, None, 4, 0, 1, 64, None, None, 0, None) == E_ARG
    assert L.pka_merge_states(None, None, 4, 2, 1, 66, None, None, 0, None) == E_ARG
    assert L.pka_merge_states(None, None, 0, 2, 1, 64, None, None, 0, None) == pka.PKA_OK  # nothing to do
    L.pka_plan_destroy(None)  # no-op
    # PKA_ERR_WORKSPACE: the sizes are checked before anything is allocated,
    # uploaded or dereferenced (the workspace pointers below are never used)
    i32 = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    qo, kv, idx, last = [0, 3, 5], [0, 2, 3], [4, 1, 0], [2, 1]
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.pka_plan_workspace_size(i32(qo), i32(kv), i32(last), 2, 4, 2, 64, 4, 1, 0, ctypes.byref(a),
                                     ctypes.byref(b)) == pka.PKA_OK
    assert a.value > 0 and b.value > 0
    fake = ctypes.c_void_p(4096)
    for iw, fw in ((a.value - 4, b.value), (a.value, b.value - 4), (0, 0)):
        h = ctypes.c_void_p()
        rc = L.pka_plan_create(i32(qo), i32(kv), i32(idx), i32(last), 2, 3, 8, 4, 2, 64, 4, 1, 0.0, 0, fake, iw,
                               fake, fw, None, ctypes.byref(h))
        assert rc == pka.PKA_ERR_WORKSPACE, (iw, fw, L.pka_last_error())
        assert b"workspace" in L.pka_last_error() and not h.value
    # after a size query, create still validates the page ids itself
    assert L.pka_plan_workspace_size(i32(qo), i32(kv), i32(last), 2, 4, 2, 64, 4, 1, 0, ctypes.byref(a),
                                     ctypes.byref(b)) == pka.PKA_OK
    h = ctypes.c_void_p()
    rc = L.pka_plan_create(i32(qo), i32(kv), i32([4, 1, 9]), i32(last), 2, 3, 8, 4, 2, 64, 4, 1, 0.0, 0, fake,
                           a.value, fake, b.value, None, ctypes.byref(h))
    assert rc == E_ARG and b"outside" in L.pka_last_error()
    assert L.pka_plan_workspace_size(i32(qo), i32(kv), i32(last), 2, 4, 2, 64, 4, 1, 0, ctypes.byref(a),
                                     ctypes.byref(b)) == pka.PKA_OK
    rc = L.pka_plan_create(i32(qo), i32(kv), i32(idx), i32(last), 2, 2, 8, 4, 2, 64, 4, 1, 0.0, 0, fake,
                           a.value, fake, b.value, None, ctypes.byref(h))
    assert rc == E_ARG and b"nnz" in L.pka_last_error()


def test_empty_batch_and_edge_lengths():
    img, info = pka.plan_host_image([0], [0], [], [], 4, 2, 64, 4, True, 1)
    assert info["num_units"] == 0 and info["total_q"] == 0
    # kv_len 0 and qo_len 0 requests plan without error
    w = W.build("edge", 3, [3, 0, 70, 1], [0, 5, 20, 1], 4, 2, 64, 4, causal=True, pool_slack=0.5)
    _image(w)


# ---------------------------------------------------------------------------
# Mixed prefill + decode batches (PKA_MIXED_BATCH)
# ---------------------------------------------------------------------------

def _mixed_random(seed):
    rng = random.Random(1000 + seed)
    B = rng.randint(2, 12)
    Hkv = rng.choice([1, 2, 8])
    G = rng.choice([1, 4, 8])
    ps = rng.choice([1, 4, 16])
    qo = [rng.choice([0, 1, 1, 1, rng.randint(2, 300)]) for _ in range(B)]
    i, j = rng.sample(range(B), 2)  # at least one request of each kind
    qo[i], qo[j] = rng.randint(2, 300), 1
    kv = [rng.choice([0, rng.randint(1, 50), rng.randint(50, 3000)]) for _ in range(B)]
    kv = [max(k, q) for k, q in zip(kv, qo)]
    return W.build("mixed", seed, qo, kv, Hkv * G, Hkv, rng.choice([64, 128]), ps, causal=rng.random() < 0.8,
                   pool_slack=0.2, poison=False)


MIXED_MODES = [pka.PKA_MIXED_BATCH | pka.PKA_MIXED_TWO_LAUNCHES, pka.PKA_MIXED_BATCH]


@pytest.mark.parametrize("flags", MIXED_MODES, ids=["two_launches", "one_grid"])
@pytest.mark.parametrize("seed", range(16))
def test_mixed_restatement(seed, flags):
    w = _mixed_random(seed)
    img, info = _image(w, flags)
    want = restate_mixed(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                         w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size, w.causal,
                         flags, D=w.head_dim)
    assert img.tolist() == want
    assert info["kernel"] == pka.PKA_KERNEL_MIXED
    if not flags & pka.PKA_MIXED_TWO_LAUNCHES:
        # one launch: every workgroup serves both images, so both have the launch's worker count
        h = img[:64].tolist()
        pre, dec = img[h[2]:h[3]], img[h[3]:]
        assert h[9] == 1 and int(pre[16]) == int(dec[16]) == info["num_workers"] == NUM_CUS * wg_per_cu(w.head_dim)
        assert h[10] == info["decode_cus"] // NUM_XCDS * wg_per_cu(w.head_dim)
    assert info["prefill_cus"] + info["decode_cus"] == NUM_CUS and info["prefill_cus"] % NUM_XCDS == 0
    a, b = pka.workspace_size(w.qo_indptr, w.kv_indptr, w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads,
                              w.head_dim, w.page_size, w.causal, flags)
    assert a == info["int_ws_bytes"] == img.numel() * 4 and b == info["float_ws_bytes"]


@pytest.mark.parametrize("flags", MIXED_MODES, ids=["two_launches", "one_grid"])
@pytest.mark.parametrize("seed", range(16))
def test_mixed_coverage(seed, flags):
    """Both sub-plans together cover every visible (request, head, row, key)
    once: prefill requests only in the prefill image, decode requests only in
    the decode image (each sub-request is mapped back through its row offset)."""
    w = _mixed_random(seed)
    img, _ = _image(w, flags)
    h = img[:64].tolist()
    by_row = {int(w.qo_indptr[r]): r for r in range(w.batch) if w.qo_lens[r] > 0}
    G = w.num_qo_heads // w.num_kv_heads
    covered = {}
    for off, end, kind in ((h[2], h[3], pka.PKA_KERNEL_PREFILL), (h[3], img.numel(), pka.PKA_KERNEL_DECODE)):
        sub = img[off:end]
        sh, units, req, _, _ = _unpack(sub)
        assert sh[0] == 0x31414b50 and sh[1] == kind
        for u in units:
            sr, hk, r0, r1, lo, hi = u[:6]
            r = by_row[req[sr][0]]
            assert (w.qo_lens[r] == 1) == (kind == pka.PKA_KERNEL_DECODE)
            assert req[sr][1] == w.qo_lens[r] and req[sr][3] == w.kv_lens[r]
            for p in range(r0, r1):
                covered.setdefault((r, hk, p), []).append((lo, hi))
    for r in range(w.batch):
        qo, kv = w.qo_lens[r], w.kv_lens[r]
        for hk in range(w.num_kv_heads):
            for p in range(qo * G):
                i = p // G
                vis_hi = kv if not w.causal else max(0, min(kv, i + kv - qo + 1))
                pos = 0
                for lo, hi in sorted(covered.get((r, hk, p), [])):
                    assert lo == pos
                    pos = hi
                assert pos >= vis_hi


def test_mixed_one_kind_plans_as_without_flag():
    for w in (W.gqa_append(batch=3, prefix_range=(10, 90), chunk_range=(2, 20)), W.batch_decode(batch=7)):
        a, ia = _image(w, pka.PKA_MIXED_BATCH)
        b, ib = _image(w, 0)
        # identical but for the flags word of the header
        a[13] = b[13]
        assert torch.equal(a, b) and ia["kernel"] == ib["kernel"]


def test_mixed_named_workload_split():
    """The chunked-prefill serving step: both kinds present, the split follows
    the restated cost model."""
    w = W.mixed_batch(num_decode=24, num_prefill=2, prefix_range=(100, 400), chunk_range=(50, 120))
    img, info = _image(w, pka.PKA_MIXED_BATCH)
    want = restate_mixed(w.qo_indptr.tolist(), w.kv_indptr.tolist(), w.kv_indices.tolist(),
                         w.kv_last_page_len.tolist(), w.num_qo_heads, w.num_kv_heads, w.page_size, w.causal,
                         pka.PKA_MIXED_BATCH, D=w.head_dim)
    assert img.tolist() == want and info["kernel"] == pka.PKA_KERNEL_MIXED


def test_mixed_cu_split_extremes():
    assert restate_mixed_cus(1e12, 0.0) == NUM_CUS - NUM_XCDS        # decode has nothing to do
    # prefill has nothing to do: decode gets the units it can use (its total
    # rate saturates at 6300 / 30 = 210 units), ties go to prefill
    assert restate_mixed_cus(0.0, 1e9) == 40
    p = restate_mixed_cus(4.0e11, 2.6e9)
    assert NUM_XCDS < p < NUM_CUS - NUM_XCDS


def test_mixed_rejects_graph_stable():
    w = W.mixed_batch(num_decode=4, num_prefill=1, prefix_range=(10, 40), chunk_range=(5, 9))
    _expect(pka.PKA_ERR_UNSUPPORTED, lambda: _image(w, pka.PKA_MIXED_BATCH | pka.PKA_GRAPH_STABLE))
    _expect(pka.PKA_ERR_UNSUPPORTED,
            lambda: _image(w, pka.PKA_MIXED_BATCH | pka.PKA_MIXED_TWO_LAUNCHES | pka.PKA_GRAPH_STABLE))


def test_two_launches_needs_the_mixed_flag():
    w = W.mixed_batch(num_decode=4, num_prefill=1, prefix_range=(10, 40), chunk_range=(5, 9))
    _expect(pka.PKA_ERR_INVALID_ARG, lambda: _image(w, pka.PKA_MIXED_TWO_LAUNCHES))
