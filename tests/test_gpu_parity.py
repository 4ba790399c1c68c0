"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that still
span several tiles and ragged tails, plus the edge cases of the method."""
import math

import pytest
import torch

import oracle
import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, cuda, oracle_paged, run_paged, run_ragged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("out_fp32", [False, True])
def test_tiny_causal_paged(out_fp32):
    w = W.tiny()
    o, lse, info = run_paged(w, out_fp32=out_fp32)
    ref_o, ref_l = oracle_paged(w)
    err = compare(o, lse, ref_o, ref_l, "tiny")
    print(f"tiny (out_fp32={out_fp32}): max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)
    assert info["kernel"] == pka.PKA_KERNEL_PREFILL


def test_tiny_non_causal():
    w = W.tiny(causal=False)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), "tiny non-causal")


@pytest.mark.parametrize("ps", [1, 2, 3, 4, 8, 16, 64, 128])
def test_page_sizes(ps):
    w = W.gqa_append(seed=30 + ps, batch=3, prefix_range=(40, 400), chunk_range=(5, 150),
                     page_size=ps)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), f"ps={ps}")


@pytest.mark.parametrize("ps", [1, 2, 3, 16])
def test_page_sizes_d64(ps):
    w = W.gqa_append(seed=50 + ps, batch=3, prefix_range=(40, 400), chunk_range=(5, 150),
                     page_size=ps, head_dim=64)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), f"D=64 ps={ps}")


@pytest.mark.parametrize("ps", [16, 1, 3])
def test_head_dim_64_three_workgroups_per_cu(ps):
    """A D=64 batch of long units (prefixes of 2000-4000 keys) is planned for
    three workgroups per CU and run by the build of the kernel made for
    three; sampled rows (and every request's first and last) against the
    oracle."""
    from tests.gpu_common import sample_rows
    w = W.gqa_append(seed=60 + ps, batch=32, prefix_range=(2000, 4000), chunk_range=(64, 300),
                     page_size=ps, head_dim=64)
    o, lse, info = run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_PREFILL and info["num_workers"] > 2 * 256, info["num_workers"]
    ends = [int(x) for x in w.qo_indptr[:-1]] + [int(x) - 1 for x in w.qo_indptr[1:]]
    rows = sample_rows(w.total_q, 512, 70 + ps, must=ends)
    err = compare(o[rows], lse[rows], *oracle_paged(w, rows=rows), f"D=64 three per CU ps={ps}")
    print(f"D=64 three workgroups per CU, ps={ps}: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)


def test_repeat_runs_of_one_plan():
    """Prefill workgroups take units from queues whose counters reset at the
    end of each launch: every run of one plan must redo the whole batch."""
    w = W.dense_vs_sparse(seed=7, batch=3, length=300, heads=4)
    dev = cuda()
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=w.causal, sm_scale=w.sm_scale,
                    num_pages=w.num_pages, device=dev)
    assert plan.info["num_queues"] > 1
    q, pool = w.q.to(dev), w.paged_kv.to(dev)
    outs = []
    for _ in range(4):
        o = torch.full((w.total_q, w.num_qo_heads, w.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((w.total_q, w.num_qo_heads), float("nan"), dtype=torch.float32, device=dev)
        plan.run(q, pool, o, lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    plan.close()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    compare(outs[0][0].float(), outs[0][1], *oracle_paged(w), "repeat")


def test_dense_vs_vector_sparse_small():
    w = W.dense_vs_sparse(batch=3, length=333, heads=4)
    op, lp, _ = run_paged(w)
    orr, lr, _ = run_ragged(w)
    ref_o, ref_l = oracle.batch_attention_ragged(w.q, w.k, w.v, w.qo_indptr, w.kv_token_indptr,
                                                 True, w.sm_scale)
    compare(op, lp, ref_o, ref_l, "paged ps=1")
    compare(orr, lr, ref_o, ref_l, "ragged")
    # same values, same tiles: the two address policies give identical bits
    assert torch.equal(op, orr) and torch.equal(lp, lr)


def test_gqa_append_small():
    w = W.gqa_append(batch=4, prefix_range=(512, 2048), chunk_range=(64, 300))
    o, lse, info = run_paged(w)
    compare(o, lse, *oracle_paged(w), "append")


def test_long_causal_small():
    w = W.long_causal(batch=1, length=2048)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), "long causal 2048")


def test_p5_shape():
    w = W.p5_shape()
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), "h16 kv1 d128 ps64")


@pytest.mark.parametrize("split", [True, False])
def test_decode_small(split):
    w = W.batch_decode(batch=16, kv_log2_range=(5.0, 12.0), kv_clamp=(1, 4096))
    o, lse, info = run_paged(w, disable_split_kv=not split)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE
    if split:
        assert info["num_merge_groups"] > 0
    else:
        assert info["num_merge_groups"] == 0
    compare(o, lse, *oracle_paged(w), f"decode split={split}")


def test_decode_head_dim_64_and_mha():
    w = W.batch_decode(seed=51, batch=6, kv_log2_range=(3.0, 10.0), kv_clamp=(1, 1024), head_dim=64,
                       heads=8, kv_heads=8, page_size=4)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), "decode D=64 MHA")


@pytest.mark.parametrize("ps,D,Hq,Hkv", [(1, 128, 32, 8), (3, 128, 32, 8), (7, 64, 4, 1), (16, 128, 16, 1),
                                         (64, 128, 8, 2), (128, 64, 8, 8), (2, 64, 16, 16)])
def test_decode_page_sizes_and_groups(ps, D, Hq, Hkv):
    """Decode across the page-id modes (one id per row for page_size < 16
    or not a power of two, two per 32-key step otherwise), group sizes up
    to 16, with and without split KV; KV lengths include 1 and non-multiples
    of the page size."""
    w = W.batch_decode(seed=60 + ps + D, batch=12, kv_log2_range=(0.0, 11.5), kv_clamp=(1, 3000), head_dim=D,
                       heads=Hq, kv_heads=Hkv, page_size=ps)
    for split in (True, False):
        o, lse, info = run_paged(w, disable_split_kv=not split)
        assert info["kernel"] == pka.PKA_KERNEL_DECODE
        compare(o, lse, *oracle_paged(w), f"decode ps={ps} D={D} G={Hq // Hkv} split={split}")


# KV lengths around the decode kernel's step boundaries: 32 keys per step,
# four waves taking steps in turn, steps run in pairs plus an odd last one,
# so these give every wave 0..3 steps, odd and even counts, and partial steps
_STEP_EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 161, 255, 256, 257, 288, 289, 511, 512, 513]


@pytest.mark.parametrize("ps", [1, 3, 4, 16, 32])
def test_decode_step_boundaries(ps):
    """Every K/V load of a decode step is issued unconditionally (keys past
    the unit's end are clamped to its last row and masked), so lengths at and
    around the step and pair boundaries must read no slot past kv_len: the
    unused tails of the last pages are NaN-poisoned."""
    w = W.build(f"dec_edges_ps{ps}", 70 + ps, [1] * len(_STEP_EDGES), _STEP_EDGES, 16, 4, 128, ps, causal=True,
                pool_slack=0.1)
    for split in (True, False):
        o, lse, info = run_paged(w, disable_split_kv=not split)
        assert info["kernel"] == pka.PKA_KERNEL_DECODE
        compare(o, lse, *oracle_paged(w), f"decode step edges ps={ps} split={split}")


def test_decode_step_boundaries_ragged():
    w = W.build("dec_edges_ragged", 79, [1] * len(_STEP_EDGES), _STEP_EDGES, 16, 4, 128, 1, causal=True,
                ragged=True, poison=False)
    o, lse, info = run_ragged(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE
    compare(o, lse, *oracle_paged(w), "decode step edges ragged")


def test_decode_ragged():
    w = W.build("dec_ragged", 61, [1] * 9, [1, 5, 33, 64, 65, 700, 1500, 2, 2049], 16, 4, 128, 1, causal=True,
                ragged=True, poison=False)
    o, lse, info = run_ragged(w)
    assert info["kernel"] == pka.PKA_KERNEL_DECODE
    compare(o, lse, *oracle_paged(w), "decode ragged")


@pytest.mark.parametrize("Hq,Hkv", [(12, 4), (24, 4), (10, 2), (32, 1)])
def test_group_sizes_not_powers_of_two(Hq, Hkv):
    """Packed row = token * G + head in group, so with G = 3, 5 or 6 a wave's
    32 rows start and end mid-token; G = 32 is past the decode kernel's 16
    heads per KV head, and its single-token batches take the prefill kernel."""
    G = Hq // Hkv
    w = W.build(f"grp{G}", 80 + G, [37, 1, 70, 5, 130], [300, 19, 70, 5, 131], Hq, Hkv, 128, 16,
                causal=True, pool_slack=0.1)
    o, lse, info = run_paged(w)
    assert info["kernel"] == pka.PKA_KERNEL_PREFILL
    compare(o, lse, *oracle_paged(w), f"prefill G={G}")
    wd = W.batch_decode(seed=90 + G, batch=10, kv_log2_range=(0.0, 11.0), kv_clamp=(1, 2000), head_dim=128,
                        heads=Hq, kv_heads=Hkv, page_size=16)
    for split in (True, False):
        o, lse, info = run_paged(wd, disable_split_kv=not split)
        assert info["kernel"] == (pka.PKA_KERNEL_DECODE if G <= 16 else pka.PKA_KERNEL_PREFILL)
        compare(o, lse, *oracle_paged(wd), f"decode G={G} split={split}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_non_causal(D):
    w = W.build("nc", 62 + D, [130, 7, 300], [400, 7, 90], 8, 2, D, 16, causal=False, pool_slack=0.2)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), f"non-causal D={D}")


def test_prefill_split_kv():
    # few row blocks -> the planner splits the KV and merges afterwards
    w = W.build("split", 7, [40], [3000], 8, 2, 128, 16, causal=True, pool_slack=0.1)
    o, lse, info = run_paged(w)
    assert info["num_merge_groups"] > 0
    compare(o, lse, *oracle_paged(w), "prefill split")
    o2, l2, info2 = run_paged(w, disable_split_kv=True)
    assert info2["num_merge_groups"] == 0
    compare(o2, l2, *oracle_paged(w), "prefill no split")


def test_edge_cases():
    # kv_len 0, qo_len 0, qo_len > kv_len (top rows see nothing), D=64
    w = W.build("edge", 3, [3, 0, 70, 1], [0, 5, 20, 1], 4, 2, 64, 4, causal=True, pool_slack=0.5)
    o, lse, _ = run_paged(w)
    compare(o, lse, *oracle_paged(w), "edge")


def _growing_keys(w, top=5.0):
    """A copy of w whose K rows are scaled by 1 at key 0 up to `top` at each
    request's last key, so that a row's largest logits come late."""
    pool = w.paged_kv.clone()
    ps = w.page_size
    for r in range(w.batch):
        n = int(w.kv_indptr[r + 1] - w.kv_indptr[r])
        kv = int((n - 1) * ps + w.kv_last_page_len[r]) if n else 0
        for j, pid in enumerate(w.kv_indices[int(w.kv_indptr[r]):int(w.kv_indptr[r + 1])].tolist()):
            pos = torch.arange(j * ps, (j + 1) * ps, dtype=torch.float32)
            f = (1.0 + (top - 1.0) * pos / max(kv, 1)).clamp(max=top)
            pool[pid, 0] = (pool[pid, 0].float() * f[:, None, None]).to(torch.bfloat16)
    w.paged_kv = pool
    return w


@pytest.mark.parametrize("decode", [False, True])
def test_reference_max_moves_late(decode):
    """K rows scaled up along each sequence (x1 to x5), so that a row's max
    logit rises by more than the rescale slack after its first tiles: the
    softmax reference moves, and O and the row sum are rescaled, in the
    middle of a row's keys, not only on its first tile."""
    qo = [1, 1, 1] if decode else [700, 300, 64]
    kv = [2000, 1500, 4096]
    w = _growing_keys(W.build(f"growing_{decode}", 61, qo, kv, 8, 2, 128, 16, causal=True))
    # premise: for the last request, the last tile's max logit (base 2) is
    # more than 8 above the first tile's for most (row, head) pairs
    r = 2
    q = w.q[int(w.qo_indptr[r]):int(w.qo_indptr[r + 1])].double()
    pages = w.kv_indices[int(w.kv_indptr[r]):int(w.kv_indptr[r + 1])]
    k = w.paged_kv[pages, 0].reshape(-1, w.num_kv_heads, w.head_dim)[:kv[r]].double()
    G = w.num_qo_heads // w.num_kv_heads
    s = torch.einsum("qhd,khd->hqk", q, k.repeat_interleave(G, dim=1)) * w.sm_scale / math.log(2.0)
    rise = s[:, :, -64:].amax(-1) - s[:, :, :64].amax(-1)
    assert (rise > 8).float().mean() > 0.5, rise
    for split in (True, False):
        o, lse, info = run_paged(w, disable_split_kv=not split)
        assert info["kernel"] == (pka.PKA_KERNEL_DECODE if decode else pka.PKA_KERNEL_PREFILL)
        err = compare(o, lse, *oracle_paged(w), f"growing keys decode={decode} split={split}")
        print(f"growing keys decode={decode} split={split}: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}",
              flush=True)


@pytest.mark.parametrize("sm_scale", [0.02, 0.5])
@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_explicit_sm_scale(sm_scale, decode, D):
    """sm_scale given by the caller instead of 1/sqrt(D): a nearly flat
    softmax (0.02) and a sharp one (0.5, logits with a standard deviation of
    about 8 base-2 units at D=128)."""
    qo = [1, 1, 1, 1] if decode else [200, 33, 1, 90]
    w = W.build(f"scale_{sm_scale}_{decode}_{D}", 71, qo, [300, 33, 900, 150], 8, 2, D, 16, causal=True)
    w.sm_scale = sm_scale
    o, lse, info = run_paged(w)
    assert info["kernel"] == (pka.PKA_KERNEL_DECODE if decode else pka.PKA_KERNEL_PREFILL)
    err = compare(o, lse, *oracle_paged(w), f"sm_scale={sm_scale} decode={decode} D={D}")
    print(f"sm_scale={sm_scale} decode={decode} D={D}: max |dO| {err[0]:.2e}, max |dlse| {err[1]:.2e}", flush=True)


@pytest.mark.parametrize("ps", [1, 16])
def test_decode_empty_kv(ps):
    """Decode requests with no keys (kv_len 0) next to short ones: (0, -inf)
    rows, and no load of the empty requests' (absent) pages."""
    w = W.build(f"dec_empty_ps{ps}", 80 + ps, [1] * 6, [0, 1, 33, 0, 200, 0], 8, 2, 128, ps, causal=True,
                pool_slack=0.2)
    for split in (True, False):
        o, lse, info = run_paged(w, disable_split_kv=not split)
        assert info["kernel"] == pka.PKA_KERNEL_DECODE
        compare(o, lse, *oracle_paged(w), f"decode empty kv ps={ps} split={split}")


def test_plan_upload_bit_exact():
    w = W.gqa_append(batch=5, prefix_range=(10, 900), chunk_range=(1, 200))
    img, _ = pka.plan_host_image(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len,
                                 w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, True,
                                 w.num_pages)
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=True, num_pages=w.num_pages,
                    device=cuda())
    torch.cuda.synchronize()
    dev_img = plan.int_ws[: img.numel() * 4].cpu().view(torch.int32)
    assert torch.equal(dev_img, img)
    plan.close()


def test_debug_gather_bit_exact():
    w = W.gqa_append(seed=8, batch=4, prefix_range=(10, 300), chunk_range=(1, 50), page_size=16)
    plan = pka.Plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, w.num_qo_heads,
                    w.num_kv_heads, w.head_dim, w.page_size, causal=True, num_pages=w.num_pages,
                    device=cuda())
    k, v = plan.debug_gather(w.paged_kv.to(cuda()))
    torch.cuda.synchronize()
    plan.close()
    ks, vs = [], []
    for r in range(w.batch):
        pages = w.kv_indices[int(w.kv_indptr[r]):int(w.kv_indptr[r + 1])].long()
        ks.append(w.paged_kv[pages, 0].reshape(-1, w.num_kv_heads, w.head_dim)[: w.kv_lens[r]])
        vs.append(w.paged_kv[pages, 1].reshape(-1, w.num_kv_heads, w.head_dim)[: w.kv_lens[r]])
    assert torch.equal(k.cpu().view(torch.int16), torch.cat(ks).view(torch.int16))
    assert torch.equal(v.cpu().view(torch.int16), torch.cat(vs).view(torch.int16))


def test_merge_states_kernel():
    g = torch.Generator().manual_seed(0)
    n, S, H, D = 37, 5, 3, 128
    v = torch.randn(n, S, H, D, generator=g)
    s = torch.randn(n, S, H, generator=g) * 4
    s[0, :, 0] = float("-inf")
    s[3, 1:, 2] = float("-inf")
    ref_v, ref_s = oracle.merge_states(v, s)
    vo, so = pka.merge_states(v.to(cuda()), s.to(cuda()), out_fp32=True)
    torch.cuda.synchronize()
    vo, so = vo.cpu(), so.cpu()
    assert torch.equal(torch.isneginf(so), torch.isneginf(ref_s))
    fin = torch.isfinite(ref_s)
    assert (vo.double() - ref_v).abs().max() < 1e-5
    assert (so.double()[fin] - ref_s[fin]).abs().max() < 1e-5
    vb, _ = pka.merge_states(v.to(cuda()), s.to(cuda()), out_fp32=False)
    assert (vb.float().cpu().double() - ref_v).abs().max() < 2e-2


def test_deterministic():
    w = W.batch_decode(seed=9, batch=8, kv_log2_range=(8.0, 12.0))
    a = run_paged(w)
    b = run_paged(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
