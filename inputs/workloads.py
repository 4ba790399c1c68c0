"""Seeded synthetic inputs for batch attention over a paged KV cache.

This module only *builds inputs*: request lengths, a flat page table, a
page pool and query rows.  It holds none of the attention arithmetic, and it
is the one module that both the CPU oracle's tests and the GPU path's tests
and benchmark draw their inputs from.

Layouts (FlashInfer 0.2 release blog, "flexible block sparsity and vector
sparsity"; flashinfer-trace discussion #15, "Notes on fa3_gqa_prefill_v1"):

* ``q``        bf16 ``[total_q, Hq, D]``, ragged by ``qo_indptr[B+1]``;
* ``paged_kv`` bf16 ``[num_pages, 2, page_size, Hkv, D]`` (NHD; index 0 = K,
  1 = V);
* flat page table ``kv_indptr[B+1]`` (offsets into ``kv_indices``),
  ``kv_indices[nnz]`` (page ids), ``kv_last_page_len[B]`` (valid slots in each
  request's last page);
* ragged dense K/V ``k, v`` bf16 ``[total_kv, Hkv, D]`` with token offsets
  ``kv_token_indptr[B+1]`` (only built where the workload asks for it).

Every random draw is seeded, in a fixed order: lengths -> page permutation ->
Q -> K/V -> poison.  Lengths and page permutations always come from
``torch.Generator('cpu').manual_seed(seed)``.  Q and K/V values are fp32
N(0, 1) rounded to bf16, drawn on ``device``: with the default ``device='cpu'``
they continue the same CPU generator; with a GPU device they come from
``torch.Generator(device).manual_seed(seed)`` on that device (multi-GB pools
would take minutes on the host).  Large tensors are drawn in fixed-size chunks
so that memory stays bounded; the chunk size is part of the recipe.

Unused pool pages and the slots past ``kv_last_page_len`` in each last page are
filled with NaN ("poison") wherever the workload enables it: a kernel that reads
a slot it must not read turns its output into NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

# Fixed chunk (elements) for drawing large normal tensors; part of the recipe.
_DRAW_CHUNK = 1 << 24


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    causal: bool
    sm_scale: float
    qo_lens: list
    kv_lens: list
    qo_indptr: torch.Tensor          # int32 [B+1]
    kv_indptr: torch.Tensor          # int32 [B+1] (pages)
    kv_indices: torch.Tensor         # int32 [nnz]
    kv_last_page_len: torch.Tensor   # int32 [B]
    num_pages: int
    q: torch.Tensor                  # bf16 [total_q, Hq, D]
    paged_kv: torch.Tensor           # bf16 [num_pages, 2, ps, Hkv, D]
    k: Optional[torch.Tensor] = None  # bf16 [total_kv, Hkv, D] (ragged dense)
    v: Optional[torch.Tensor] = None
    kv_token_indptr: Optional[torch.Tensor] = None  # int32 [B+1]
    poisoned: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def nnz_pages(self) -> int:
        return int(self.kv_indptr[-1])


def _randn_bf16(shape, gen) -> torch.Tensor:
    """fp32 N(0,1) draws rounded to bf16, drawn in fixed-size chunks on the
    generator's device."""
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=torch.bfloat16, device=gen.device)
    pos = 0
    while pos < n:
        m = min(_DRAW_CHUNK, n - pos)
        out[pos:pos + m] = torch.randn(m, generator=gen, dtype=torch.float32,
                                       device=gen.device).to(torch.bfloat16)
        pos += m
    return out.view(*shape)


def page_table_for(kv_lens, page_size, num_pages, gen):
    """Build a flat page table for the given KV lengths.

    Pages are assigned in request order from one random permutation of the
    pool: ``perm[:nnz]`` in order, so request r owns
    ``kv_indices[kv_indptr[r]:kv_indptr[r+1]]``.
    Returns (kv_indptr, kv_indices, kv_last_page_len).
    """
    npages = [(L + page_size - 1) // page_size for L in kv_lens]
    last = [0 if L == 0 else L - (n - 1) * page_size for L, n in zip(kv_lens, npages)]
    indptr = [0]
    for n in npages:
        indptr.append(indptr[-1] + n)
    nnz = indptr[-1]
    assert nnz <= num_pages
    perm = torch.randperm(num_pages, generator=gen)
    kv_indices = perm[:nnz].to(torch.int32).contiguous()
    return (torch.tensor(indptr, dtype=torch.int32), kv_indices,
            torch.tensor(last, dtype=torch.int32))


def _poison(paged_kv, kv_indptr, kv_indices, kv_last_page_len, page_size):
    """NaN-fill every pool slot the page table does not reference."""
    num_pages = paged_kv.shape[0]
    used = torch.zeros(num_pages, dtype=torch.bool, device=paged_kv.device)
    used[kv_indices.long().to(paged_kv.device)] = True
    paged_kv[~used] = float("nan")
    B = kv_last_page_len.numel()
    for r in range(B):
        a, b = int(kv_indptr[r]), int(kv_indptr[r + 1])
        if b > a:
            last_page = int(kv_indices[b - 1])
            n = int(kv_last_page_len[r])
            if n < page_size:
                paged_kv[last_page, :, n:] = float("nan")


def build(name, seed, qo_lens, kv_lens, num_qo_heads, num_kv_heads, head_dim,
          page_size, causal=True, pool_slack=0.0, poison=True, ragged=False,
          gen=None, notes=None, num_pages=None, device="cpu") -> Workload:
    """Assemble a workload from explicit lengths.

    Draw order after the lengths: page permutation -> Q -> K/V -> poison.
    With ``ragged=True`` the K/V values are drawn once as dense ragged
    ``k, v`` tensors and scattered into the pool through the page table, so
    the dense and the paged form hold identical values.
    """
    gen = gen if gen is not None else torch.Generator("cpu").manual_seed(seed)
    B = len(qo_lens)
    assert len(kv_lens) == B
    ps = page_size
    nnz = sum((L + ps - 1) // ps for L in kv_lens)
    if num_pages is None:
        num_pages = max(1, nnz + int(math.ceil(nnz * pool_slack)))
    num_pages = max(num_pages, nnz, 1)
    kv_indptr, kv_indices, last = page_table_for(kv_lens, ps, num_pages, gen)
    qo_indptr = torch.tensor([0] + list(torch.tensor(qo_lens).cumsum(0).tolist()),
                             dtype=torch.int32)
    total_q = int(qo_indptr[-1])
    H, Hk, D = num_qo_heads, num_kv_heads, head_dim
    dev = torch.device(device)
    vgen = gen if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    q = _randn_bf16((total_q, H, D), vgen)
    k = v = kv_tok = None
    if ragged:
        total_kv = sum(kv_lens)
        kv_tok = torch.tensor([0] + list(torch.tensor(kv_lens).cumsum(0).tolist()),
                              dtype=torch.int32)
        k = _randn_bf16((total_kv, Hk, D), vgen)
        v = _randn_bf16((total_kv, Hk, D), vgen)
        paged_kv = torch.zeros((num_pages, 2, ps, Hk, D), dtype=torch.bfloat16, device=dev)
        for r in range(B):
            t0, L = int(kv_tok[r]), kv_lens[r]
            t = torch.arange(L)
            page = kv_indices[int(kv_indptr[r]) + t // ps].long().to(dev)
            slot = (t % ps).to(dev)
            paged_kv[page, 0, slot] = k[t0:t0 + L]
            paged_kv[page, 1, slot] = v[t0:t0 + L]
    else:
        paged_kv = _randn_bf16((num_pages, 2, ps, Hk, D), vgen)
    if poison:
        _poison(paged_kv, kv_indptr, kv_indices, last, ps)
    return Workload(
        name=name, seed=seed, batch=B, num_qo_heads=H, num_kv_heads=Hk,
        head_dim=D, page_size=ps, causal=causal, sm_scale=1.0 / math.sqrt(D),
        qo_lens=list(qo_lens), kv_lens=list(kv_lens), qo_indptr=qo_indptr,
        kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
        num_pages=num_pages, q=q, paged_kv=paged_kv, k=k, v=v,
        kv_token_indptr=kv_tok, poisoned=poison, notes=dict(notes or {}))


def _uniform_int(gen, lo, hi, n):
    """n draws from U{lo..hi} (inclusive)."""
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


# ---------------------------------------------------------------------------
# The named workloads.  Each takes optional size overrides so that tests can
# run the same recipe at a size the CPU oracle finishes in seconds.
# ---------------------------------------------------------------------------

def tiny(seed=1, lens=(17, 33), page_size=4, causal=True, pool_pages=64, **kw) -> Workload:
    """Causal paged prefill, B=2 with qo_len = kv_len in {17, 33}, Hq=4, Hkv=1,
    D=64, page_size=4, 64-page pool, partially filled last pages, poisoned."""
    lens = list(lens)
    return build("tiny", seed, lens, lens, 4, 1, 64, page_size, causal=causal,
                 num_pages=pool_pages, **kw)


def dense_vs_sparse(seed=2, batch=16, length=1024, heads=32, head_dim=128, **kw) -> Workload:
    """B requests of L tokens, Hq = Hkv, causal; dense ragged K/V scattered into
    a page_size=1 pool through a random permutation (vector sparsity)."""
    lens = [length] * batch
    return build("dense_vs_sparse", seed, lens, lens, heads, heads, head_dim, 1,
                 causal=True, ragged=True, poison=kw.pop("poison", False), **kw)


def gqa_append(seed=3, batch=32, prefix_range=(512, 8192), chunk_range=(64, 1024),
               **kw) -> Workload:
    """Chunked prefill with a prefix: prefix P ~ U{...}, chunk n ~ U{...},
    qo_len = n, kv_len = P + n, Hq=32, Hkv=8, D=128, page_size=16, pool with
    10% slack, causal mask offset by the prefix."""
    gen = torch.Generator("cpu").manual_seed(seed)
    P = _uniform_int(gen, prefix_range[0], prefix_range[1], batch)
    n = _uniform_int(gen, chunk_range[0], chunk_range[1], batch)
    return build("gqa_append", seed, n, [a + b for a, b in zip(P, n)],
                 kw.pop("heads", 32), kw.pop("kv_heads", 8), kw.pop("head_dim", 128),
                 kw.pop("page_size", 16), causal=True, pool_slack=0.10, gen=gen,
                 notes={"prefix": P}, **kw)


def long_causal(seed=4, batch=2, length=16384, **kw) -> Workload:
    """B=2 requests of L=16384, Hq=32, Hkv=8, D=128, page_size=16, permuted
    pages with 10% slack."""
    lens = [length] * batch
    return build("long_causal", seed, lens, lens, kw.pop("heads", 32),
                 kw.pop("kv_heads", 8), kw.pop("head_dim", 128),
                 kw.pop("page_size", 16), causal=True, pool_slack=0.10,
                 poison=kw.pop("poison", True), **kw)


def batch_decode(seed=5, batch=256, kv_log2_range=(7.0, 15.0), kv_clamp=(128, 32768),
                 **kw) -> Workload:
    """B single-token queries, Hq=32, Hkv=8, D=128, page_size=16; kv_len =
    clamp(round(2^U(a, b)), lo, hi) (log-uniform), permuted pages, 2% slack."""
    gen = torch.Generator("cpu").manual_seed(seed)
    a, b = kv_log2_range
    u = torch.rand(batch, generator=gen, dtype=torch.float64) * (b - a) + a
    kv = [int(min(max(round(2.0 ** float(x)), kv_clamp[0]), kv_clamp[1])) for x in u]
    return build("batch_decode", seed, [1] * batch, kv, kw.pop("heads", 32),
                 kw.pop("kv_heads", 8), kw.pop("head_dim", 128),
                 kw.pop("page_size", 16), causal=kw.pop("causal", True),
                 pool_slack=0.02, gen=gen, poison=kw.pop("poison", True), **kw)


def mixed_batch(seed=9, num_prefill=4, num_decode=192, prefix_range=(1024, 8192),
                chunk_range=(512, 2048), kv_log2_range=(7.0, 14.0), kv_clamp=(128, 16384),
                **kw) -> Workload:
    """One step of chunked-prefill serving: num_prefill prefill chunks (prefix
    P ~ U{...} cached, chunk n ~ U{...} appended: qo_len = n, kv_len = P + n)
    and num_decode single-token requests (kv_len = clamp(round(2^U(a, b)))),
    in a seeded random order; Hq=32, Hkv=8, D=128, page_size=16, causal,
    permuted pages with 5% slack."""
    gen = torch.Generator("cpu").manual_seed(seed)
    P = _uniform_int(gen, prefix_range[0], prefix_range[1], num_prefill)
    n = _uniform_int(gen, chunk_range[0], chunk_range[1], num_prefill)
    a, b = kv_log2_range
    u = torch.rand(num_decode, generator=gen, dtype=torch.float64) * (b - a) + a
    kv_d = [int(min(max(round(2.0 ** float(x)), kv_clamp[0]), kv_clamp[1])) for x in u]
    order = torch.randperm(num_prefill + num_decode, generator=gen).tolist()
    reqs = [(n[i], P[i] + n[i]) for i in range(num_prefill)] + [(1, k) for k in kv_d]
    qo = [reqs[i][0] for i in order]
    kv = [reqs[i][1] for i in order]
    return build("mixed_batch", seed, qo, kv, kw.pop("heads", 32), kw.pop("kv_heads", 8),
                 kw.pop("head_dim", 128), kw.pop("page_size", 16), causal=True, pool_slack=0.05,
                 gen=gen, notes={"num_prefill": num_prefill, "num_decode": num_decode}, **kw)


def p5_shape(seed=6, batch=4, max_len=700, **kw) -> Workload:
    """Hq=16, Hkv=1, D=128, page_size=64, causal prefill with qo = kv ~ U{1..700}
    (the shape named gqa_paged_prefill_causal_h16_kv1_d128_ps64)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lens = _uniform_int(gen, 1, max_len, batch)
    return build("p5_shape", seed, lens, lens, 16, 1, 128, 64, causal=True,
                 pool_slack=0.25, gen=gen, **kw)


def shared_prefix_decode(seed=10, batch=64, prefix=16384, suffix_range=(128, 1024), heads=32, kv_heads=8,
                         head_dim=128, page_size=16, device="cpu") -> Workload:
    """Batch decode over one long shared prefix (cascade inference): every
    request's keys are the same `prefix` tokens (a multiple of page_size)
    followed by its own suffix of S_r ~ U{...} tokens, one query token each.

    The flat page table lists the prefix pages in every request.
    ``notes["levels"]`` holds the same keys in two-level cascade form: level 0
    is one group of all requests over the prefix pages, level 1 one group per
    request over its suffix pages.  Draw order: suffix lengths -> page
    permutation -> Q -> pool.  Unused slots of the last suffix pages are
    poisoned."""
    ps = page_size
    if prefix % ps:
        raise ValueError("prefix must be a multiple of page_size")
    gen = torch.Generator("cpu").manual_seed(seed)
    suf = _uniform_int(gen, suffix_range[0], suffix_range[1], batch)
    n_pre = prefix // ps
    n_suf = [(s + ps - 1) // ps for s in suf]
    num_pages = n_pre + sum(n_suf)
    perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
    pre_ids = perm[:n_pre]
    suf_ids, pos = [], n_pre
    for n in n_suf:
        suf_ids.append(perm[pos:pos + n])
        pos += n
    last = torch.tensor([s - (n - 1) * ps for s, n in zip(suf, n_suf)], dtype=torch.int32)
    kv_indices = torch.cat([torch.cat([pre_ids, ids]) for ids in suf_ids])
    kv_indptr = torch.tensor([0] + list(torch.tensor([n_pre + n for n in n_suf]).cumsum(0).tolist()),
                             dtype=torch.int32)
    qo_indptr = torch.arange(batch + 1, dtype=torch.int32)
    dev = torch.device(device)
    vgen = gen if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    q = _randn_bf16((batch, heads, head_dim), vgen)
    paged_kv = _randn_bf16((num_pages, 2, ps, kv_heads, head_dim), vgen)
    kv_lens = [prefix + s for s in suf]
    _poison(paged_kv, kv_indptr, kv_indices, last, ps)
    levels = [
        (torch.tensor([0, batch], dtype=torch.int32), torch.tensor([0, n_pre], dtype=torch.int32), pre_ids.clone(),
         torch.tensor([ps], dtype=torch.int32)),
        (qo_indptr.clone(), torch.tensor([0] + list(torch.tensor(n_suf).cumsum(0).tolist()), dtype=torch.int32),
         torch.cat(suf_ids), last.clone()),
    ]
    return Workload(
        name="shared_prefix_decode", seed=seed, batch=batch, num_qo_heads=heads, num_kv_heads=kv_heads,
        head_dim=head_dim, page_size=ps, causal=True, sm_scale=1.0 / math.sqrt(head_dim),
        qo_lens=[1] * batch, kv_lens=kv_lens, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
        kv_indices=kv_indices, kv_last_page_len=last, num_pages=num_pages, q=q, paged_kv=paged_kv,
        poisoned=True, notes={"levels": levels, "prefix": prefix, "suffixes": suf})


WORKLOADS = {
    "tiny": tiny,
    "dense_vs_sparse": dense_vs_sparse,
    "gqa_append": gqa_append,
    "long_causal": long_causal,
    "batch_decode": batch_decode,
    "p5_shape": p5_shape,
    "mixed_batch": mixed_batch,
    "shared_prefix_decode": shared_prefix_decode,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)


# ---------------------------------------------------------------------------
# Appending K/V rows to the paged cache.
# ---------------------------------------------------------------------------

@dataclass
class AppendWorkload:
    name: str
    seed: int
    batch: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    prior_lens: list       # KV length of each request before the append
    append_lens: list      # tokens appended to each request
    append_indptr: torch.Tensor   # int32 [B+1]
    seq_lens: torch.Tensor        # int32 [B], lengths after the append
    kv_indptr: torch.Tensor       # int32 [B+1], page table for seq_lens
    kv_indices: torch.Tensor
    kv_last_page_len: torch.Tensor
    num_pages: int
    paged_kv: torch.Tensor        # bf16 [num_pages, 2, ps, Hkv, D], the cache before the append
    append_k: torch.Tensor        # bf16 [nnz, Hkv, D]
    append_v: torch.Tensor

    @property
    def nnz(self):
        return int(self.append_indptr[-1])


def build_append(name, seed, prior_lens, append_lens, num_kv_heads, head_dim, page_size,
                 pool_slack=0.1, gen=None, device="cpu") -> AppendWorkload:
    """Draw order after the lengths: page permutation -> pool -> appended K -> V."""
    gen = gen if gen is not None else torch.Generator("cpu").manual_seed(seed)
    B = len(prior_lens)
    seq = [a + b for a, b in zip(prior_lens, append_lens)]
    ps = page_size
    nnz_pages = sum((L + ps - 1) // ps for L in seq)
    num_pages = max(1, nnz_pages + int(math.ceil(nnz_pages * pool_slack)))
    kv_indptr, kv_indices, last = page_table_for(seq, ps, num_pages, gen)
    app = torch.tensor([0] + list(torch.tensor(append_lens, dtype=torch.int64).cumsum(0).tolist()),
                       dtype=torch.int32)
    dev = torch.device(device)
    vgen = gen if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    pool = _randn_bf16((num_pages, 2, ps, num_kv_heads, head_dim), vgen)
    nnz = int(app[-1])
    k = _randn_bf16((nnz, num_kv_heads, head_dim), vgen)
    v = _randn_bf16((nnz, num_kv_heads, head_dim), vgen)
    return AppendWorkload(name=name, seed=seed, batch=B, num_kv_heads=num_kv_heads, head_dim=head_dim,
                          page_size=ps, prior_lens=list(prior_lens), append_lens=list(append_lens),
                          append_indptr=app, seq_lens=torch.tensor(seq, dtype=torch.int32),
                          kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                          num_pages=num_pages, paged_kv=pool, append_k=k, append_v=v)


def chunk_append(seed=7, batch=32, prefix_range=(512, 8192), chunk_range=(64, 1024), num_kv_heads=8,
                 head_dim=128, page_size=16, **kw) -> AppendWorkload:
    """The append in front of the GQA append-prefill: B=32 requests with a
    prefix ~U{512..8192} already cached append a chunk ~U{64..1024} of
    tokens, Hkv=8, D=128, page_size=16, 10% pool slack."""
    gen = torch.Generator("cpu").manual_seed(seed)
    P = _uniform_int(gen, prefix_range[0], prefix_range[1], batch)
    n = _uniform_int(gen, chunk_range[0], chunk_range[1], batch)
    return build_append("chunk_append", seed, P, n, num_kv_heads, head_dim, page_size, gen=gen, **kw)


def decode_append(seed=8, batch=256, kv_log2_range=(7.0, 15.0), kv_clamp=(128, 32768), num_kv_heads=8,
                  head_dim=128, page_size=16, **kw) -> AppendWorkload:
    """One decode step's append: every request of the batch-decode shape
    appends one token (lengths log-uniform, clamped)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    u = torch.rand(batch, generator=gen, dtype=torch.float64)
    lo, hi = kv_log2_range
    L = [int(min(kv_clamp[1], max(kv_clamp[0], round(2.0 ** (lo + (hi - lo) * float(x)))))) for x in u]
    return build_append("decode_append", seed, [x - 1 for x in L], [1] * batch, num_kv_heads, head_dim,
                        page_size, gen=gen, **kw)
