"""CPU fp64 oracle: batch attention over a paged (or ragged dense) KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package.  The product
path (the HIP library and its Python binding) never does, and this package
imports nothing from it.

What is computed, and from which passage of the pages:

* PageAttention is block-sparse attention whose block width is page_size;
  page_size = 1 is per-token (vector) sparsity.  The page table only changes
  *which* KV rows a request reads, never the arithmetic (FlashInfer 0.2
  release blog, "flexible block sparsity and vector sparsity").  So the oracle
  gathers each request's K/V rows through the page table and then runs plain
  softmax attention on them.
* The flat page table is ``kv_indptr`` / ``kv_indices`` / ``kv_last_page_len``
  and Q is ragged ``[total_q, num_qo_heads, head_dim]`` (flashinfer-trace
  discussion #15, "Notes on fa3_gqa_prefill_v1").
* The log-sum-exp is base 2 (same passage: natural-log LSE is converted to
  base 2 to match the FlashInfer convention).
* Attention states (o, lse) of disjoint KV parts merge into the state of the
  whole (FlashInfer documentation, tutorial "Attention States and Recursive
  Attention"; API "flashinfer.cascade - Merge Attention States").

Readings where the pages are silent (each listed in the design notes):

* GQA: query head h reads KV head h // (Hq / Hkv).
* Causal alignment is bottom-right: query i of a request with qo_len queries
  and kv_len keys sees key j iff j <= i + kv_len - qo_len.  This is the
  "causal mask offset by the prefix length" of chunked prefill; it equals
  top-left alignment when qo_len == kv_len.
* kv_len = (npages - 1) * page_size + last_page_len, and 0 when npages == 0.
* A row that sees no key has o = 0 and lse = -inf.
* lse is log2 of the sum of exp over the *scaled* logits sm_scale * q.k, so
  that states merge with the same sm_scale; sm_scale defaults to 1/sqrt(D).

Everything runs in float64 on the exact input values (bf16 inputs upcast).
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import torch

LN2 = math.log(2.0)
NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# Page table (flashinfer-trace discussion #15, "Notes on fa3_gqa_prefill_v1":
# the flat layout kv_indices + kv_indptr + kv_last_page_len).
# ---------------------------------------------------------------------------

def kv_len_of(npages: int, last_page_len: int, page_size: int) -> int:
    """Tokens held by a request that owns ``npages`` pages: every page but the
    last is full, the last holds ``last_page_len`` slots."""
    if npages == 0:
        return 0
    return (npages - 1) * page_size + last_page_len


def kv_lengths(kv_indptr, kv_last_page_len, page_size: int) -> list:
    B = len(kv_indptr) - 1
    return [kv_len_of(int(kv_indptr[r + 1]) - int(kv_indptr[r]),
                      int(kv_last_page_len[r]), page_size) for r in range(B)]


def token_location(t: torch.Tensor, page_size: int):
    """Token t of a request sits in the request's page number t // page_size,
    at slot t % page_size of that page."""
    return t // page_size, t % page_size


def gather_paged_kv(paged_kv: torch.Tensor, kv_indptr, kv_indices, kv_last_page_len,
                    page_size: int, r: int):
    """Dense K, V ``[kv_len, Hkv, D]`` (float64) of request r.

    ``paged_kv`` is ``[num_pages, 2, page_size, Hkv, D]``, index 0 = K and
    1 = V.  Token t is ``paged_kv[kv_indices[kv_indptr[r] + t // ps], :, t % ps]``.
    Slots past kv_len are never read.
    """
    first = int(kv_indptr[r])
    npages = int(kv_indptr[r + 1]) - first
    L = kv_len_of(npages, int(kv_last_page_len[r]), page_size)
    t = torch.arange(L)
    page_no, slot = token_location(t, page_size)
    pages = kv_indices[first + page_no].long()
    K = paged_kv[pages, 0, slot].to(torch.float64)
    V = paged_kv[pages, 1, slot].to(torch.float64)
    return K, V


def gather_ragged_kv(k: torch.Tensor, v: torch.Tensor, kv_indptr, r: int):
    """Dense K, V of request r from ragged ``[total_kv, Hkv, D]`` tensors whose
    request r spans token rows ``kv_indptr[r] .. kv_indptr[r+1]``."""
    a, b = int(kv_indptr[r]), int(kv_indptr[r + 1])
    return k[a:b].to(torch.float64), v[a:b].to(torch.float64)


# ---------------------------------------------------------------------------
# Attention of one query head over one request's keys.
# ---------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """GQA: query heads are grouped contiguously, ``group`` per KV head."""
    return h // group


def visibility(qo_len: int, kv_len: int, causal: bool, rows: torch.Tensor) -> torch.Tensor:
    """bool ``[len(rows), kv_len]``: may query row i (local index) see key j?

    Keys past kv_len do not exist.  With ``causal`` the mask is aligned
    bottom-right: i sees j iff j <= i + kv_len - qo_len.
    """
    j = torch.arange(kv_len)
    if not causal:
        return torch.ones((rows.numel(), kv_len), dtype=torch.bool)
    return j[None, :] <= (rows[:, None] + (kv_len - qo_len))


def attention_state(q_rows: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                    vis: torch.Tensor, sm_scale: float):
    """Softmax attention state of query rows over keys.

    q_rows ``[n, D]``, K and V ``[m, D]`` (float64), vis bool ``[n, m]``.
    Returns (o ``[n, D]``, lse2 ``[n]``) with

        s_j  = sm_scale * q . K_j                  over visible j
        o    = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s)
        lse2 = log2 sum_j exp(s_j)

    and (0, -inf) for a row with no visible key.
    """
    n, D = q_rows.shape
    if K.shape[0] == 0:
        return (torch.zeros((n, V.shape[-1]), dtype=torch.float64),
                torch.full((n,), NEG_INF, dtype=torch.float64))
    s = sm_scale * (q_rows @ K.T)
    s = torch.where(vis, s, torch.full_like(s, NEG_INF))
    m = s.max(dim=1).values
    seen = vis.any(dim=1)
    m_safe = torch.where(seen, m, torch.zeros_like(m))
    p = torch.exp(s - m_safe[:, None])
    l = p.sum(dim=1)
    l_safe = torch.where(seen, l, torch.ones_like(l))
    o = (p @ V) / l_safe[:, None]
    o = torch.where(seen[:, None], o, torch.zeros_like(o))
    lse2 = torch.where(seen, (m_safe + torch.log(l_safe)) / LN2,
                       torch.full_like(m, NEG_INF))
    return o, lse2


def batch_attention(q: torch.Tensor, qo_indptr, kv_source: Callable[[int], tuple],
                    num_kv_heads: int, causal: bool, sm_scale: Optional[float] = None,
                    rows: Optional[Sequence[int]] = None):
    """Attention for every request of a ragged batch.

    q ``[total_q, Hq, D]``; request r owns query rows
    ``qo_indptr[r] .. qo_indptr[r+1]``; ``kv_source(r)`` returns its dense
    ``(K, V)`` ``[kv_len, Hkv, D]``.  With ``rows`` (global query rows) only
    those rows are computed, in the given order.  Returns float64
    (o ``[n, Hq, D]``, lse2 ``[n, Hq]``).
    """
    total_q, Hq, D = q.shape
    G = Hq // num_kv_heads
    scale = (1.0 / math.sqrt(D)) if (sm_scale is None or sm_scale <= 0) else float(sm_scale)
    sel = torch.arange(total_q) if rows is None else torch.as_tensor(rows, dtype=torch.long)
    o_out = torch.zeros((sel.numel(), Hq, D), dtype=torch.float64)
    lse_out = torch.full((sel.numel(), Hq), NEG_INF, dtype=torch.float64)
    B = len(qo_indptr) - 1
    for r in range(B):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        pick = ((sel >= q0) & (sel < q1)).nonzero().flatten()
        if pick.numel() == 0:
            continue
        local = sel[pick] - q0
        K, V = kv_source(r)
        vis = visibility(q1 - q0, K.shape[0], causal, local)
        for h in range(Hq):
            hk = kv_head_of(h, G)
            o, lse = attention_state(q[q0 + local, h].to(torch.float64),
                                     K[:, hk], V[:, hk], vis, scale)
            o_out[pick, h] = o
            lse_out[pick, h] = lse
    return o_out, lse_out


def batch_attention_paged(q, paged_kv, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                          causal: bool, sm_scale: Optional[float] = None, rows=None):
    """``batch_attention`` with K/V read through the flat page table."""
    ps = paged_kv.shape[2]
    Hkv = paged_kv.shape[3]
    return batch_attention(
        q, qo_indptr,
        lambda r: gather_paged_kv(paged_kv, kv_indptr, kv_indices, kv_last_page_len, ps, r),
        Hkv, causal, sm_scale, rows)


def batch_attention_ragged(q, k, v, qo_indptr, kv_indptr, causal: bool,
                           sm_scale: Optional[float] = None, rows=None):
    """``batch_attention`` with K/V from ragged dense tensors."""
    return batch_attention(q, qo_indptr, lambda r: gather_ragged_kv(k, v, kv_indptr, r),
                           k.shape[1], causal, sm_scale, rows)


# ---------------------------------------------------------------------------
# Merging attention states (FlashInfer documentation, "Attention States and
# Recursive Attention" and "flashinfer.cascade - Merge Attention States").
# ---------------------------------------------------------------------------

def merge_states(v: torch.Tensor, s: torch.Tensor):
    """Merge S attention states per (row, head).

    v ``[n, S, H, D]``, s ``[n, S, H]`` (base-2 LSE).  With M = max_s s_s and
    w_s = 2^(s_s - M):  lse = M + log2 sum_s w_s,  o = sum_s w_s o_s / sum_s w_s.
    A state with lse = -inf has weight 0; if all are empty the result is
    (0, -inf).  Returns float64 (v ``[n, H, D]``, s ``[n, H]``).
    """
    v = v.to(torch.float64)
    s = s.to(torch.float64)
    M = s.max(dim=1).values
    empty = torch.isneginf(M)
    M_safe = torch.where(empty, torch.zeros_like(M), M)
    w = torch.exp2(s - M_safe[:, None])
    W = w.sum(dim=1)
    contrib = torch.where(w[..., None] > 0, w[..., None] * v, torch.zeros_like(v))
    W_safe = torch.where(empty, torch.ones_like(W), W)
    v_out = contrib.sum(dim=1) / W_safe[..., None]
    v_out = torch.where(empty[..., None], torch.zeros_like(v_out), v_out)
    s_out = torch.where(empty, torch.full_like(M, NEG_INF), M_safe + torch.log2(W_safe))
    return v_out, s_out
