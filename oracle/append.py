"""CPU oracle: appending new K/V rows to a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package.  The product
path never does, and this module imports nothing from it.

What is computed, and from which passage of the pages:

* New K/V rows of a batch are written into the paged cache
  (FlashInfer documentation, table of contents, "flashinfer.page: Append new
  K/V tensors to Paged KV-Cache").
* The append is parallelised per appended element rather than per request,
  with a helper that gives every appended token its request and its position
  (FlashInfer 0.2 release blog, "KV-cache append optimisation":
  get_batch_indices_positions).
* Token t of a request lives in page ``kv_indices[kv_indptr[r] + t // ps]``
  at slot ``t % ps`` of ``paged_kv[num_pages, 2, ps, Hkv, D]`` (0 = K,
  1 = V); this is the flat page table of flashinfer-trace discussion #15,
  "Notes on fa3_gqa_prefill_v1", the same rule the attention gather reads
  with.

Readings where the pages are silent (listed in the design notes):

* ``seq_lens[r]`` is the request's KV length *after* the append, and its
  ``n_r = append_indptr[r + 1] - append_indptr[r]`` appended tokens are its
  last n_r tokens: appended token j of request r has position
  ``seq_lens[r] - n_r + j``.
* Rows are copied bit for bit; nothing else in the pool changes.
"""
from __future__ import annotations

import torch


def batch_indices_positions(append_indptr, seq_lens):
    """(batch_indices, positions) int32 ``[nnz]`` for a ragged append batch.

    Appended token i (global, ``append_indptr[r] <= i < append_indptr[r+1]``)
    belongs to request r and lands at position ``seq_lens[r] - n_r + (i -
    append_indptr[r])``.
    """
    indptr = [int(x) for x in append_indptr]
    lens = [int(x) for x in seq_lens]
    nnz = indptr[-1]
    batch = torch.empty(nnz, dtype=torch.int32)
    pos = torch.empty(nnz, dtype=torch.int32)
    for r in range(len(indptr) - 1):
        a, b = indptr[r], indptr[r + 1]
        n = b - a
        for j in range(n):
            batch[a + j] = r
            pos[a + j] = lens[r] - n + j
    return batch, pos


def append_paged_kv(paged_kv: torch.Tensor, append_k: torch.Tensor, append_v: torch.Tensor,
                    batch_indices, positions, kv_indices, kv_indptr) -> torch.Tensor:
    """A copy of ``paged_kv`` with appended token i written at the page and
    slot of position ``positions[i]`` of request ``batch_indices[i]``.

    ``append_k`` / ``append_v`` are ``[nnz, Hkv, D]`` in the pool's dtype.
    """
    out = paged_kv.clone()
    ps = paged_kv.shape[2]
    for i in range(append_k.shape[0]):
        r = int(batch_indices[i])
        p = int(positions[i])
        page = int(kv_indices[int(kv_indptr[r]) + p // ps])
        slot = p % ps
        out[page, 0, slot] = append_k[i]
        out[page, 1, slot] = append_v[i]
    return out
