// Appending new K/V rows to a paged KV cache, gfx950.
//
// The append is parallel over appended elements, not over requests
// (FlashInfer 0.2 release blog, "KV-cache append optimisation"): a first
// kernel gives every appended token its request and position
// (get_batch_indices_positions), a second copies each token's rows to the
// page and slot that the attention gather reads them from (flashinfer-trace
// discussion #15, "Notes on fa3_gqa_prefill_v1": the flat page table).
//
// A token's K row of all KV heads (Hkv * D bf16) is contiguous both in the
// appended tensor and in its page slot of paged_kv [num_pages, 2, ps, Hkv, D],
// so a wave moves a token's K and V rows with coalesced 16-byte loads and
// stores.  The copy is bound by HBM bandwidth.
#include "args.h"
#include "device.h"
#include "launch.h"

namespace pka {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void batch_indices_positions_kernel(BatchPosArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < a.nnz; i += stride) {
    // request r: the last r with append_indptr[r] <= i
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.append_indptr[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int first = a.append_indptr[r];
    const int n = a.append_indptr[r + 1] - first;
    a.batch_indices[i] = r;
    a.positions[i] = a.seq_lens[r] - n + static_cast<int>(i - first);
  }
}

// Each wave takes kTPW appended tokens at a time (grid-stride over groups of
// tokens): their requests, positions and page ids are wave-uniform scalar
// loads, all their K/V loads are issued before the stores, and each lane
// moves 16-byte chunks of the tokens' K and V rows.  One token per wave
// measured fastest (more waves in flight beat more loads per wave).
constexpr int kTPW = 1;

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int cpt = a.row_elems / 8;  // 16-byte chunks per token row
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  const int64_t groups = (a.nnz + kTPW - 1) / kTPW;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6); gi < groups;
       gi += waves) {
    const int i0 = __builtin_amdgcn_readfirstlane(static_cast<int>(gi * kTPW));
    int64_t dst[kTPW];  // element offset of each token's K row in the pool, -1: skip
#pragma unroll
    for (int u = 0; u < kTPW; ++u) {
      dst[u] = -1;
      const int i = i0 + u;
      if (i >= a.nnz) continue;
      const int r = a.batch_indices[i];
      const int p = a.positions[i];
      if (r < 0 || r >= a.batch || p < 0) continue;
      const int q = a.page_shift >= 0 ? (p >> a.page_shift) : p / a.page_size;
      const int slot = p - q * a.page_size;
      const int first = a.kv_indptr[r];
      if (q >= a.kv_indptr[r + 1] - first) continue;  // beyond the request's pages
      const int page = a.kv_indices[first + q];
      if (page < 0 || page >= a.num_pages) continue;
      dst[u] = ((static_cast<int64_t>(page) * 2) * a.page_size + slot) * a.row_elems;
    }
    const int64_t v_off = static_cast<int64_t>(a.page_size) * a.row_elems;
    for (int c = lane; c < cpt; c += 64) {
      u32x4 k[kTPW], v[kTPW];
#pragma unroll
      for (int u = 0; u < kTPW; ++u) {
        if (dst[u] < 0) continue;
        const int64_t src = static_cast<int64_t>(i0 + u) * a.row_elems + 8 * c;
        k[u] = ld16(a.append_k + src);
        v[u] = ld16(a.append_v + src);
      }
#pragma unroll
      for (int u = 0; u < kTPW; ++u) {
        if (dst[u] < 0) continue;
        st16(a.paged_kv + dst[u] + 8 * c, k[u]);
        st16(a.paged_kv + dst[u] + v_off + 8 * c, v[u]);
      }
    }
  }
}

int grid_for(int64_t items) {
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  return static_cast<int>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_batch_indices_positions(const BatchPosArgs& a, hipStream_t stream) {
  if (a.nnz <= 0) return hipSuccess;
  batch_indices_positions_kernel<<<grid_for(a.nnz), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.nnz <= 0) return hipSuccess;
  append_kernel<<<grid_for((static_cast<int64_t>(a.nnz) + kTPW - 1) / kTPW * 64), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pka
