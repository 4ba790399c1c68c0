// Merging attention states (FlashInfer documentation, "Attention States and
// Recursive Attention" and "flashinfer.cascade - Merge Attention States"; the
// base-2 LSE of flashinfer-trace discussion #15, "Notes on fa3_gqa_prefill_v1").
//
// For states (o_s, lse_s): M = max lse_s, w_s = 2^(lse_s - M),
//   lse = M + log2 sum w_s,   o = sum w_s o_s / sum w_s,
// empty states (lse = -inf) weigh 0, all-empty rows give (0, -inf).  States
// are combined in index order, so results are run-to-run deterministic.
//
// Both kernels are memory-bound: each thread owns 4 consecutive d of one row
// and reads every state's 16 bytes once.  Also here: the test-only page
// gather, which copies exactly the K/V rows the attention kernels address.
#include "args.h"
#include "device.h"
#include "launch.h"

namespace pka {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void store4(void* out, int64_t idx, f32x4 v, bool fp32) {
  if (fp32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
  } else {
    u32x2 pk;
    pk[0] = pack_bf16(v[0], v[1]);
    pk[1] = pack_bf16(v[2], v[3]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx) = pk;
  }
}

// Split groups: rows [row0, row1) of (request, kv head), each row with S
// partial states.  A group's items (row, 4 d) are cut into whole blocks of
// kMergeBlock items and spread over up to merge_slices workgroups (the plan
// gives the slice count of its largest group), and workgroups take
// (slice, group) pairs grid-stride, slice-major: a few large groups (a long
// prefill split over many chunks) spread over the GPU as well as many small
// ones (decode).  Each thread keeps eight states' loads in flight.  The group
// list and the counts come from the plan image, so the launch does not depend
// on the batch.
static_assert(kThreads == kMergeBlock, "one item per thread per block");

template <int D>
__global__ __launch_bounds__(kThreads) void merge_split_kernel(MergeArgs a) {
  constexpr int C4 = D / 4;
  constexpr int kBatch = 8;  // states per batch of loads
  const PlanView pv = plan_view(a.ws);
  const float* part_lse = a.part_o + pv.partial_lse;
  const int G = a.group, Hq = a.num_qo_heads;
  const int n_groups = pv.num_merge, n_sl = pv.merge_slices;
  for (int v = blockIdx.x; v < n_groups * n_sl; v += gridDim.x) {
    const int slice = v / n_groups, gi = v - slice * n_groups;
    const int32_t* g = pv.merge + static_cast<int64_t>(gi) * 8;
    const int r = g[0], hk = g[1], row0 = g[2], row1 = g[3], pbase = g[4], S = g[5];
    const int nrows = row1 - row0;
    const int items = nrows * C4;
    const int blocks = (items + kMergeBlock - 1) / kMergeBlock;
    const int g_sl = min(n_sl, blocks);  // this group's slices
    if (slice >= g_sl) continue;
    const int per = (blocks + g_sl - 1) / g_sl * kMergeBlock;
    const int lo = slice * per, hi = min(items, lo + per);
    const int qo_begin = pv.req[static_cast<int64_t>(r) * 8];
    for (int it = lo + threadIdx.x; it < hi; it += kThreads) {
      const int row = it / C4, c4 = it - row * C4;
      const int64_t base = static_cast<int64_t>(pbase) + row;  // partial row of state s: base + s * nrows
      float M = -INFINITY;
      for (int s0 = 0; s0 < S; s0 += kBatch) {
        float l[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          l[j] = s0 + j < S ? part_lse[base + static_cast<int64_t>(s0 + j) * nrows] : -INFINITY;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) M = fmaxf(M, l[j]);
      }
      float W = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
        // an empty state (lse = -inf) weighs 0 and holds o = 0; states past S
        // read state s0's (finite) row with weight 0
        for (int s0 = 0; s0 < S; s0 += kBatch) {
          float l[kBatch];
          f32x4 x[kBatch];
#pragma unroll
          for (int j = 0; j < kBatch; ++j) {
            const bool ok = s0 + j < S;
            const int64_t prow = base + static_cast<int64_t>(ok ? s0 + j : s0) * nrows;
            l[j] = ok ? part_lse[prow] : -INFINITY;
            x[j] = *reinterpret_cast<const f32x4*>(a.part_o + prow * D + 4 * c4);
          }
#pragma unroll
          for (int j = 0; j < kBatch; ++j) {
            const float w = fast_exp2(l[j] - M);
            W += w;
            acc += w * x[j];
          }
        }
      }
      const bool seen = W > 0.f;
      const float inv = seen ? 1.f / W : 0.f;
      const int p = row0 + row;
      const int tok = p / G;
      const int64_t orow = static_cast<int64_t>(qo_begin + tok) * Hq + hk * G + (p - tok * G);
      store4(a.o, orow * D + 4 * c4, acc * inv, a.out_fp32 != 0);
      if (a.lse && c4 == 0) a.lse[orow] = seen ? M + __log2f(W) : -INFINITY;
    }
  }
}

__global__ __launch_bounds__(kThreads) void merge_states_kernel(MergeStatesArgs a) {
  const int D = a.head_dim, C4 = D / 4, H = a.num_heads, S = a.num_states;
  const int64_t items = a.n * H * C4;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; it < items;
       it += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int c4 = static_cast<int>(it % C4);
    const int64_t nh = it / C4;
    const int h = static_cast<int>(nh % H);
    const int64_t i = nh / H;
    const float* sp = a.s + i * a.s_row_stride + h;
    const float* vp = a.v + i * a.v_row_stride + static_cast<int64_t>(h) * D + 4 * c4;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, sp[s * a.s_state_stride]);
    float W = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      for (int s = 0; s < S; ++s) {
        const float w = fast_exp2(sp[s * a.s_state_stride] - M);
        if (w > 0.f) {
          W += w;
          acc += w * *reinterpret_cast<const f32x4*>(vp + s * a.v_state_stride);
        }
      }
    }
    const bool seen = W > 0.f;
    store4(a.v_out, (i * H + h) * D + 4 * c4, acc * (seen ? 1.f / W : 0.f), a.out_fp32 != 0);
    if (a.s_out && c4 == 0) a.s_out[i * H + h] = seen ? M + __log2f(W) : -INFINITY;
  }
}

// One workgroup per request: copy its kv_len K and V rows (all KV heads) into
// the dense outputs, addressing them exactly like the attention kernels do.
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
  const int32_t* rq = a.req + static_cast<int64_t>(blockIdx.x) * 8;
  const int kv_base = rq[2], kv_len = rq[3], dense = rq[4];
  const int CPR = a.head_dim / 8;
  const int per_tok = a.num_kv_heads * CPR;
  const int64_t items = static_cast<int64_t>(kv_len) * per_tok;
  for (int64_t it = threadIdx.x; it < items; it += kThreads) {
    const int t = static_cast<int>(it / per_tok);
    const int rem = static_cast<int>(it - static_cast<int64_t>(t) * per_tok);
    const int hk = rem / CPR, c = rem - hk * CPR;
    const int pg = a.kv_indices[kv_base + t / a.page_size];
    const int slot = t % a.page_size;
    const int64_t src = static_cast<int64_t>(pg) * a.page_stride + static_cast<int64_t>(slot) * a.row_stride +
                        hk * a.head_dim + 8 * c;
    const int64_t dst = (static_cast<int64_t>(dense + t) * a.num_kv_heads + hk) * a.head_dim + 8 * c;
    st16(a.k_out + dst, ld16(a.pool + src));
    st16(a.v_out + dst, ld16(a.pool + src + a.v_offset));
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    merge_split_kernel<128><<<grid, kThreads, 0, stream>>>(a);
  else
    merge_split_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge_states(const MergeStatesArgs& a, hipStream_t stream) {
  const int64_t items = a.n * a.num_heads * (a.head_dim / 4);
  if (items <= 0) return hipSuccess;
  int64_t grid = (items + kThreads - 1) / kThreads;
  if (grid > 65536) grid = 65536;
  merge_states_kernel<<<static_cast<int>(grid), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  gather_kernel<<<batch, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pka
