// Prefill / append attention over a paged (or ragged dense) KV cache, gfx950:
// the prefill kernel and its launch (the work itself: prefill_worker.h).
#include "launch.h"
#include "prefill_worker.h"

namespace pka {
namespace {

// WGS: resident workgroups per CU the build is for (its launch bound)
template <int D, int MODE, bool CAUSAL, int WGS>
__global__ __launch_bounds__(64 * prefill_waves(D), WGS) void prefill_kernel(AttnArgs a) {
  prefill_worker<D, MODE, CAUSAL>(a);
}

template <int D, int MODE, int WGS>
hipError_t launch_prefill_m(const AttnArgs& a, bool causal, int grid, hipStream_t stream) {
  if (causal)
    prefill_kernel<D, MODE, true, WGS><<<grid, 64 * prefill_waves(D), 0, stream>>>(a);
  else
    prefill_kernel<D, MODE, false, WGS><<<grid, 64 * prefill_waves(D), 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int WGS>
hipError_t launch_prefill_d(const AttnArgs& a, bool paged, bool causal, int grid, hipStream_t stream) {
  constexpr int kRun = kBN * (D / 8) / (64 * prefill_waves(D));  // keys per loader thread
  if (!paged) return launch_prefill_m<D, kKvRagged, WGS>(a, causal, grid, stream);
  if (a.page_shift >= 0 && a.page_size >= kRun) return launch_prefill_m<D, kKvPagedRun, WGS>(a, causal, grid, stream);
  if (a.page_shift >= 0) return launch_prefill_m<D, kKvPagedPow2, WGS>(a, causal, grid, stream);
  return launch_prefill_m<D, kKvPagedAny, WGS>(a, causal, grid, stream);
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, int head_dim, bool paged, bool causal, int grid, int wg_per_cu,
                          hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) return launch_prefill_d<128, prefill_wg_per_cu(128)>(a, paged, causal, grid, stream);
  if (wg_per_cu == kPrefillWgPerCuLong64)
    return launch_prefill_d<64, kPrefillWgPerCuLong64>(a, paged, causal, grid, stream);
  return launch_prefill_d<64, prefill_wg_per_cu(64)>(a, paged, causal, grid, stream);
}

}  // namespace pka
