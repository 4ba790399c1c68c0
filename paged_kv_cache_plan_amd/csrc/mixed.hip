// One-grid mixed prefill + decode attention, gfx950: one persistent launch
// in which every workgroup runs both the prefill worker (over the prefill
// image's queues until they are empty) and the decode worker (with as many
// waves as the prefill workgroup has, over the decode image's queue).  The
// workgroups of the first decode_first_slots slots of every XCD start with
// decode, the rest with prefill; whichever kind runs out first, its
// workgroups move on to the other, so prefill (matrix-bound) and decode
// (HBM-bound) run side by side and the split corrects itself ("[Roadmap]
// FlashInfer v0.2 to v0.3", milestone "POD-Attention Integration": prefill
// and decode attention in one kernel).
#include "decode_worker.h"
#include "launch.h"
#include "prefill_worker.h"

namespace pka {
namespace {

// Workgroup b runs on XCD b % xcds, in slot b / xcds of it.
template <int D, int PMODE, bool CAUSAL, int DMODE>
__global__ __launch_bounds__(64 * prefill_waves(D), prefill_wg_per_cu(D)) void mixed_kernel(
    AttnArgs ap, AttnArgs ad, int xcds, int decode_first_slots) {
  // (each order is straight-line code of its own: the two workers share no
  // live registers, which a loop over the two phases made the allocator
  // spill)
  if (static_cast<int>(blockIdx.x) / xcds < decode_first_slots) {
    decode_worker<D, DMODE, prefill_waves(D)>(ad);
    prefill_worker<D, PMODE, CAUSAL>(ap);
  } else {
    prefill_worker<D, PMODE, CAUSAL>(ap);
    decode_worker<D, DMODE, prefill_waves(D)>(ad);
  }
}

template <int D, int PMODE, int DMODE>
hipError_t launch_mixed_m(const AttnArgs& ap, const AttnArgs& ad, bool causal, const MixedGrid& g,
                          hipStream_t stream) {
  if (causal)
    mixed_kernel<D, PMODE, true, DMODE><<<g.grid, 64 * prefill_waves(D), 0, stream>>>(ap, ad, g.xcds,
                                                                                     g.decode_first_slots);
  else
    mixed_kernel<D, PMODE, false, DMODE><<<g.grid, 64 * prefill_waves(D), 0, stream>>>(ap, ad, g.xcds,
                                                                                      g.decode_first_slots);
  return hipGetLastError();
}

// The page addressing of each worker, chosen as the prefill and decode
// launchers choose it (both sides share the page size).
template <int D>
hipError_t launch_mixed_d(const AttnArgs& ap, const AttnArgs& ad, bool paged, bool causal, const MixedGrid& g,
                          hipStream_t stream) {
  constexpr int kRun = kBN * (D / 8) / (64 * prefill_waves(D));  // keys per prefill loader thread
  static_assert(kRun <= 16, "page sizes of 16 and more are whole prefill loader runs");
  if (!paged) return launch_mixed_m<D, kKvRagged, kRagged>(ap, ad, causal, g, stream);
  if (ap.page_shift >= 4) return launch_mixed_m<D, kKvPagedRun, kPagedUniform>(ap, ad, causal, g, stream);
  if (ap.page_shift >= 0 && ap.page_size >= kRun)
    return launch_mixed_m<D, kKvPagedRun, kPagedLane>(ap, ad, causal, g, stream);
  if (ap.page_shift >= 0) return launch_mixed_m<D, kKvPagedPow2, kPagedLane>(ap, ad, causal, g, stream);
  return launch_mixed_m<D, kKvPagedAny, kPagedLaneDiv>(ap, ad, causal, g, stream);
}

}  // namespace

hipError_t launch_mixed(const AttnArgs& prefill, const AttnArgs& decode, int head_dim, bool paged, bool causal,
                        const MixedGrid& g, hipStream_t stream) {
  if (g.grid <= 0 || g.xcds <= 0) return hipSuccess;
  if (head_dim == 128) return launch_mixed_d<128>(prefill, decode, paged, causal, g, stream);
  return launch_mixed_d<64>(prefill, decode, paged, causal, g, stream);
}

}  // namespace pka
