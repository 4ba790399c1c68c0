// Single-token decode attention over a paged (or ragged dense) KV cache, gfx950:
// the decode kernel and its launch (the work itself: decode_worker.h).
#include "decode_worker.h"
#include "launch.h"

namespace pka {
namespace {

template <int D, int MODE>
__global__ __launch_bounds__(64 * kDecodeWaves, kDecodeWgPerCu) void decode_kernel(AttnArgs a) {
  decode_worker<D, MODE, kDecodeWaves>(a);
}

template <int D>
hipError_t launch_decode_d(const AttnArgs& a, bool paged, int grid, hipStream_t stream) {
  if (!paged)
    decode_kernel<D, kRagged><<<grid, 64 * kDecodeWaves, 0, stream>>>(a);
  else if (a.page_shift >= 4)
    decode_kernel<D, kPagedUniform><<<grid, 64 * kDecodeWaves, 0, stream>>>(a);
  else if (a.page_shift >= 0)
    decode_kernel<D, kPagedLane><<<grid, 64 * kDecodeWaves, 0, stream>>>(a);
  else
    decode_kernel<D, kPagedLaneDiv><<<grid, 64 * kDecodeWaves, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, int head_dim, bool paged, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  return head_dim == 128 ? launch_decode_d<128>(a, paged, grid, stream)
                         : launch_decode_d<64>(a, paged, grid, stream);
}

}  // namespace pka
