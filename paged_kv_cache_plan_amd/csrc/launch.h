// Host launchers of the gfx950 kernels (defined next to the kernels).
#pragma once

#include <hip/hip_runtime_api.h>

#include "args.h"

namespace pka {

// wg_per_cu: workgroups per CU the plan was made for (selects the build at D=64)
hipError_t launch_prefill(const AttnArgs& a, int head_dim, bool paged, bool causal, int grid, int wg_per_cu,
                          hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, int head_dim, bool paged, int grid, hipStream_t stream);
// One-grid mixed batch: every workgroup runs the prefill worker and the decode
// worker (the two images' worker counts both equal grid); workgroup b starts
// with decode when b / xcds < decode_first_slots.
struct MixedGrid {
  int grid, xcds, decode_first_slots;
};
hipError_t launch_mixed(const AttnArgs& prefill, const AttnArgs& decode, int head_dim, bool paged, bool causal,
                        const MixedGrid& g, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_merge_states(const MergeStatesArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int batch, hipStream_t stream);
hipError_t launch_batch_indices_positions(const BatchPosArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// pka_run_noalloc: bytes of the static device scratch that holds a run's
// split-KV partial states, and its address on the current device (looked up
// once per device).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** out);

}  // namespace pka
