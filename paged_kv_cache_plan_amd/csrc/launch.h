// Host launchers of the gfx950 kernels (defined next to the kernels).
#pragma once

#include <hip/hip_runtime_api.h>

#include "args.h"

namespace pka {

hipError_t launch_prefill(const AttnArgs& a, int head_dim, bool paged, bool causal, int grid,
                          hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, int head_dim, bool paged, int grid, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_merge_states(const MergeStatesArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int batch, hipStream_t stream);
hipError_t launch_batch_indices_positions(const BatchPosArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

}  // namespace pka
