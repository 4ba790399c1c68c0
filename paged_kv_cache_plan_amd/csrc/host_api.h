// The HIP-free half of the C ABI: planning on host arrays, the per-thread
// error message, and the plan info.  Built into libpka.so and, on its own,
// into the host-only planner library that runs under a host sanitizer.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pka.h"
#include "planner.h"

namespace pka {

constexpr uint32_t kKnownFlags =
    PKA_DISABLE_SPLIT_KV | PKA_OUT_FP32 | PKA_RAGGED_KV | PKA_GRAPH_STABLE | PKA_MIXED_BATCH | PKA_MIXED_TWO_LAUNCHES;

// Record msg as this thread's last error and return code.
int set_error(int code, const std::string& msg);

// The whole plan of a batch: one image, or a mixed batch's header and two.
struct Planned {
  MixedPlan mp;
  const std::vector<int32_t>& image() const { return mp.mixed ? mp.image : mp.single.image; }
  size_t float_ws_bytes() const { return mp.mixed ? mp.float_ws_bytes : mp.single.float_ws_bytes; }
};

PlanInput make_input(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* kv_last_page_len, int32_t batch, int32_t nnz_pages, int32_t num_pages,
                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t causal, uint32_t flags, bool check_indices);

// Validate and plan; on failure the message is recorded and the status returned.
int plan_or_error(const PlanInput& in, Planned* res);

// plan_or_error for pka_plan_create: when the last pka_plan_workspace_size
// call on this thread planned the same batch (same arrays, sizes and flags),
// its work decomposition is taken over and only the page ids are checked and
// copied into the image, so that a size query followed by a create plans
// once.  (Work units never depend on the page ids, only on the lengths.)
int plan_for_create(const PlanInput& in, Planned* res);

void fill_plan_info(const Planned& pl, int32_t batch, int32_t nnz, pka_plan_info* info);

// Where a cascade keeps its parts: level l's plan workspaces at
// int_off[l] / float_off[l] (bytes, 256-aligned) inside the caller's two
// workspaces, then, in the float workspace, the levels' fp32 states
// v [L, total_q, Hq, D] at states_v and s [L, total_q, Hq] at states_s.
struct CascadeLayout {
  std::vector<size_t> int_off, int_bytes, float_off, float_bytes;
  size_t states_v = 0, states_s = 0;
  size_t int_total = 0, float_total = 0;
  int64_t total_q = 0;
};

// The flags a cascade passes to its level plans: fp32 states, split-KV as
// the caller asked.
constexpr uint32_t kCascadeLevelFlags = PKA_OUT_FP32;
constexpr uint32_t kCascadeFlags = PKA_OUT_FP32 | PKA_DISABLE_SPLIT_KV;

// Validate the levels (same query rows on every level) and size the
// workspaces; kv_indices may be null (sizes only).
int cascade_layout(int32_t num_levels, const int32_t* const* qo_indptr, const int32_t* const* kv_indptr,
                   const int32_t* const* kv_indices, const int32_t* const* kv_last_page_len, const int32_t* batch,
                   const int32_t* nnz_pages, int32_t num_pages, int32_t num_qo_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t page_size, int32_t causal, uint32_t flags, CascadeLayout* out);

}  // namespace pka
