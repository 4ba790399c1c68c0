// C ABI of the paged-KV attention library (declared in include/pka.h): the
// plan objects, their uploads and the kernel launches.  The HIP-free entry
// points (size query, host-only planning, error message) are in host_api.cpp.
//
// The plan runs the host planner on host index arrays, stages the resulting
// int workspace image in pinned host memory and enqueues one asynchronous
// host-to-device copy on the caller's stream; it never waits for the device
// (FlashInfer 0.2 release blog, "faster plan function").  Pinned staging
// comes from a library-wide pool, so planning in a loop allocates and frees
// no pinned memory once the pool holds buffers of the sizes in use.  Runs only
// enqueue kernels.  Errors become status codes plus a per-thread message.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pka.h"
#include "args.h"
#include "host_api.h"
#include "launch.h"
#include "planner.h"

using pka::set_error;

namespace {

int hip_error(const char* what, hipError_t e) {
  return set_error(PKA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr uint32_t kPlanMagic = 0x4e4c5050u;     // "PPLN"
constexpr uint32_t kCascadeMagic = 0x43534350u;  // "PCSC"

int env_int(const char* name) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : 0;
}

// One attention launch of a plan (and its split merge): a mixed batch has
// two, the prefill one first.
struct PartLaunch {
  int32_t kernel, num_workers, num_merge;
  int32_t merge_slices;  // workgroup slices of its largest merge group
  int32_t off_words;  // its image inside the int workspace
  size_t float_off;   // its partial states inside the float workspace (bytes)
  int32_t wg_per_cu;  // prefill: workgroups per CU planned for (selects the kernel build)
};

// A pinned host buffer that a plan stages its image in, and the event
// recorded after the copy that last read it.  The buffer may be reused once
// that event has completed.
struct Staging {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t copied = nullptr;
};

// Library-wide pool of staging buffers no plan holds.  Buffers go back to the
// pool when a plan is destroyed or outgrows them, and stay allocated until
// the process ends.
std::mutex g_pool_mu;
std::vector<Staging> g_pool;

bool copy_done(const Staging& s) { return hipEventQuery(s.copied) == hipSuccess; }

// A free staging buffer of at least `bytes` whose last copy has completed:
// the smallest such pooled buffer, else a new one (power-of-two size, at
// least 64 KiB).  Never waits for the device.
int acquire_staging(size_t bytes, Staging* out) {
  {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    size_t best = g_pool.size();
    for (size_t i = 0; i < g_pool.size(); ++i)
      if (g_pool[i].bytes >= bytes && (best == g_pool.size() || g_pool[i].bytes < g_pool[best].bytes) &&
          copy_done(g_pool[i]))
        best = i;
    if (best < g_pool.size()) {
      *out = g_pool[best];
      g_pool.erase(g_pool.begin() + static_cast<std::ptrdiff_t>(best));
      return PKA_OK;
    }
  }
  size_t sz = 64 << 10;
  while (sz < bytes) sz *= 2;
  Staging s;
  hipError_t e = hipHostMalloc(&s.ptr, sz, hipHostMallocDefault);
  if (e != hipSuccess) return hip_error("hipHostMalloc(plan staging)", e);
  e = hipEventCreateWithFlags(&s.copied, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipHostFree(s.ptr);
    return hip_error("hipEventCreateWithFlags(plan staging)", e);
  }
  s.bytes = sz;
  *out = s;
  return PKA_OK;
}

void release_staging(std::vector<Staging>* held) {
  std::lock_guard<std::mutex> lock(g_pool_mu);
  for (const Staging& s : *held) g_pool.push_back(s);
  held->clear();
}

// A mixed-batch plan's side stream and its fork / join events.  Creating a
// stream costs milliseconds, so they come from a library-wide pool (per
// device) and go back to it when the plan is destroyed (the caller has then
// made sure every run of the plan completed, so the stream is idle).
struct SideStream {
  int device = -1;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::vector<SideStream> g_side_pool;  // guarded by g_pool_mu

int acquire_side(SideStream* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error("hipGetDevice", e);
  {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    for (size_t i = 0; i < g_side_pool.size(); ++i)
      if (g_side_pool[i].device == dev) {
        *out = g_side_pool[i];
        g_side_pool.erase(g_side_pool.begin() + static_cast<std::ptrdiff_t>(i));
        return PKA_OK;
      }
  }
  SideStream s;
  s.device = dev;
  // default priority, like every stream here
  e = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&s.join, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (s.join) (void)hipEventDestroy(s.join);
    if (s.fork) (void)hipEventDestroy(s.fork);
    if (s.stream) (void)hipStreamDestroy(s.stream);
    return hip_error("plan side stream", e);
  }
  *out = s;
  return PKA_OK;
}

void release_side(const SideStream& s) {
  if (!s.stream) return;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  g_side_pool.push_back(s);
}

}  // namespace

struct pka_plan {
  uint32_t magic;
  pka_plan_info info;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group, causal, num_pages;
  uint32_t flags;
  float sm_scale;
  void* int_ws;
  void* float_ws;
  size_t partial_lse_offset;
  int32_t off_units, off_req, off_merge, off_idx, off_sched;
  size_t int_ws_bytes, float_ws_bytes;  // capacities of the caller's workspaces
  // Staging buffers this plan has uploaded from; one whose copy has
  // completed is reused, otherwise another comes from the pool, so an
  // update never waits for the device.
  std::vector<Staging> staging;
  int32_t num_parts;
  PartLaunch parts[2];
  bool one_grid;  // a mixed batch in one launch (not PKA_MIXED_TWO_LAUNCHES)
  int32_t xcds, decode_first_slots;  // one grid: which workgroups start with decode
  // PKA_MIXED_TWO_LAUNCHES: the decode launch runs on side.stream, forked
  // from and joined back into the caller's stream with the two events.
  SideStream side;
};

// A cascade: one plan per level over its share of the workspaces, and the
// levels' fp32 states merged into the output.
struct pka_cascade {
  uint32_t magic;
  int32_t num_levels, num_qo_heads, head_dim;
  int64_t total_q;
  uint32_t flags;
  std::vector<pka_plan*> plans;
  float* states_v;
  float* states_s;
};

namespace {

using pka::Planned;

bool plan_ok(const pka_plan* p) { return p && p->magic == kPlanMagic; }

// Copy a planned image into pinned staging and enqueue its upload to the
// int workspace, then record the plan's launch facts.  The staging buffer is
// one of the plan's whose previous copy has completed (checked with an event
// query, never waited for), or one taken from the pool.
int upload(pka_plan* p, const Planned& pl, int32_t batch, int32_t nnz, hipStream_t stream) {
  const std::vector<int32_t>& image = pl.image();
  const size_t need = image.size() * sizeof(int32_t);
  size_t idx = p->staging.size();
  for (size_t i = 0; i < p->staging.size(); ++i)
    if (p->staging[i].bytes >= need && copy_done(p->staging[i])) {
      idx = i;
      break;
    }
  if (idx == p->staging.size()) {
    Staging s;
    const int st = acquire_staging(need, &s);
    if (st != PKA_OK) return st;
    // A plan keeps at most two buffers: the smallest other one goes back to
    // the pool, with its event, so that nobody reuses it before its copy
    // has completed.
    if (p->staging.size() >= 2) {
      size_t drop = 0;
      for (size_t i = 1; i < p->staging.size(); ++i)
        if (p->staging[i].bytes < p->staging[drop].bytes) drop = i;
      std::vector<Staging> back{p->staging[drop]};
      p->staging.erase(p->staging.begin() + static_cast<std::ptrdiff_t>(drop));
      release_staging(&back);
    }
    p->staging.push_back(s);
    idx = p->staging.size() - 1;
  }
  Staging& slot = p->staging[idx];
  std::memcpy(slot.ptr, image.data(), need);
  hipError_t e = hipMemcpyAsync(p->int_ws, slot.ptr, need, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_error("hipMemcpyAsync(plan upload)", e);
  e = hipEventRecord(slot.copied, stream);
  if (e != hipSuccess) return hip_error("hipEventRecord(plan upload)", e);
  pka::fill_plan_info(pl, batch, nnz, &p->info);
  const pka::PlanResult& res = pl.mp.single;
  p->partial_lse_offset = res.partial_lse_offset;
  p->off_units = res.image[pka::kHdrOffUnits];
  p->off_req = res.image[pka::kHdrOffReq];
  p->off_merge = res.image[pka::kHdrOffMerge];
  p->off_idx = res.image[pka::kHdrOffIndices];
  p->off_sched = res.image[pka::kHdrOffSched];
  p->one_grid = pl.mp.mixed && pl.mp.one_grid;
  p->xcds = pl.mp.xcds;
  p->decode_first_slots = pl.mp.decode_first_slots;
  if (pl.mp.mixed) {
    const pka::MixedPlan& mp = pl.mp;
    p->num_parts = 2;
    p->parts[0] = {mp.prefill.kernel, mp.prefill.num_workers, mp.prefill.num_merge,
                   mp.prefill.image[pka::kHdrMergeSlices], mp.off_prefill, 0, mp.prefill.wg_per_cu};
    p->parts[1] = {mp.decode.kernel, mp.decode.num_workers, mp.decode.num_merge,
                   mp.decode.image[pka::kHdrMergeSlices], mp.off_decode, mp.float_off_decode, mp.decode.wg_per_cu};
  } else {
    p->num_parts = 1;
    p->parts[0] = {res.kernel, res.num_workers, res.num_merge, res.image[pka::kHdrMergeSlices], 0, 0, res.wg_per_cu};
  }
  return PKA_OK;
}

// KV addressing: element strides between pages (ragged: tokens), slots and
// KV heads; V rows sit at the same offsets from v as K rows from k.
struct KvLayout {
  int64_t page_stride, slot_stride, head_stride;
};

// The layouts of pka_run (NHD pool [num_pages, 2, ps, Hkv, D]) and
// pka_run_ragged ([total_kv, Hkv, D] K and V).
KvLayout standard_layout(const pka_plan* p) {
  const int64_t row = static_cast<int64_t>(p->num_kv_heads) * p->head_dim;
  if (p->flags & PKA_RAGGED_KV) return {row, row, p->head_dim};
  return {2 * static_cast<int64_t>(p->page_size) * row, row, p->head_dim};
}

pka::AttnArgs attn_args(const pka_plan* p, const PartLaunch& part, const void* q, const void* k, const void* v,
                        const KvLayout& kv, void* o, float* lse, void* float_base) {
  pka::AttnArgs a{};
  const int32_t* iw = static_cast<const int32_t*>(p->int_ws) + part.off_words;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.lse = lse;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(float_base) + part.float_off);
  a.ws = const_cast<int32_t*>(iw);
  const bool ragged = p->flags & PKA_RAGGED_KV;
  a.page_size = ragged ? 1 : p->page_size;
  a.page_stride = kv.page_stride;
  a.row_stride = static_cast<int32_t>(kv.slot_stride);
  a.head_stride = kv.head_stride;
  int shift = -1;
  for (int s = 0; s < 8; ++s)
    if ((1 << s) == a.page_size) shift = s;
  a.page_shift = shift;
  a.num_qo_heads = p->num_qo_heads;
  a.group = p->group;
  a.out_fp32 = (p->flags & PKA_OUT_FP32) ? 1 : 0;
  a.scale_log2 = p->sm_scale * 1.4426950408889634f;
  return a;
}

// A part's split merge, if it split any KV (a graph-stable plan: always).
int run_merge(const pka_plan* p, const PartLaunch& part, const pka::AttnArgs& a, void* o, float* lse,
              hipStream_t stream) {
  const bool stable = (p->flags & PKA_GRAPH_STABLE) != 0;
  if (part.num_merge > 0 || stable) {
    pka::MergeArgs m{};
    m.part_o = a.part_o;
    m.ws = a.ws;
    m.o = o;
    m.lse = lse;
    m.num_qo_heads = p->num_qo_heads;
    m.group = p->group;
    m.out_fp32 = a.out_fp32;
    // one workgroup per (slice, group), up to a cap (the kernel is grid-stride)
    const int64_t pairs = int64_t(part.num_merge) * std::max(1, part.merge_slices);
    const int grid = stable ? pka::kMergeGrid : static_cast<int>(std::min<int64_t>(pairs, 8 * pka::kMergeGrid));
    const hipError_t e = pka::launch_merge(m, p->head_dim, grid, stream);
    if (e != hipSuccess) return hip_error("merge launch", e);
  }
  return PKA_OK;
}

// One part's attention launch and, if it split any KV, its merge.
int run_part(const pka_plan* p, const PartLaunch& part, const void* q, const void* k, const void* v,
             const KvLayout& kv, void* o, float* lse, void* float_base, hipStream_t stream) {
  const pka::AttnArgs a = attn_args(p, part, q, k, v, kv, o, lse, float_base);
  const bool paged = !(p->flags & PKA_RAGGED_KV);
  hipError_t e;
  if (part.kernel == PKA_KERNEL_DECODE)
    e = pka::launch_decode(a, p->head_dim, paged, part.num_workers, stream);
  else
    e = pka::launch_prefill(a, p->head_dim, paged, p->causal != 0, part.num_workers, part.wg_per_cu, stream);
  if (e != hipSuccess) return hip_error("attention launch", e);
  return run_merge(p, part, a, o, lse, stream);
}

// float_base: where the plan's partial states go (its float workspace, or
// the static scratch of pka_run_noalloc).
int run_common(const pka_plan* p, const void* q, const void* k, const void* v, const KvLayout& kv, void* o,
               float* lse, hipStream_t stream, void* float_base = nullptr) {
  if (!float_base) float_base = p->float_ws;
  // A graph-stable plan always enqueues the same launches (a captured run is
  // replayed for later batches); the kernels find an empty batch empty.
  const bool stable = (p->flags & PKA_GRAPH_STABLE) != 0;
  if (p->info.total_q == 0 && !stable) return PKA_OK;
  if (!q || !o) return set_error(PKA_ERR_INVALID_ARG, "q and o must not be NULL");
  if (p->info.total_kv > 0 && !k) return set_error(PKA_ERR_INVALID_ARG, "KV pointer must not be NULL");
  if (p->num_parts == 1) return run_part(p, p->parts[0], q, k, v, kv, o, lse, float_base, stream);
  if (p->one_grid) {
    // One launch serves both images (the planner gave both the same worker
    // count), then each part's merge.
    const pka::AttnArgs ap = attn_args(p, p->parts[0], q, k, v, kv, o, lse, float_base);
    const pka::AttnArgs ad = attn_args(p, p->parts[1], q, k, v, kv, o, lse, float_base);
    const pka::MixedGrid g{p->parts[0].num_workers, p->xcds, p->decode_first_slots};
    const hipError_t e =
        pka::launch_mixed(ap, ad, p->head_dim, !(p->flags & PKA_RAGGED_KV), p->causal != 0, g, stream);
    if (e != hipSuccess) return hip_error("mixed attention launch", e);
    const int st = run_merge(p, p->parts[0], ap, o, lse, stream);
    if (st != PKA_OK) return st;
    return run_merge(p, p->parts[1], ad, o, lse, stream);
  }
  // Mixed batch: the prefill launch goes first, on the caller's stream, so
  // that its workgroups take their compute units before the decode launch
  // (forked onto the plan's side stream) fills the rest; the caller's stream
  // then waits for the side stream.  The two write disjoint output rows.
  hipError_t e = hipEventRecord(p->side.fork, stream);
  if (e != hipSuccess) return hip_error("hipEventRecord(fork)", e);
  e = hipStreamWaitEvent(p->side.stream, p->side.fork, 0);
  if (e != hipSuccess) return hip_error("hipStreamWaitEvent(fork)", e);
  int st = run_part(p, p->parts[0], q, k, v, kv, o, lse, float_base, stream);
  if (st != PKA_OK) return st;
  st = run_part(p, p->parts[1], q, k, v, kv, o, lse, float_base, p->side.stream);
  if (st != PKA_OK) return st;
  e = hipEventRecord(p->side.join, p->side.stream);
  if (e != hipSuccess) return hip_error("hipEventRecord(join)", e);
  e = hipStreamWaitEvent(stream, p->side.join, 0);
  if (e != hipSuccess) return hip_error("hipStreamWaitEvent(join)", e);
  return PKA_OK;
}

}  // namespace

extern "C" {

int pka_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* kv_last_page_len, int32_t batch, int32_t nnz_pages, int32_t num_pages_in_pool,
                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                    int32_t causal, float sm_scale, uint32_t flags, void* int_ws, size_t int_ws_bytes,
                    void* float_ws, size_t float_ws_bytes, pka_stream_t stream, pka_plan** out) {
  try {
    if (!out) return set_error(PKA_ERR_INVALID_ARG, "out must not be NULL");
    *out = nullptr;
    if (!int_ws || !float_ws) return set_error(PKA_ERR_INVALID_ARG, "workspaces must not be NULL");
    if (!std::isfinite(sm_scale)) return set_error(PKA_ERR_INVALID_ARG, "sm_scale must be finite");
    pka::PlanInput in = pka::make_input(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, nnz_pages,
                                        num_pages_in_pool, num_qo_heads, num_kv_heads, head_dim, page_size,
                                        causal, flags, true);
    Planned res;
    int st = pka::plan_for_create(in, &res);
    if (st != PKA_OK) return st;
    const size_t need = res.image().size() * sizeof(int32_t);
    if (int_ws_bytes < need)
      return set_error(PKA_ERR_WORKSPACE, "int workspace has " + std::to_string(int_ws_bytes) + " bytes, needs " +
                                              std::to_string(need));
    if (float_ws_bytes < res.float_ws_bytes())
      return set_error(PKA_ERR_WORKSPACE, "float workspace has " + std::to_string(float_ws_bytes) +
                                              " bytes, needs " + std::to_string(res.float_ws_bytes()));
    pka_plan* p = new pka_plan{};
    p->magic = kPlanMagic;
    p->num_qo_heads = num_qo_heads;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->page_size = page_size;
    p->group = num_qo_heads / num_kv_heads;
    p->causal = causal ? 1 : 0;
    p->num_pages = num_pages_in_pool;
    p->flags = flags;
    p->sm_scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
    p->int_ws = int_ws;
    p->float_ws = float_ws;
    p->int_ws_bytes = int_ws_bytes;
    p->float_ws_bytes = float_ws_bytes;
    if ((flags & PKA_MIXED_BATCH) && (flags & PKA_MIXED_TWO_LAUNCHES)) {
      st = acquire_side(&p->side);
      if (st != PKA_OK) {
        pka_plan_destroy(p);
        return st;
      }
    }
    st = upload(p, res, batch, (flags & PKA_RAGGED_KV) ? 0 : nnz_pages, stream);
    if (st != PKA_OK) {
      pka_plan_destroy(p);
      return st;
    }
    if (env_int("PKA_LOG"))
      std::fprintf(stderr, "[pka] plan: kernel=%d units=%d merge_groups=%d partial_rows=%d kv_chunk=%d "
                   "workers=%d prefill_cus=%d decode_cus=%d int_ws=%zu float_ws=%lld\n",
                   p->info.kernel, p->info.num_units, p->info.num_merge_groups, p->info.num_partial_rows,
                   p->info.kv_chunk, p->info.num_workers, p->info.prefill_cus, p->info.decode_cus, need,
                   static_cast<long long>(p->info.float_ws_bytes));
    *out = p;
    return PKA_OK;
  } catch (const std::exception& ex) {
    return set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

int pka_plan_get_info(const pka_plan* plan, pka_plan_info* info) {
  if (!plan_ok(plan) || !info) return set_error(PKA_ERR_INVALID_ARG, "invalid plan or info pointer");
  *info = plan->info;
  return PKA_OK;
}

int pka_run(const pka_plan* plan, const void* q, const void* paged_kv, void* o, float* lse,
            pka_stream_t stream) {
  if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
  if (plan->flags & PKA_RAGGED_KV)
    return set_error(PKA_ERR_INVALID_ARG, "plan was made with PKA_RAGGED_KV: use pka_run_ragged");
  const int64_t half = static_cast<int64_t>(plan->page_size) * plan->num_kv_heads * plan->head_dim;
  const void* v = paged_kv ? static_cast<const uint16_t*>(paged_kv) + half : nullptr;
  return run_common(plan, q, paged_kv, v, standard_layout(plan), o, lse, stream);
}

int pka_run_noalloc(const pka_plan* plan, const void* q, const void* paged_kv, void* o, float* lse,
                    pka_stream_t stream) {
  if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
  if (plan->flags & PKA_RAGGED_KV)
    return set_error(PKA_ERR_INVALID_ARG, "plan was made with PKA_RAGGED_KV: pka_run_noalloc takes a paged plan");
  if (static_cast<size_t>(plan->info.float_ws_bytes) > pka::kNoallocScratchBytes)
    return set_error(PKA_ERR_WORKSPACE, "pka_run_noalloc: the plan's partial states need " +
                                            std::to_string(plan->info.float_ws_bytes) +
                                            " bytes; the static scratch holds " +
                                            std::to_string(pka::kNoallocScratchBytes));
  void* scratch = nullptr;
  const hipError_t e = pka::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_error("pka_run_noalloc: scratch address", e);
  const int64_t half = static_cast<int64_t>(plan->page_size) * plan->num_kv_heads * plan->head_dim;
  const void* v = paged_kv ? static_cast<const uint16_t*>(paged_kv) + half : nullptr;
  return run_common(plan, q, paged_kv, v, standard_layout(plan), o, lse, stream, scratch);
}

int pka_run_paged_strided(const pka_plan* plan, const void* q, const void* k_cache, const void* v_cache,
                          int64_t page_stride, int64_t slot_stride, int64_t head_stride, void* o, float* lse,
                          pka_stream_t stream) {
  if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
  if (plan->flags & PKA_RAGGED_KV)
    return set_error(PKA_ERR_INVALID_ARG, "plan was made with PKA_RAGGED_KV: use pka_run_ragged");
  if (plan->info.total_kv > 0 && (!k_cache || !v_cache))
    return set_error(PKA_ERR_INVALID_ARG, "k_cache and v_cache must not be NULL");
  if (page_stride <= 0 || slot_stride <= 0 || head_stride <= 0 || page_stride % 8 || slot_stride % 8 ||
      head_stride % 8)
    return set_error(PKA_ERR_INVALID_ARG, "strides must be positive multiples of 8 elements");
  if (page_stride >= (int64_t(1) << 31) || slot_stride >= (int64_t(1) << 24))
    return set_error(PKA_ERR_UNSUPPORTED, "page stride must be < 2^31 and slot stride < 2^24 elements");
  for (const void* ptr : {k_cache, v_cache})
    if (ptr && reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return set_error(PKA_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
  return run_common(plan, q, k_cache, v_cache, {page_stride, slot_stride, head_stride}, o, lse, stream);
}

int pka_run_ragged(const pka_plan* plan, const void* q, const void* k, const void* v, void* o, float* lse,
                   pka_stream_t stream) {
  if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
  if (!(plan->flags & PKA_RAGGED_KV))
    return set_error(PKA_ERR_INVALID_ARG, "plan was made for a paged KV cache: use pka_run");
  if (plan->info.total_kv > 0 && !v) return set_error(PKA_ERR_INVALID_ARG, "v must not be NULL");
  return run_common(plan, q, k, v, standard_layout(plan), o, lse, stream);
}

int pka_merge_states(const float* v, const float* s, int64_t n, int32_t num_states, int32_t num_heads,
                     int32_t head_dim, void* v_out, float* s_out, uint32_t flags, pka_stream_t stream) {
  const int64_t S = num_states, H = num_heads, D = head_dim;
  return pka_merge_states_strided(v, s, n, num_states, num_heads, head_dim, S * H * D, H * D, S * H, H, v_out,
                                  s_out, flags, stream);
}

int pka_merge_states_strided(const float* v, const float* s, int64_t n, int32_t num_states, int32_t num_heads,
                             int32_t head_dim, int64_t v_row_stride, int64_t v_state_stride,
                             int64_t s_row_stride, int64_t s_state_stride, void* v_out, float* s_out,
                             uint32_t flags, pka_stream_t stream) {
  if (n < 0 || num_states < 1 || num_heads < 1 || head_dim < 4 || head_dim % 4 != 0 || head_dim > 1024)
    return set_error(PKA_ERR_INVALID_ARG, "merge_states: bad sizes");
  if (v_row_stride < 0 || v_state_stride < 0 || s_row_stride < 0 || s_state_stride < 0 || v_row_stride % 4 ||
      v_state_stride % 4)
    return set_error(PKA_ERR_INVALID_ARG, "merge_states: v strides must be non-negative multiples of 4");
  if ((v && reinterpret_cast<uintptr_t>(v) % 16) || (v_out && reinterpret_cast<uintptr_t>(v_out) % 16))
    return set_error(PKA_ERR_INVALID_ARG, "merge_states: v and v_out must be 16-byte aligned");
  if (flags & ~uint32_t(PKA_OUT_FP32)) return set_error(PKA_ERR_INVALID_ARG, "merge_states: unknown flags");
  if (n == 0) return PKA_OK;
  if (!v || !s || !v_out) return set_error(PKA_ERR_INVALID_ARG, "merge_states: null pointer");
  pka::MergeStatesArgs a{};
  a.v = v;
  a.s = s;
  a.v_row_stride = v_row_stride;
  a.v_state_stride = v_state_stride;
  a.s_row_stride = s_row_stride;
  a.s_state_stride = s_state_stride;
  a.v_out = v_out;
  a.s_out = s_out;
  a.n = n;
  a.num_states = num_states;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.out_fp32 = (flags & PKA_OUT_FP32) ? 1 : 0;
  const hipError_t e = pka::launch_merge_states(a, stream);
  if (e != hipSuccess) return hip_error("merge_states launch", e);
  return PKA_OK;
}

int pka_debug_gather(const pka_plan* plan, const void* paged_kv, void* k_dense, void* v_dense,
                     pka_stream_t stream) {
  if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
  if (plan->flags & PKA_RAGGED_KV) return set_error(PKA_ERR_INVALID_ARG, "debug_gather needs a paged plan");
  if (plan->num_parts != 1) return set_error(PKA_ERR_UNSUPPORTED, "debug_gather does not take a mixed-batch plan");
  if (plan->info.total_kv == 0) return PKA_OK;
  if (!paged_kv || !k_dense || !v_dense) return set_error(PKA_ERR_INVALID_ARG, "null pointer");
  pka::GatherArgs a{};
  const int32_t* iw = static_cast<const int32_t*>(plan->int_ws);
  a.pool = static_cast<const uint16_t*>(paged_kv);
  a.k_out = static_cast<uint16_t*>(k_dense);
  a.v_out = static_cast<uint16_t*>(v_dense);
  a.req = iw + plan->off_req;
  a.kv_indices = iw + plan->off_idx;
  const int64_t row = static_cast<int64_t>(plan->num_kv_heads) * plan->head_dim;
  a.row_stride = static_cast<int32_t>(row);
  a.v_offset = static_cast<int64_t>(plan->page_size) * row;
  a.page_stride = 2 * a.v_offset;
  a.num_kv_heads = plan->num_kv_heads;
  a.page_size = plan->page_size;
  a.head_dim = plan->head_dim;
  const hipError_t e = pka::launch_gather(a, plan->info.batch, stream);
  if (e != hipSuccess) return hip_error("debug_gather launch", e);
  return PKA_OK;
}

int pka_get_batch_indices_positions(const int32_t* append_indptr, const int32_t* seq_lens, int32_t batch,
                                    int32_t nnz, int32_t* batch_indices, int32_t* positions,
                                    pka_stream_t stream) {
  if (batch < 0 || nnz < 0) return set_error(PKA_ERR_INVALID_ARG, "batch_indices_positions: negative size");
  if (nnz == 0) return PKA_OK;
  if (batch == 0) return set_error(PKA_ERR_INVALID_ARG, "batch_indices_positions: nnz > 0 with no request");
  if (!append_indptr || !seq_lens || !batch_indices || !positions)
    return set_error(PKA_ERR_INVALID_ARG, "batch_indices_positions: null pointer");
  pka::BatchPosArgs a{};
  a.append_indptr = append_indptr;
  a.seq_lens = seq_lens;
  a.batch_indices = batch_indices;
  a.positions = positions;
  a.batch = batch;
  a.nnz = nnz;
  const hipError_t e = pka::launch_batch_indices_positions(a, stream);
  if (e != hipSuccess) return hip_error("batch_indices_positions launch", e);
  return PKA_OK;
}

int pka_append_paged_kv(const void* append_k, const void* append_v, const int32_t* batch_indices,
                        const int32_t* positions, int32_t nnz, void* paged_kv, int32_t num_pages,
                        int32_t page_size, int32_t num_kv_heads, int32_t head_dim, const int32_t* kv_indices,
                        const int32_t* kv_indptr, int32_t batch, pka_stream_t stream) {
  if (nnz < 0 || batch < 0 || num_pages < 0) return set_error(PKA_ERR_INVALID_ARG, "append: negative size");
  if (head_dim != 64 && head_dim != 128) return set_error(PKA_ERR_UNSUPPORTED, "append: head_dim must be 64 or 128");
  if (num_kv_heads < 1) return set_error(PKA_ERR_INVALID_ARG, "append: num_kv_heads must be >= 1");
  if (page_size < 1 || page_size > 128) return set_error(PKA_ERR_UNSUPPORTED, "append: page_size must be in [1, 128]");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (row > (int64_t(1) << 24) || static_cast<int64_t>(num_pages) * 2 * page_size * row > (int64_t(1) << 62))
    return set_error(PKA_ERR_UNSUPPORTED, "append: sizes too large");
  if (nnz == 0) return PKA_OK;
  if (!append_k || !append_v || !batch_indices || !positions || !paged_kv || !kv_indices || !kv_indptr)
    return set_error(PKA_ERR_INVALID_ARG, "append: null pointer");
  for (const void* ptr : {append_k, append_v, static_cast<const void*>(paged_kv)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return set_error(PKA_ERR_INVALID_ARG, "append: K/V tensors must be 16-byte aligned");
  pka::AppendArgs a{};
  a.append_k = static_cast<const uint16_t*>(append_k);
  a.append_v = static_cast<const uint16_t*>(append_v);
  a.batch_indices = batch_indices;
  a.positions = positions;
  a.paged_kv = static_cast<uint16_t*>(paged_kv);
  a.kv_indices = kv_indices;
  a.kv_indptr = kv_indptr;
  a.nnz = nnz;
  a.batch = batch;
  a.num_pages = num_pages;
  a.page_size = page_size;
  int shift = -1;
  for (int sh = 0; sh < 8; ++sh)
    if ((1 << sh) == page_size) shift = sh;
  a.page_shift = shift;
  a.row_elems = static_cast<int32_t>(row);
  const hipError_t e = pka::launch_append(a, stream);
  if (e != hipSuccess) return hip_error("append launch", e);
  return PKA_OK;
}

int pka_plan_update(pka_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* kv_last_page_len, int32_t batch, int32_t nnz_pages, pka_stream_t stream) {
  try {
    if (!plan_ok(plan)) return set_error(PKA_ERR_INVALID_ARG, "invalid plan");
    pka::PlanInput in = pka::make_input(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, nnz_pages,
                                        plan->num_pages, plan->num_qo_heads, plan->num_kv_heads, plan->head_dim,
                                        plan->page_size, plan->causal, plan->flags, true);
    Planned res;
    const int st = pka::plan_or_error(in, &res);
    if (st != PKA_OK) return st;
    const size_t need = res.image().size() * sizeof(int32_t);
    if (plan->int_ws_bytes < need)
      return set_error(PKA_ERR_WORKSPACE, "int workspace has " + std::to_string(plan->int_ws_bytes) +
                                              " bytes, needs " + std::to_string(need));
    if (plan->float_ws_bytes < res.float_ws_bytes())
      return set_error(PKA_ERR_WORKSPACE, "float workspace has " + std::to_string(plan->float_ws_bytes) +
                                              " bytes, needs " + std::to_string(res.float_ws_bytes()));
    const pka::PlanResult& one = res.mp.single;
    if ((plan->flags & PKA_GRAPH_STABLE) &&
        (one.kernel != plan->info.kernel || one.num_workers != plan->info.num_workers))
      return set_error(PKA_ERR_INVALID_ARG,
                       "a graph-stable plan cannot switch between prefill and decode batches");
    return upload(plan, res, batch, (plan->flags & PKA_RAGGED_KV) ? 0 : nnz_pages, stream);
  } catch (const std::exception& ex) {
    return set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

int pka_cascade_create(int32_t num_levels, const int32_t* const* qo_indptr, const int32_t* const* kv_indptr,
                       const int32_t* const* kv_indices, const int32_t* const* kv_last_page_len, const int32_t* batch,
                       const int32_t* nnz_pages, int32_t num_pages_in_pool, int32_t num_qo_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size, int32_t causal, float sm_scale, uint32_t flags, void* int_ws,
                       size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes, pka_stream_t stream,
                       pka_cascade** out) {
  try {
    if (!out) return set_error(PKA_ERR_INVALID_ARG, "out must not be NULL");
    *out = nullptr;
    if (!int_ws || !float_ws) return set_error(PKA_ERR_INVALID_ARG, "workspaces must not be NULL");
    if (!kv_indices || !nnz_pages) return set_error(PKA_ERR_INVALID_ARG, "cascade: kv_indices and nnz_pages must not be NULL");
    pka::CascadeLayout lay;
    int st = pka::cascade_layout(num_levels, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, nnz_pages,
                                 num_pages_in_pool, num_qo_heads, num_kv_heads, head_dim, page_size, causal, flags,
                                 &lay);
    if (st != PKA_OK) return st;
    if (int_ws_bytes < lay.int_total || float_ws_bytes < lay.float_total)
      return set_error(PKA_ERR_WORKSPACE, "cascade workspaces have " + std::to_string(int_ws_bytes) + " / " +
                                              std::to_string(float_ws_bytes) + " bytes, need " +
                                              std::to_string(lay.int_total) + " / " + std::to_string(lay.float_total));
    pka_cascade* c = new pka_cascade{};
    c->magic = kCascadeMagic;
    c->num_levels = num_levels;
    c->num_qo_heads = num_qo_heads;
    c->head_dim = head_dim;
    c->total_q = lay.total_q;
    c->flags = flags;
    c->states_v = reinterpret_cast<float*>(static_cast<char*>(float_ws) + lay.states_v);
    c->states_s = reinterpret_cast<float*>(static_cast<char*>(float_ws) + lay.states_s);
    for (int l = 0; l < num_levels; ++l) {
      pka_plan* p = nullptr;
      st = pka_plan_create(qo_indptr[l], kv_indptr[l], kv_indices[l], kv_last_page_len[l], batch[l], nnz_pages[l],
                           num_pages_in_pool, num_qo_heads, num_kv_heads, head_dim, page_size,
                           (causal && l == num_levels - 1) ? 1 : 0, sm_scale,
                           (flags & PKA_DISABLE_SPLIT_KV) | pka::kCascadeLevelFlags,
                           static_cast<char*>(int_ws) + lay.int_off[l], lay.int_bytes[l],
                           static_cast<char*>(float_ws) + lay.float_off[l], lay.float_bytes[l], stream, &p);
      if (st != PKA_OK) {
        const std::string msg = std::string("cascade: level ") + std::to_string(l) + ": " + pka_last_error();
        pka_cascade_destroy(c);
        return set_error(st, msg);
      }
      c->plans.push_back(p);
    }
    *out = c;
    return PKA_OK;
  } catch (const std::exception& ex) {
    return set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

int pka_cascade_run(const pka_cascade* c, const void* q, const void* paged_kv, void* o, float* lse,
                    pka_stream_t stream) {
  if (!c || c->magic != kCascadeMagic) return set_error(PKA_ERR_INVALID_ARG, "invalid cascade");
  if (c->total_q == 0) return PKA_OK;
  if (!o) return set_error(PKA_ERR_INVALID_ARG, "o must not be NULL");
  const int64_t n = c->total_q, H = c->num_qo_heads, D = c->head_dim;
  for (int l = 0; l < c->num_levels; ++l) {
    const int st = pka_run(c->plans[l], q, paged_kv, c->states_v + l * n * H * D, c->states_s + l * n * H, stream);
    if (st != PKA_OK) return st;
  }
  // state s of row i, head h: v[i*H*D + s*n*H*D + h*D ..], s[i*H + s*n*H + h]
  return pka_merge_states_strided(c->states_v, c->states_s, n, c->num_levels, c->num_qo_heads, c->head_dim, H * D,
                                  n * H * D, H, n * H, o, lse, c->flags & PKA_OUT_FP32, stream);
}

void pka_cascade_destroy(pka_cascade* c) {
  if (!c || c->magic != kCascadeMagic) return;
  for (pka_plan* p : c->plans) pka_plan_destroy(p);
  c->magic = 0;
  delete c;
}

void pka_plan_destroy(pka_plan* plan) {
  if (!plan_ok(plan)) return;
  release_side(plan->side);  // back to the pool, idle (the caller waited for the runs)
  release_staging(&plan->staging);  // pooled with their events, never freed here
  plan->magic = 0;
  delete plan;
}

}  // extern "C"
