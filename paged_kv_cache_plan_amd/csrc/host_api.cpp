// The HIP-free entry points of the C ABI (include/pka.h): the size query,
// host-only planning and the error message.  The plan never needs a GPU to be
// computed (FlashInfer 0.2 release blog, "faster plan function": planning
// runs on host arrays), so this file links without the HIP runtime.
#include "host_api.h"

#include <cstdlib>
#include <cstring>
#include <exception>

namespace pka {
namespace {

thread_local std::string g_last_error;

int env_int(const char* name) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : 0;
}

void fill_info(const PlanResult& res, int32_t batch, int32_t nnz, pka_plan_info* info) {
  info->kernel = res.kernel;
  info->num_units = res.num_units;
  info->num_merge_groups = res.num_merge;
  info->num_partial_rows = res.num_partial_rows;
  info->block_rows = res.block_rows;
  info->kv_chunk = res.kv_chunk;
  info->batch = batch;
  info->nnz_pages = nnz;
  info->total_q = res.total_q;
  info->total_kv = res.total_kv;
  info->int_ws_bytes = static_cast<int64_t>(res.image.size() * sizeof(int32_t));
  info->float_ws_bytes = static_cast<int64_t>(res.float_ws_bytes);
  info->num_workers = res.num_workers;
  info->num_queues = res.num_queues;
}

// What a plan's work decomposition depends on: every input but the page ids
// (which are only validated and copied) and the pool size (only validation).
struct PlanKey {
  std::vector<int32_t> qo_indptr, kv_indptr, last;
  int32_t scalars[9] = {};

  static PlanKey of(const PlanInput& in) {
    PlanKey k;
    const int B = in.batch;
    k.qo_indptr.assign(in.qo_indptr, in.qo_indptr + B + 1);
    k.kv_indptr.assign(in.kv_indptr, in.kv_indptr + B + 1);
    if (in.kv_last_page_len && !(in.flags & kFlagRagged)) k.last.assign(in.kv_last_page_len, in.kv_last_page_len + B);
    const int32_t s[9] = {in.batch, in.num_qo_heads, in.num_kv_heads, in.head_dim, in.page_size, in.causal,
                          static_cast<int32_t>(in.flags), in.kv_chunk_override, in.prefill_cus_override};
    std::memcpy(k.scalars, s, sizeof(s));
    return k;
  }
  bool same(const PlanInput& in) const {
    const int B = in.batch;
    if (B < 0 || static_cast<size_t>(B) + 1 != qo_indptr.size() || !in.qo_indptr || !in.kv_indptr) return false;
    const int32_t s[9] = {in.batch, in.num_qo_heads, in.num_kv_heads, in.head_dim, in.page_size, in.causal,
                          static_cast<int32_t>(in.flags), in.kv_chunk_override, in.prefill_cus_override};
    if (std::memcmp(s, scalars, sizeof(s)) != 0) return false;
    if (std::memcmp(in.qo_indptr, qo_indptr.data(), qo_indptr.size() * sizeof(int32_t)) != 0) return false;
    if (std::memcmp(in.kv_indptr, kv_indptr.data(), kv_indptr.size() * sizeof(int32_t)) != 0) return false;
    if (!(in.flags & kFlagRagged)) {
      if (!in.kv_last_page_len || last.size() != static_cast<size_t>(B)) return false;
      if (std::memcmp(in.kv_last_page_len, last.data(), last.size() * sizeof(int32_t)) != 0) return false;
    }
    return true;
  }
};

// The last size query's plan on this thread (not for mixed batches, whose
// sub-batch images carry their own copies of the page ids).
thread_local bool g_cached = false;
thread_local PlanKey g_cache_key;
thread_local Planned g_cache_plan;

}  // namespace

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

PlanInput make_input(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* kv_last_page_len, int32_t batch, int32_t nnz_pages, int32_t num_pages,
                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t causal, uint32_t flags, bool check_indices) {
  PlanInput in;
  in.qo_indptr = qo_indptr;
  in.kv_indptr = kv_indptr;
  in.kv_indices = kv_indices;
  in.kv_last_page_len = kv_last_page_len;
  in.batch = batch;
  in.nnz_pages = nnz_pages;
  in.num_pages = num_pages;
  in.num_qo_heads = num_qo_heads;
  in.num_kv_heads = num_kv_heads;
  in.head_dim = head_dim;
  in.page_size = page_size;
  in.causal = causal;
  in.flags = flags;
  in.check_indices = check_indices;
  in.kv_chunk_override = env_int("PKA_KV_CHUNK");
  in.prefill_cus_override = env_int("PKA_PREFILL_CUS");
  return in;
}

int plan_or_error(const PlanInput& in, Planned* res) {
  if (in.flags & ~kKnownFlags) return set_error(PKA_ERR_INVALID_ARG, "unknown flag bits");
  std::string err;
  const int st = build_mixed_plan(in, &res->mp, &err);
  if (st != kOk) return set_error(st, err);
  return PKA_OK;
}

int plan_for_create(const PlanInput& in, Planned* res) {
  if (g_cached && g_cache_key.same(in)) {
    g_cached = false;
    Planned pl = std::move(g_cache_plan);
    if (!(in.flags & kFlagRagged)) {
      if (in.nnz_pages != in.kv_indptr[in.batch])
        return set_error(PKA_ERR_INVALID_ARG, "kv_indptr[batch] = " + std::to_string(in.kv_indptr[in.batch]) +
                                                  " but nnz_pages = " + std::to_string(in.nnz_pages));
      std::string err;
      const int st = check_page_ids(in.kv_indices, in.nnz_pages, in.num_pages, &err);
      if (st != kOk) return set_error(st, err);
      std::vector<int32_t>& im = pl.mp.single.image;
      if (in.nnz_pages > 0)
        std::memcpy(im.data() + im[kHdrOffIndices], in.kv_indices, static_cast<size_t>(in.nnz_pages) * sizeof(int32_t));
      if (pl.mp.mixed) {
        // Each sub-image holds the page ids of its own requests (prefill:
        // qo_len > 1, decode: qo_len == 1), request after request, at its
        // indices section; the two sit at their offsets in the mixed image.
        auto fill = [&](int32_t off, bool prefill_side) {
          int32_t* sub = pl.mp.image.data() + off;
          int32_t* dst = sub + sub[kHdrOffIndices];
          for (int32_t r = 0; r < in.batch; ++r) {
            const int32_t n = in.qo_indptr[r + 1] - in.qo_indptr[r];
            if (prefill_side ? n > 1 : n == 1) {
              const int32_t a = in.kv_indptr[r], b = in.kv_indptr[r + 1];
              if (b > a) std::memcpy(dst, in.kv_indices + a, static_cast<size_t>(b - a) * sizeof(int32_t));
              dst += b - a;
            }
          }
        };
        fill(pl.mp.off_prefill, true);
        fill(pl.mp.off_decode, false);
      }
    }
    *res = std::move(pl);
    return PKA_OK;
  }
  return plan_or_error(in, res);
}

void fill_plan_info(const Planned& pl, int32_t batch, int32_t nnz, pka_plan_info* info) {
  const MixedPlan& mp = pl.mp;
  fill_info(mp.single, batch, nnz, info);  // totals of the whole batch
  info->prefill_cus = info->decode_cus = 0;
  if (!mp.mixed) return;
  const PlanResult& a = mp.prefill;
  const PlanResult& b = mp.decode;
  info->kernel = PKA_KERNEL_MIXED;
  info->num_units = a.num_units + b.num_units;
  info->num_merge_groups = a.num_merge + b.num_merge;
  info->num_partial_rows = a.num_partial_rows + b.num_partial_rows;
  info->block_rows = a.block_rows;
  info->kv_chunk = b.kv_chunk;
  info->int_ws_bytes = static_cast<int64_t>(mp.image.size() * sizeof(int32_t));
  info->float_ws_bytes = static_cast<int64_t>(mp.float_ws_bytes);
  // one grid: the same workgroups serve both images
  info->num_workers = mp.one_grid ? a.num_workers : a.num_workers + b.num_workers;
  info->num_queues = a.num_queues + b.num_queues;
  info->prefill_cus = mp.prefill_cus;
  info->decode_cus = mp.decode_cus;
}

int cascade_layout(int32_t num_levels, const int32_t* const* qo_indptr, const int32_t* const* kv_indptr,
                   const int32_t* const* kv_indices, const int32_t* const* kv_last_page_len, const int32_t* batch,
                   const int32_t* nnz_pages, int32_t num_pages, int32_t num_qo_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t page_size, int32_t causal, uint32_t flags, CascadeLayout* out) {
  if (num_levels < 1 || num_levels > 64) return set_error(PKA_ERR_INVALID_ARG, "cascade: num_levels must be in [1, 64]");
  if (!qo_indptr || !kv_indptr || !kv_last_page_len || !batch)
    return set_error(PKA_ERR_INVALID_ARG, "cascade: level arrays must not be NULL");
  if (flags & ~kCascadeFlags)
    return set_error(PKA_ERR_INVALID_ARG, "cascade: only PKA_OUT_FP32 and PKA_DISABLE_SPLIT_KV are accepted");
  *out = CascadeLayout{};
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t ioff = 0, foff = 0;
  for (int l = 0; l < num_levels; ++l) {
    if (!qo_indptr[l] || !kv_indptr[l] || batch[l] < 0)
      return set_error(PKA_ERR_INVALID_ARG, "cascade: level " + std::to_string(l) + " has a NULL array");
    const int32_t nnz = kv_indptr[l][batch[l]];
    if (nnz_pages && nnz_pages[l] != nnz)
      return set_error(PKA_ERR_INVALID_ARG, "cascade: level " + std::to_string(l) + ": kv_indptr[batch] = " +
                                                std::to_string(nnz) + " but nnz_pages = " + std::to_string(nnz_pages[l]));
    // Only the last level is causally masked: the keys of the earlier
    // levels precede every query of their groups.
    const uint32_t lflags = (flags & PKA_DISABLE_SPLIT_KV) | kCascadeLevelFlags;
    PlanInput in = make_input(qo_indptr[l], kv_indptr[l], kv_indices ? kv_indices[l] : nullptr, kv_last_page_len[l],
                              batch[l], nnz, num_pages, num_qo_heads, num_kv_heads, head_dim, page_size,
                              (causal && l == num_levels - 1) ? 1 : 0, lflags, kv_indices != nullptr);
    Planned pl;
    const int st = plan_or_error(in, &pl);
    if (st != PKA_OK) return set_error(st, "cascade: level " + std::to_string(l) + ": " + pka_last_error());
    if (causal && l == num_levels - 1) {
      // The earlier levels' keys precede every query, so the causal mask of
      // the whole concatenation is the last level's own bottom-right mask
      // only if each of its groups holds at least its own query rows.
      for (int32_t g = 0; g < batch[l]; ++g) {
        const int64_t pages = kv_indptr[l][g + 1] - kv_indptr[l][g];
        const int64_t keys = pages == 0 ? 0 : (pages - 1) * page_size + kv_last_page_len[l][g];
        const int64_t rows = qo_indptr[l][g + 1] - qo_indptr[l][g];
        if (keys < rows)
          return set_error(PKA_ERR_INVALID_ARG, "cascade: last level, group " + std::to_string(g) + " has " +
                                                    std::to_string(keys) + " keys for " + std::to_string(rows) +
                                                    " causal query rows");
      }
    }
    const int64_t tq = qo_indptr[l][batch[l]];
    if (l == 0) out->total_q = tq;
    else if (tq != out->total_q)
      return set_error(PKA_ERR_INVALID_ARG, "cascade: level " + std::to_string(l) + " covers " + std::to_string(tq) +
                                                " query rows, level 0 covers " + std::to_string(out->total_q));
    out->int_off.push_back(ioff);
    out->int_bytes.push_back(pl.image().size() * sizeof(int32_t));
    out->float_off.push_back(foff);
    out->float_bytes.push_back(pl.float_ws_bytes());
    ioff = align(ioff + out->int_bytes.back());
    foff = align(foff + out->float_bytes.back());
  }
  const size_t rows = static_cast<size_t>(out->total_q) * num_qo_heads;
  out->states_v = foff;
  out->states_s = align(foff + static_cast<size_t>(num_levels) * rows * head_dim * sizeof(float));
  out->float_total = align(out->states_s + static_cast<size_t>(num_levels) * rows * sizeof(float));
  out->int_total = ioff;
  return PKA_OK;
}

}  // namespace pka

extern "C" {

int pka_cascade_workspace_size(int32_t num_levels, const int32_t* const* qo_indptr, const int32_t* const* kv_indptr,
                               const int32_t* const* kv_last_page_len, const int32_t* batch, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                               uint32_t flags, size_t* int_ws_bytes, size_t* float_ws_bytes) {
  try {
    if (!int_ws_bytes || !float_ws_bytes) return pka::set_error(PKA_ERR_INVALID_ARG, "null size pointer");
    pka::CascadeLayout lay;
    const int st = pka::cascade_layout(num_levels, qo_indptr, kv_indptr, nullptr, kv_last_page_len, batch, nullptr, 0,
                                       num_qo_heads, num_kv_heads, head_dim, page_size, causal, flags, &lay);
    if (st != PKA_OK) return st;
    *int_ws_bytes = lay.int_total;
    *float_ws_bytes = lay.float_total;
    return PKA_OK;
  } catch (const std::exception& ex) {
    return pka::set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

const char* pka_last_error(void) { return pka::g_last_error.c_str(); }

int pka_plan_workspace_size(const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                            uint32_t flags, size_t* int_ws_bytes, size_t* float_ws_bytes) {
  try {
    if (!int_ws_bytes || !float_ws_bytes) return pka::set_error(PKA_ERR_INVALID_ARG, "null size pointer");
    if (!kv_indptr || batch < 0) return pka::set_error(PKA_ERR_INVALID_ARG, "kv_indptr must not be NULL");
    const int32_t nnz = kv_indptr[batch];
    pka::PlanInput in = pka::make_input(qo_indptr, kv_indptr, nullptr, kv_last_page_len, batch, nnz, 0,
                                        num_qo_heads, num_kv_heads, head_dim, page_size, causal, flags, false);
    pka::g_cached = false;
    pka::Planned res;
    const int st = pka::plan_or_error(in, &res);
    if (st != PKA_OK) return st;
    *int_ws_bytes = res.image().size() * sizeof(int32_t);
    *float_ws_bytes = res.float_ws_bytes();
    {
      pka::g_cache_key = pka::PlanKey::of(in);
      pka::g_cache_plan = std::move(res);
      pka::g_cached = true;
    }
    return PKA_OK;
  } catch (const std::exception& ex) {
    return pka::set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

int pka_plan_host_image(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                        const int32_t* kv_last_page_len, int32_t batch, int32_t nnz_pages,
                        int32_t num_pages_in_pool, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, int32_t causal, uint32_t flags, void* image,
                        size_t image_bytes, pka_plan_info* info) {
  try {
    pka::PlanInput in = pka::make_input(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch, nnz_pages,
                                        num_pages_in_pool, num_qo_heads, num_kv_heads, head_dim, page_size,
                                        causal, flags, true);
    pka::Planned res;
    const int st = pka::plan_or_error(in, &res);
    if (st != PKA_OK) return st;
    if (info) pka::fill_plan_info(res, batch, (flags & PKA_RAGGED_KV) ? 0 : nnz_pages, info);
    const size_t need = res.image().size() * sizeof(int32_t);
    if (image) {
      if (image_bytes < need) return pka::set_error(PKA_ERR_WORKSPACE, "image buffer too small");
      std::memcpy(image, res.image().data(), need);
    }
    return PKA_OK;
  } catch (const std::exception& ex) {
    return pka::set_error(PKA_ERR_INVALID_ARG, ex.what());
  }
}

}  // extern "C"
