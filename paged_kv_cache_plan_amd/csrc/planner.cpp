// Host planner: validation, kv_len, tiling, split-KV and ordering of work units.
#include "planner.h"

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <numeric>

namespace pka {
namespace {

int fail(std::string* err, int code, const char* fmt, long long a = 0, long long b = 0,
         long long c = 0) {
  char buf[512];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  if (err) *err = buf;
  return code;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int32_t align_words(int64_t w) { return static_cast<int32_t>(ceil_div(w, 64) * 64); }

struct Unit {
  int32_t f[kUnitWords];
  int64_t cost;  // keys processed, the ordering key
  int32_t seq;   // creation order, the tie-break that keeps ordering deterministic
};

}  // namespace

int check_page_ids(const int32_t* kv_indices, int32_t nnz, int32_t num_pages, std::string* err) {
  if (nnz > 0 && !kv_indices) return fail(err, kInvalid, "kv_indices must not be NULL");
  if (num_pages <= 0 && nnz > 0)
    return fail(err, kInvalid, "num_pages_in_pool must be positive (got %lld)", num_pages);
  for (int32_t i = 0; i < nnz; ++i) {
    const int32_t p = kv_indices[i];
    if (p < 0 || p >= num_pages)
      return fail(err, kInvalid, "kv_indices[%lld] = %lld is outside [0, %lld)", i, p, num_pages);
  }
  return kOk;
}

int build_plan(const PlanInput& in, PlanResult* out, std::string* err) {
  const bool ragged = (in.flags & kFlagRagged) != 0;
  const int B = in.batch;
  if (B < 0) return fail(err, kInvalid, "batch must be >= 0 (got %lld)", B);
  if (!in.qo_indptr || !in.kv_indptr) return fail(err, kInvalid, "qo_indptr and kv_indptr must not be NULL");
  if (!ragged && B > 0 && !in.kv_last_page_len)
    return fail(err, kInvalid, "kv_last_page_len must not be NULL for a paged KV cache");
  if (in.num_qo_heads <= 0 || in.num_kv_heads <= 0)
    return fail(err, kInvalid, "head counts must be positive (Hq=%lld, Hkv=%lld)", in.num_qo_heads,
                in.num_kv_heads);
  if (in.num_qo_heads % in.num_kv_heads != 0)
    return fail(err, kUnsupported, "num_qo_heads (%lld) must be a multiple of num_kv_heads (%lld)",
                in.num_qo_heads, in.num_kv_heads);
  if (in.head_dim != 64 && in.head_dim != 128)
    return fail(err, kUnsupported, "head_dim %lld is not supported (64 or 128)", in.head_dim);
  const int ps = ragged ? 1 : in.page_size;
  if (!ragged && (ps < 1 || ps > 128))
    return fail(err, kUnsupported, "page_size %lld is outside [1, 128]", ps);
  const int G = in.num_qo_heads / in.num_kv_heads;
  const int Hkv = in.num_kv_heads;

  if (in.qo_indptr[0] != 0) return fail(err, kInvalid, "qo_indptr[0] must be 0 (got %lld)", in.qo_indptr[0]);
  if (in.kv_indptr[0] != 0) return fail(err, kInvalid, "kv_indptr[0] must be 0 (got %lld)", in.kv_indptr[0]);
  for (int r = 0; r < B; ++r) {
    if (in.qo_indptr[r + 1] < in.qo_indptr[r])
      return fail(err, kInvalid, "qo_indptr decreases at %lld (%lld -> %lld)", r, in.qo_indptr[r],
                  in.qo_indptr[r + 1]);
    if (in.kv_indptr[r + 1] < in.kv_indptr[r])
      return fail(err, kInvalid, "kv_indptr decreases at %lld (%lld -> %lld)", r, in.kv_indptr[r],
                  in.kv_indptr[r + 1]);
  }
  const int32_t nnz = in.kv_indptr[B];
  if (!ragged) {
    if (in.nnz_pages != nnz)
      return fail(err, kInvalid, "kv_indptr[batch] = %lld but nnz_pages = %lld", nnz, in.nnz_pages);
    if (in.check_indices) {
      const int st = check_page_ids(in.kv_indices, nnz, in.num_pages, err);
      if (st != kOk) return st;
    }
  }

  // kv_len per request: every page but the last is full.
  std::vector<int64_t> kv_len(B), qo_len(B);
  int64_t total_kv = 0;
  int32_t max_qo = 0;
  for (int r = 0; r < B; ++r) {
    qo_len[r] = in.qo_indptr[r + 1] - in.qo_indptr[r];
    max_qo = std::max<int32_t>(max_qo, static_cast<int32_t>(qo_len[r]));
    const int64_t span = in.kv_indptr[r + 1] - in.kv_indptr[r];
    if (ragged) {
      kv_len[r] = span;
    } else {
      const int32_t last = in.kv_last_page_len[r];
      if (span == 0) {
        if (last != 0)
          return fail(err, kInvalid, "request %lld has no pages but kv_last_page_len = %lld", r, last);
        kv_len[r] = 0;
      } else {
        if (last < 1 || last > ps)
          return fail(err, kInvalid, "kv_last_page_len[%lld] = %lld is outside [1, page_size=%lld]", r,
                      last, ps);
        kv_len[r] = (span - 1) * ps + last;
      }
    }
    if (kv_len[r] > (int64_t(1) << 30)) return fail(err, kUnsupported, "request %lld: kv_len too large", r);
    if (qo_len[r] * G > (int64_t(1) << 30)) return fail(err, kUnsupported, "request %lld: qo_len too large", r);
    total_kv += kv_len[r];
  }

  const bool no_split = (in.flags & kFlagDisableSplit) != 0;
  const bool decode = B > 0 && max_qo <= 1 && G <= kDecodeMaxGroup;

  std::vector<Unit> units;
  // one entry per (request, kv head, row block): the KV range before splitting
  struct Block { int32_t r, hk, row0, row1; int64_t kv_hi; };
  std::vector<Block> blocks;
  int32_t block_rows;
  if (decode) {
    block_rows = G;
    for (int r = 0; r < B; ++r) {
      if (qo_len[r] == 0) continue;
      for (int hk = 0; hk < Hkv; ++hk) blocks.push_back({r, hk, 0, G, kv_len[r]});
    }
  } else {
    block_rows = prefill_block_rows(in.head_dim);
    for (int r = 0; r < B; ++r) {
      if (qo_len[r] == 0) continue;
      const int64_t rows = qo_len[r] * G;
      for (int hk = 0; hk < Hkv; ++hk) {
        for (int64_t r0 = 0; r0 < rows; r0 += block_rows) {
          const int64_t r1 = std::min<int64_t>(rows, r0 + block_rows);
          int64_t hi = kv_len[r];
          if (in.causal) {
            const int64_t last_tok = (r1 - 1) / G;  // bottom-right: sees j <= i + kv_len - qo_len
            hi = std::min<int64_t>(hi, last_tok + kv_len[r] - qo_len[r] + 1);
            hi = std::max<int64_t>(hi, 0);
          }
          blocks.push_back({r, hk, static_cast<int32_t>(r0), static_cast<int32_t>(r1), hi});
        }
      }
    }
  }

  // Split-KV policy.  Decode: cut long KV into chunks so that the launch has
  // several units per compute unit.  Prefill: only when the batch has too few
  // row blocks to fill the chip.
  int64_t chunk = 0;
  if (!no_split && !blocks.empty()) {
    if (decode) {
      int64_t keys = 0;
      for (const Block& b : blocks) keys += b.kv_hi;
      chunk = ceil_div(keys, int64_t(in.num_cus) * 8);
      // (measured on the batch-decode workload: 2048-key chunks stream at
      // 5.77 TB/s, 6144-16384-key chunks at 5.95-5.98 TB/s, unsplit 4.60)
      chunk = std::min<int64_t>(16384, std::max<int64_t>(256, ceil_div(chunk, 128) * 128));
    } else if (static_cast<int64_t>(blocks.size()) < 2 * in.num_cus) {
      int64_t tiles = 0;
      for (const Block& b : blocks) tiles += ceil_div(b.kv_hi, kPrefillBlockKeys);
      const int64_t chunk_tiles = std::max<int64_t>(8, ceil_div(tiles, 4 * int64_t(in.num_cus)));
      chunk = chunk_tiles * kPrefillBlockKeys;
    }
    if (in.kv_chunk_override > 0) {
      const int64_t q = decode ? kDecodeTileKeys : kPrefillBlockKeys;
      chunk = std::max<int64_t>(q, ceil_div(in.kv_chunk_override, q) * q);
    }
  }

  std::vector<int32_t> merge;
  int64_t partial_rows = 0;
  int32_t max_merge_rows = 0;
  bool any_split = false;
  for (const Block& b : blocks) {
    const int64_t n_split = (chunk > 0 && b.kv_hi > chunk) ? ceil_div(b.kv_hi, chunk) : 1;
    const int32_t nrows = b.row1 - b.row0;
    int64_t pbase = -1;
    if (n_split > 1) {
      any_split = true;
      pbase = partial_rows;
      partial_rows += n_split * nrows;
      if (partial_rows > (int64_t(1) << 30)) return fail(err, kUnsupported, "too many partial rows");
      merge.insert(merge.end(), {b.r, b.hk, b.row0, b.row1, static_cast<int32_t>(pbase),
                                 static_cast<int32_t>(n_split), 0, 0});
      max_merge_rows = std::max(max_merge_rows, nrows);
    }
    for (int64_t s = 0; s < n_split; ++s) {
      Unit u{};
      const int64_t lo = n_split > 1 ? s * chunk : 0;
      const int64_t hi = n_split > 1 ? std::min<int64_t>(b.kv_hi, lo + chunk) : b.kv_hi;
      u.f[kUnitRequest] = b.r;
      u.f[kUnitKvHead] = b.hk;
      u.f[kUnitRowBegin] = b.row0;
      u.f[kUnitRowEnd] = b.row1;
      u.f[kUnitKvBegin] = static_cast<int32_t>(lo);
      u.f[kUnitKvEnd] = static_cast<int32_t>(hi);
      u.f[kUnitPartialRow] = n_split > 1 ? static_cast<int32_t>(pbase + s * nrows) : -1;
      u.f[kUnitReserved] = 0;
      u.f[kUnitQoBegin] = in.qo_begin ? in.qo_begin[b.r] : in.qo_indptr[b.r];
      u.f[kUnitQoLen] = static_cast<int32_t>(qo_len[b.r]);
      u.f[kUnitKvBase] = (ragged && in.kv_begin) ? in.kv_begin[b.r] : in.kv_indptr[b.r];
      u.f[kUnitKvLen] = static_cast<int32_t>(kv_len[b.r]);
      u.cost = (hi - lo) * nrows + 1;
      u.seq = static_cast<int32_t>(units.size());
      units.push_back(u);
    }
  }
  if (units.size() > size_t(1) << 30) return fail(err, kUnsupported, "too many work units");

  auto longest_first = [](const Unit& a, const Unit& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    return a.seq < b.seq;
  };
  // Queues: queue_begin[q] .. queue_begin[q + 1] index the unit array.
  const bool fixed = (in.flags & kFlagGraphStable) != 0;
  // Workgroups per CU the launch is planned (and, at D=64, built) for: three
  // for D=64 batches of long units, by their mean key range times the group
  // size (kPrefillLongUnitKeys).
  int wgs = decode ? kDecodeWgPerCu : prefill_wg_per_cu(in.head_dim);
  if (!decode && in.head_dim == 64 && !fixed && in.workers_override <= 0 && !in.qo_begin && !units.empty()) {
    int64_t keys = 0;
    for (const Unit& u : units) keys += u.f[kUnitKvEnd] - u.f[kUnitKvBegin];
    if (keys * G >= kPrefillLongUnitKeys * static_cast<int64_t>(units.size())) wgs = kPrefillWgPerCuLong64;
  }
  std::vector<int32_t> queue_begin{0};
  if (decode) {
    // One queue, longest first: big units start first and small ones fill
    // the tail.  Decode reads each K/V byte once, so there is no L2 reuse to
    // keep on one XCD.
    std::stable_sort(units.begin(), units.end(), longest_first);
    queue_begin.push_back(static_cast<int32_t>(units.size()));
  } else if (in.num_xcds <= 1 || (!fixed && units.size() <= static_cast<size_t>(in.num_xcds))) {
    std::stable_sort(units.begin(), units.end(), longest_first);
    queue_begin.push_back(static_cast<int32_t>(units.size()));
  } else {
    // The units of one (request, kv head) read the same K/V, so keep them in
    // one queue, served by the workgroups of one XCD (workgroup b runs on XCD
    // b % num_xcds), for reuse in that XCD's L2.  Groups go longest-first to
    // the least loaded queue; a queue runs its groups in that order, taking
    // them in windows of kQueueWindow groups whose units run longest-first,
    // so a group's units run side by side and long units start early.
    struct Grp { int64_t cost; size_t first, count; };
    std::vector<Grp> grps;
    for (size_t i = 0; i < units.size();) {
      size_t j = i;
      int64_t c = 0;
      while (j < units.size() && units[j].f[kUnitRequest] == units[i].f[kUnitRequest] &&
             units[j].f[kUnitKvHead] == units[i].f[kUnitKvHead]) {
        c += units[j].cost;
        ++j;
      }
      grps.push_back({c, i, j - i});
      i = j;
    }
    std::vector<size_t> order(grps.size());
    std::iota(order.begin(), order.end(), size_t(0));
    std::stable_sort(order.begin(), order.end(),
                     [&](size_t a, size_t b) { return grps[a].cost > grps[b].cost; });
    const int X = in.num_xcds;
    std::vector<std::vector<Unit>> queue(X);
    std::vector<int64_t> load(X, 0);
    std::vector<int32_t> groups_in(X, 0);
    std::vector<size_t> window_start(X, 0);
    for (size_t gi : order) {
      int x = 0;
      for (int k = 1; k < X; ++k)
        if (load[k] < load[x]) x = k;
      load[x] += grps[gi].cost;
      std::vector<Unit>& q = queue[x];
      if (groups_in[x]++ % kQueueWindow == 0) window_start[x] = q.size();
      q.insert(q.end(), units.begin() + grps[gi].first, units.begin() + grps[gi].first + grps[gi].count);
      // stable, by cost only: equal costs keep group order, then planning order
      std::stable_sort(q.begin() + window_start[x], q.end(),
                       [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    }
    // The last units a queue hands out (twice as many as it can have
    // workers) run longest-first across groups, so that its workers finish
    // together; this costs some L2 reuse at the end.
    const int64_t slots_per_queue =
        std::max<int64_t>(1, int64_t(std::max(1, in.num_cus)) * wgs / X);
    const size_t tail = static_cast<size_t>(kQueueTailSlots * slots_per_queue);
    for (int x = 0; x < X; ++x) {
      std::vector<Unit>& q = queue[x];
      const size_t t0 = q.size() > tail ? q.size() - tail : 0;
      std::stable_sort(q.begin() + t0, q.end(), [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    }
    std::vector<Unit> out;
    out.reserve(units.size());
    for (int x = 0; x < X; ++x) {
      out.insert(out.end(), queue[x].begin(), queue[x].end());
      queue_begin.push_back(static_cast<int32_t>(out.size()));
    }
    units.swap(out);
  }
  // Workers: at most one per resident slot.  With kFlagGraphStable the
  // count does not depend on the batch (queues may be empty).
  const int32_t n_queues = static_cast<int32_t>(queue_begin.size()) - 1;
  int64_t longest = 0;
  for (int q = 0; q < n_queues; ++q) longest = std::max<int64_t>(longest, queue_begin[q + 1] - queue_begin[q]);
  const int64_t slots = in.workers_override > 0 ? int64_t(in.workers_override) : int64_t(std::max(1, in.num_cus)) * wgs;
  const int64_t per_queue_max = std::max<int64_t>(1, slots / n_queues);
  const int32_t workers_per_queue = static_cast<int32_t>(
      (fixed || in.workers_override > 0) ? per_queue_max
                                         : std::max<int64_t>(1, std::min<int64_t>(longest, per_queue_max)));
  const int32_t n_workers = n_queues * workers_per_queue;

  // Assemble the image.
  const int32_t n_units = static_cast<int32_t>(units.size());
  const int32_t n_merge = static_cast<int32_t>(merge.size() / kMergeWords);
  const int32_t off_units = align_words(kHdrWords);
  const int32_t off_req = off_units + align_words(int64_t(n_units) * kUnitWords);
  const int32_t off_merge = off_req + align_words(int64_t(B) * kReqWords);
  const int32_t off_sched = off_merge + align_words(int64_t(n_merge) * kMergeWords);
  const int32_t off_idx = off_sched + align_words(int64_t(n_queues) * kSchedWords);
  const int64_t n_idx = ragged ? 0 : nnz;
  const int64_t total_words = off_idx + align_words(std::max<int64_t>(n_idx, 1));
  out->image.assign(static_cast<size_t>(total_words), 0);
  int32_t* im = out->image.data();
  im[kHdrMagic] = kMagic;
  im[kHdrKernel] = decode ? kDecode : kPrefill;
  im[kHdrNumUnits] = n_units;
  im[kHdrNumMerge] = n_merge;
  im[kHdrBatch] = B;
  im[kHdrNnz] = ragged ? 0 : nnz;
  im[kHdrOffUnits] = off_units;
  im[kHdrOffReq] = off_req;
  im[kHdrOffMerge] = off_merge;
  im[kHdrOffIndices] = off_idx;
  im[kHdrNumPartialRows] = static_cast<int32_t>(partial_rows);
  im[kHdrBlockRows] = block_rows;
  im[kHdrKvChunk] = any_split ? static_cast<int32_t>(chunk) : 0;
  im[kHdrFlags] = static_cast<int32_t>(in.flags);
  im[kHdrOffSched] = off_sched;
  im[kHdrNumQueues] = n_queues;
  im[kHdrNumWorkers] = n_workers;
  im[kHdrMergeSlices] = merge_slices(max_merge_rows, in.head_dim);
  for (int32_t q = 0; q < n_queues; ++q) {
    int32_t* rec = im + off_sched + int64_t(q) * kSchedWords;
    rec[kSchedBegin] = queue_begin[q];
    rec[kSchedEnd] = queue_begin[q + 1];
    rec[kSchedWorkers] = workers_per_queue;
  }
  for (int32_t i = 0; i < n_units; ++i)
    std::memcpy(im + off_units + int64_t(i) * kUnitWords, units[i].f, sizeof(units[i].f));
  int64_t dense = 0;
  for (int r = 0; r < B; ++r) {
    int32_t* q = im + off_req + int64_t(r) * kReqWords;
    q[kReqQoBegin] = in.qo_begin ? in.qo_begin[r] : in.qo_indptr[r];
    q[kReqQoLen] = static_cast<int32_t>(qo_len[r]);
    q[kReqKvBegin] = (ragged && in.kv_begin) ? in.kv_begin[r] : in.kv_indptr[r];
    q[kReqKvLen] = static_cast<int32_t>(kv_len[r]);
    q[kReqKvDense] = static_cast<int32_t>(dense);
    dense += kv_len[r];
  }
  if (dense > (int64_t(1) << 31) - 1) return fail(err, kUnsupported, "total kv length too large");
  if (n_merge) std::memcpy(im + off_merge, merge.data(), merge.size() * sizeof(int32_t));
  if (n_idx && in.kv_indices) std::memcpy(im + off_idx, in.kv_indices, size_t(n_idx) * sizeof(int32_t));

  out->kernel = decode ? kDecode : kPrefill;
  out->num_units = n_units;
  out->num_merge = n_merge;
  out->num_partial_rows = static_cast<int32_t>(partial_rows);
  out->block_rows = block_rows;
  out->kv_chunk = any_split ? static_cast<int32_t>(chunk) : 0;
  out->num_queues = n_queues;
  out->num_workers = n_workers;
  out->wg_per_cu = wgs;
  out->total_q = in.qo_indptr[B];
  out->total_kv = total_kv;
  const size_t o_bytes = static_cast<size_t>(partial_rows) * in.head_dim * sizeof(float);
  out->partial_lse_offset = (o_bytes + 255) / 256 * 256;
  if (out->partial_lse_offset / sizeof(float) >= (size_t(1) << 31))
    return fail(err, kUnsupported, "too many partial rows");
  out->image[kHdrPartialLse] = static_cast<int32_t>(out->partial_lse_offset / sizeof(float));
  out->float_ws_bytes = out->partial_lse_offset +
                        (static_cast<size_t>(partial_rows) * sizeof(float) + 255) / 256 * 256;
  if (out->float_ws_bytes == 0) out->float_ws_bytes = 256;
  return kOk;
}

int32_t mixed_prefill_cus(double prefill_flop, double decode_bytes, int32_t num_cus, int32_t num_xcds) {
  const int32_t step = std::max(1, num_xcds);
  int32_t best = step;
  double best_t = -1.0;
  for (int32_t p = step; p + step <= num_cus; p += step) {
    const double tp = prefill_flop / (kPrefillFlopPerCuNs * p);
    const double td = decode_bytes / std::min(kDecodeBytePerNs, kDecodeBytePerCuNs * (num_cus - p));
    const double t = std::max(tp, td);
    if (best_t < 0.0 || t <= best_t) {
      best_t = t;
      best = p;
    }
  }
  return best;
}

int build_mixed_plan(const PlanInput& in, MixedPlan* out, std::string* err) {
  *out = MixedPlan{};
  // The whole batch is always planned first: it validates every array, with
  // the batch's own request numbers in the messages.
  PlanInput whole = in;
  whole.flags &= ~(kFlagMixed | kFlagMixedTwoLaunches);
  if ((in.flags & kFlagMixedTwoLaunches) && !(in.flags & kFlagMixed))
    return fail(err, kInvalid, "the two-launch flag needs the mixed-batch flag");
  int st = build_plan(whole, &out->single, err);
  if (st != kOk || !(in.flags & kFlagMixed)) return st;
  if (in.flags & kFlagGraphStable)
    return fail(err, kUnsupported, "a mixed-batch plan cannot be graph-stable");
  const int B = in.batch;
  const bool ragged = (in.flags & kFlagRagged) != 0;
  const int G = in.num_qo_heads / in.num_kv_heads;
  std::vector<int> pre, dec;
  for (int r = 0; r < B; ++r) {
    const int32_t n = in.qo_indptr[r + 1] - in.qo_indptr[r];
    if (n > 1) pre.push_back(r);
    else if (n == 1) dec.push_back(r);
  }
  if (pre.empty() || dec.empty() || G > kDecodeMaxGroup) return kOk;  // one kind: the whole-batch plan

  // Sub-batch inputs: indptr arrays over the subset, offsets of the whole batch.
  struct Sub {
    std::vector<int32_t> qo_indptr{0}, kv_indptr{0}, kv_indices, last, qo_begin, kv_begin;
  };
  auto make = [&](const std::vector<int>& rs, Sub* sb, PlanInput* pi) {
    for (int r : rs) {
      sb->qo_indptr.push_back(sb->qo_indptr.back() + (in.qo_indptr[r + 1] - in.qo_indptr[r]));
      sb->kv_indptr.push_back(sb->kv_indptr.back() + (in.kv_indptr[r + 1] - in.kv_indptr[r]));
      if (!ragged && in.kv_indices)
        sb->kv_indices.insert(sb->kv_indices.end(), in.kv_indices + in.kv_indptr[r],
                              in.kv_indices + in.kv_indptr[r + 1]);
      if (!ragged) sb->last.push_back(in.kv_last_page_len[r]);
      sb->qo_begin.push_back(in.qo_indptr[r]);
      sb->kv_begin.push_back(in.kv_indptr[r]);
    }
    *pi = whole;
    pi->qo_indptr = sb->qo_indptr.data();
    pi->kv_indptr = sb->kv_indptr.data();
    pi->kv_indices = (!ragged && in.kv_indices) ? sb->kv_indices.data() : nullptr;
    pi->kv_last_page_len = ragged ? nullptr : sb->last.data();
    pi->batch = static_cast<int32_t>(rs.size());
    pi->nnz_pages = ragged ? 0 : sb->kv_indptr.back();
    pi->qo_begin = sb->qo_begin.data();
    pi->kv_begin = sb->kv_begin.data();
  };
  Sub sp, sd;
  PlanInput ip, id;
  make(pre, &sp, &ip);
  make(dec, &sd, &id);

  // The compute-unit split, from the algorithmic work of each side.
  auto kv_len_of = [&](int r) -> int64_t {
    const int64_t span = in.kv_indptr[r + 1] - in.kv_indptr[r];
    if (ragged) return span;
    return span == 0 ? 0 : (span - 1) * in.page_size + in.kv_last_page_len[r];
  };
  double flop = 0.0, bytes = 0.0;
  for (int r : pre) {
    const int64_t n = in.qo_indptr[r + 1] - in.qo_indptr[r], kv = kv_len_of(r);
    double pairs = 0.0;  // visible (query, key) pairs
    for (int64_t i = 0; i < n; ++i) {
      const int64_t lim = in.causal ? std::min<int64_t>(kv, i + kv - n + 1) : kv;
      pairs += static_cast<double>(std::max<int64_t>(0, lim));
    }
    flop += 4.0 * in.head_dim * in.num_qo_heads * pairs;
  }
  for (int r : dec) bytes += 4.0 * in.num_kv_heads * in.head_dim * static_cast<double>(kv_len_of(r));
  int32_t pcus = in.prefill_cus_override > 0 ? in.prefill_cus_override
                                             : mixed_prefill_cus(flop, bytes, in.num_cus, in.num_xcds);
  pcus = std::max(1, std::min(pcus, in.num_cus - 1));
  if (!(in.flags & kFlagMixedTwoLaunches)) {
    // One launch: both sides planned for the whole chip; the decode side
    // gets exactly as many workers as the prefill side ended with (its one
    // queue then has every workgroup of the launch).
    ip.num_cus = id.num_cus = in.num_cus;
    ip.workers_override = std::max(1, in.num_cus) * prefill_wg_per_cu(in.head_dim);
    st = build_plan(ip, &out->prefill, err);
    if (st != kOk) return st;
    id.workers_override = out->prefill.num_workers;
    st = build_plan(id, &out->decode, err);
    if (st != kOk) return st;
    if (out->decode.num_workers != out->prefill.num_workers)
      return fail(err, kUnsupported, "one-grid mixed plan: worker counts differ");
    out->one_grid = true;
    // the cost model's split decides which workgroups start with decode
    out->prefill_cus = pcus;
    out->decode_cus = in.num_cus - pcus;
    out->xcds = std::max(1, in.num_xcds);
    out->decode_first_slots = (in.num_cus - pcus) / out->xcds * prefill_wg_per_cu(in.head_dim);
  } else {
    ip.num_cus = pcus;
    id.num_cus = in.num_cus - pcus;
    st = build_plan(ip, &out->prefill, err);
    if (st != kOk) return st;
    st = build_plan(id, &out->decode, err);
    if (st != kOk) return st;
    out->prefill_cus = pcus;
    out->decode_cus = in.num_cus - pcus;
  }
  out->mixed = true;
  out->off_prefill = kMixWords;
  out->off_decode = out->off_prefill + align_words(static_cast<int64_t>(out->prefill.image.size()));
  out->float_off_decode = (out->prefill.float_ws_bytes + 255) / 256 * 256;
  out->float_ws_bytes = out->float_off_decode + out->decode.float_ws_bytes;
  out->image.assign(static_cast<size_t>(out->off_decode) + out->decode.image.size(), 0);
  int32_t* im = out->image.data();
  im[kMixMagic] = kMixedMagic;
  im[kMixKernel] = kMixed;
  im[kMixOffPrefill] = out->off_prefill;
  im[kMixOffDecode] = out->off_decode;
  im[kMixFloatOffDecode] = static_cast<int32_t>(out->float_off_decode / sizeof(float));
  im[kMixPrefillCus] = out->prefill_cus;
  im[kMixDecodeCus] = out->decode_cus;
  im[kMixBatch] = B;
  im[kMixNnz] = ragged ? 0 : in.kv_indptr[B];
  im[kMixOneGrid] = out->one_grid ? 1 : 0;
  im[kMixDecodeFirstSlots] = out->decode_first_slots;
  std::memcpy(im + out->off_prefill, out->prefill.image.data(), out->prefill.image.size() * sizeof(int32_t));
  std::memcpy(im + out->off_decode, out->decode.image.data(), out->decode.image.size() * sizeof(int32_t));
  return kOk;
}

}  // namespace pka
