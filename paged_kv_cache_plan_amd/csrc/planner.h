// Host planner for batch attention over a paged KV cache.  Plain C++17 with
// no HIP dependency, so it builds and runs on a machine without a GPU.
//
// It turns the flat page table (flashinfer-trace discussion #15, "Notes on
// fa3_gqa_prefill_v1": kv_indptr / kv_indices / kv_last_page_len) and the
// ragged query layout into fixed-size integer work arrays that the kernels
// read.  Planning from host arrays, with the result shipped to the device by
// one asynchronous copy, follows the FlashInfer 0.2 release blog ("faster plan
// function").  Whether to split one request's KV over several work units is a
// plan-time choice that a flag can switch off (flashinfer-trace discussion
// #15, table of tunable runtime knobs: disable_split_kv).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace pka {

// Layout of the int workspace image (int32 words).  Every section starts on a
// 64-word (256-byte) boundary.
enum HeaderField : int {
  kHdrMagic = 0,
  kHdrKernel,
  kHdrNumUnits,
  kHdrNumMerge,
  kHdrBatch,
  kHdrNnz,
  kHdrOffUnits,
  kHdrOffReq,
  kHdrOffMerge,
  kHdrOffIndices,
  kHdrNumPartialRows,
  kHdrBlockRows,
  kHdrKvChunk,
  kHdrFlags,
  kHdrOffSched,     // per-queue scheduling records (see SchedField)
  kHdrNumQueues,    // number of unit queues
  kHdrNumWorkers,   // workgroups of the attention launch
  kHdrPartialLse,   // float index of the partial lse section in the float workspace
  kHdrMergeSlices,  // slices the split merge cuts the largest merge group into (>= 1)
  kHdrWords = 32
};
constexpr int32_t kMagic = 0x31414b50;  // "PKA1"

// One work unit = one workgroup of the attention launch.  Words 8-11 copy
// the request's fields, so that a kernel starting a unit waits for one
// record load instead of two dependent ones.
enum UnitField : int {
  kUnitRequest = 0,
  kUnitKvHead,
  kUnitRowBegin,  // packed row = token * group + head-in-group, within the request
  kUnitRowEnd,
  kUnitKvBegin,   // first key (token index within the request)
  kUnitKvEnd,     // one past the last key
  kUnitPartialRow,  // -1: write o/lse; otherwise first fp32 partial row
  kUnitReserved,
  kUnitQoBegin,   // = the request's kReqQoBegin
  kUnitQoLen,     // = kReqQoLen
  kUnitKvBase,    // = kReqKvBegin
  kUnitKvLen,     // = kReqKvLen
  kUnitWords = 16
};

// Per-request facts the kernels need.
enum ReqField : int {
  kReqQoBegin = 0,
  kReqQoLen,
  kReqKvBegin,   // paged: offset into kv_indices; ragged: first token row of k/v
  kReqKvLen,
  kReqKvDense,   // first row of this request in a dense [total_kv, ...] copy
  kReqWords = 8
};

// A split group: one (request, kv head, row block) whose KV was cut into
// num_splits chunks; chunk s wrote partial rows
// partial_row_begin + s * (row_end - row_begin) + (row - row_begin).
enum MergeField : int {
  kMergeRequest = 0,
  kMergeKvHead,
  kMergeRowBegin,
  kMergeRowEnd,
  kMergePartialBegin,
  kMergeNumSplits,
  kMergeWords = 8
};

// Attention runs as a persistent launch: kHdrNumWorkers workgroups, worker b
// serving queue b % kHdrNumQueues (prefill: one queue per XCD; decode: one).
// The kernels find every section and count through this header, so a launch
// whose grid does not depend on the batch can be replayed after the image
// has been replaced by another batch's.  Queue q owns units [begin, end) of the
// unit array; a worker takes the next unit with an atomic increment of the
// queue's counter.  Decode: the last worker of the queue to finish sets both
// counters back to zero.  Prefill: a worker whose queue is empty goes on to
// the other queues, and the launch's last worker to finish (counted in queue
// 0's done counter) sets every queue's counters back to zero.  Either way the
// next run of the plan starts from a clean state without a clearing launch.
// One 64-word record per queue; the two counters sit on their own 128-byte
// line, apart from the read-only fields.
enum SchedField : int {
  kSchedNext = 0,     // counter: units taken from this queue
  kSchedDone = 1,     // counter: workers done (prefill: of the launch, on queue 0)
  kSchedBegin = 32,
  kSchedEnd,
  kSchedWorkers,      // workers serving this queue
  kSchedWords = 64
};

enum Kernel : int { kPrefill = 0, kDecode = 1, kMixed = 2 };

// Tile shapes the kernels are built for.
constexpr int kPrefillBlockKeys = 64;   // keys per prefill KV tile
constexpr int kDecodeTileKeys = 32;     // keys per decode wave step
constexpr int kDecodeMaxGroup = 16;     // decode kernel holds up to 16 query heads per KV head
constexpr int kDecodeWgPerCu = 2;       // resident decode workgroups per CU (persistent launch)
constexpr int kMergeGrid = 1024;        // split-merge workgroups of a batch-independent launch
constexpr int kMergeBlock = 256;        // split merge: items (row, 4 d) per workgroup pass
constexpr int kMergeSlicesMax = 32;     // split merge: at most this many workgroups per group

// Slices of a merge group of `rows` rows: whole kMergeBlock blocks of its
// rows * head_dim / 4 items, at most kMergeSlicesMax.
constexpr int32_t merge_slices(int64_t rows, int32_t head_dim) {
  return static_cast<int32_t>(
      rows <= 0 ? 1
                : ((rows * (head_dim / 4) + kMergeBlock - 1) / kMergeBlock < kMergeSlicesMax
                       ? (rows * (head_dim / 4) + kMergeBlock - 1) / kMergeBlock
                       : kMergeSlicesMax));
}
constexpr int kQueueWindow = 2;         // prefill queue: groups per longest-first window
constexpr int kQueueTailSlots = 2;      // prefill queue: tail run longest-first, per worker slot

constexpr uint32_t kFlagDisableSplit = 0x1u;
constexpr uint32_t kFlagOutFp32 = 0x2u;
constexpr uint32_t kFlagRagged = 0x4u;
constexpr uint32_t kFlagGraphStable = 0x8u;  // launch shapes that do not depend on the batch
constexpr uint32_t kFlagMixed = 0x10u;       // prefill and decode requests together, in one launch
constexpr uint32_t kFlagMixedTwoLaunches = 0x20u;  // with kFlagMixed: two launches on a compute-unit split

enum Status : int { kOk = 0, kInvalid = 1, kUnsupported = 2, kWorkspace = 3, kHip = 4 };

struct PlanInput {
  const int32_t* qo_indptr = nullptr;
  const int32_t* kv_indptr = nullptr;
  const int32_t* kv_indices = nullptr;  // may be null when only sizes are wanted
  const int32_t* kv_last_page_len = nullptr;
  int32_t batch = 0;
  int32_t nnz_pages = 0;
  int32_t num_pages = 0;
  int32_t num_qo_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t page_size = 0;
  int32_t causal = 0;
  uint32_t flags = 0;
  bool check_indices = true;   // validate kv_indices (needs the array)
  int32_t kv_chunk_override = 0;  // >0: keys per split chunk (tuning); 0: heuristic
  int32_t num_cus = 256;          // compute units the split heuristic aims to fill
  int32_t num_xcds = 8;           // XCDs workgroups are dealt to round-robin (prefill order)
  // Optional per-request overrides of where a request's rows and (ragged) K/V
  // rows start, used for the sub-batches of a mixed plan: they keep the
  // offsets of the whole batch while the indptr arrays describe the subset.
  const int32_t* qo_begin = nullptr;
  const int32_t* kv_begin = nullptr;
  int32_t prefill_cus_override = 0;  // >0: compute units of a mixed plan's prefill launch (tuning)
  // >0: exactly this many workers, the same number for every queue (a
  // launch whose workgroups also serve another plan's queues)
  int32_t workers_override = 0;
};

// Prefill workgroup shape per head_dim: 32 packed query rows per wave, 8
// waves (256 rows, one resident workgroup per CU) at D=128 and 4 waves (128
// rows, two per CU) at D=64.  The kernel is built with the matching thread
// count and launch bound.
constexpr int prefill_waves(int head_dim) { return head_dim == 128 ? 8 : 4; }
constexpr int prefill_block_rows(int head_dim) { return 32 * prefill_waves(head_dim); }
constexpr int prefill_wg_per_cu(int head_dim) { return head_dim == 128 ? 1 : 2; }
// At D=64 a batch whose units average at least kPrefillLongUnitKeys keys
// times the group size (query heads per KV head: the rows that share each
// K/V tile) is planned for three workgroups per CU, run by a build of the
// kernel whose launch bound caps it at 168 VGPRs; other batches keep two
// (that build loses more to its register cap there than the third workgroup
// brings).  Graph-stable plans and the sub-plans of a mixed batch keep two.
constexpr int kPrefillWgPerCuLong64 = 3;
constexpr int64_t kPrefillLongUnitKeys = 2048;

struct PlanResult {
  int32_t kernel = kPrefill;
  int32_t num_units = 0;
  int32_t num_merge = 0;
  int32_t num_partial_rows = 0;
  int32_t block_rows = 0;
  int32_t kv_chunk = 0;
  int32_t num_queues = 0;   // prefill only
  int32_t num_workers = 0;  // workgroups of the attention launch
  int32_t wg_per_cu = 0;    // prefill: workgroups per CU the launch is planned (and built) for
  int64_t total_q = 0;
  int64_t total_kv = 0;
  std::vector<int32_t> image;  // the int workspace image
  size_t float_ws_bytes = 0;
  size_t partial_lse_offset = 0;  // byte offset of partial lse inside the float workspace
};

// Validate and plan.  Returns a Status and fills *err on failure.
int build_plan(const PlanInput& in, PlanResult* out, std::string* err);

// Every page id of kv_indices[0, nnz) lies in [0, num_pages) (kv_indices may
// be null only when nnz == 0).  The only use build_plan makes of kv_indices
// and num_pages besides copying the ids into the image's index section.
int check_page_ids(const int32_t* kv_indices, int32_t nnz, int32_t num_pages, std::string* err);

// A mixed batch (kFlagMixed with both prefill requests, qo_len > 1, and
// decode requests, qo_len == 1) is planned as two images, each over its own
// requests as an ordinary batch.  By default both run in one persistent
// launch: the images are planned for the whole chip and the same number of
// workers, and every workgroup serves both, one kind after the other.  The
// workgroups of decode_cus compute units (from the cost model below) start
// with the decode queue, the others with the prefill queues; a workgroup
// whose first kind runs out of units moves on to the other kind's queues,
// so the split adjusts itself to the speeds met.  With kFlagMixedTwoLaunches
// they run as two persistent launches side by side instead: the prefill
// kernel on prefill_cus compute units and the decode kernel on the rest.  The int workspace holds a 64-word header, then the
// prefill image, then the decode image; the float workspace holds the
// prefill partial states, then the decode ones.
enum MixedField : int {
  kMixMagic = 0,
  kMixKernel,          // kMixed
  kMixOffPrefill,      // word offset of the prefill image
  kMixOffDecode,       // word offset of the decode image
  kMixFloatOffDecode,  // float offset of the decode partial states
  kMixPrefillCus,
  kMixDecodeCus,
  kMixBatch,
  kMixNnz,
  kMixOneGrid,  // 1: one launch serves both images (its workgroup count: each image's workers)
  kMixDecodeFirstSlots,  // one grid: workgroup slots per XCD that start with the decode queue
  kMixWords = 64
};
constexpr int32_t kMixedMagic = 0x4d414b50;  // "PKAM"

// Rates the compute-unit split is sized with, measured on MI355X with the
// kernels here: the prefill kernel retires about kPrefillFlopPerCuNs flop per
// ns per compute unit; the decode kernel streams about kDecodeBytePerCuNs
// bytes per ns per compute unit and kDecodeBytePerNs in all.
constexpr double kPrefillFlopPerCuNs = 3500.0;
constexpr double kDecodeBytePerCuNs = 30.0;
constexpr double kDecodeBytePerNs = 6300.0;

struct MixedPlan {
  bool mixed = false;      // false: `single` is the whole plan
  PlanResult single;       // the plan of the whole batch (always built: it validates)
  PlanResult prefill, decode;
  int32_t prefill_cus = 0, decode_cus = 0;
  bool one_grid = false;  // one launch (not kFlagMixedTwoLaunches): prefill.num_workers == decode.num_workers
  // one grid: workgroup b starts with the decode queue when b / xcds < decode_first_slots
  int32_t xcds = 0, decode_first_slots = 0;
  int32_t off_prefill = 0, off_decode = 0;  // words
  size_t float_off_decode = 0;              // bytes
  std::vector<int32_t> image;               // mixed: header + both images
  size_t float_ws_bytes = 0;
};

// Compute units for the prefill launch of a mixed batch: the multiple of
// num_xcds that minimises the later of the two launches' ends under the
// rates above (ties: more prefill units).
int32_t mixed_prefill_cus(double prefill_flop, double decode_bytes, int32_t num_cus, int32_t num_xcds);

// Plan a batch, as two sub-batches when in.flags has kFlagMixed and the
// batch mixes both kinds of request (else as build_plan does).
int build_mixed_plan(const PlanInput& in, MixedPlan* out, std::string* err);

}  // namespace pka
