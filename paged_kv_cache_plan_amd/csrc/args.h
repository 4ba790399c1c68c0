// Kernel argument blocks shared by the host launchers and the kernels.
#pragma once

#include <cstdint>

namespace pka {

// Arguments of the attention kernels (prefill and decode).  Element offsets
// count bf16 elements.
struct AttnArgs {
  const uint16_t* q;         // bf16 [total_q, Hq, D]
  // K row of (page or token p, slot s, KV head h): k + p * page_stride +
  // s * row_stride + h * head_stride, D contiguous elements; V rows at the
  // same offsets from v.  Ragged: p is the token row and s = 0.
  const uint16_t* k;
  const uint16_t* v;
  void* o;                   // bf16 or fp32 [total_q, Hq, D]
  float* lse;                // fp32 [total_q, Hq] or null
  float* part_o;             // float workspace: partial O [rows, D], then partial lse
  int32_t* ws;               // int workspace: the plan image (sections found via its header)
  int64_t page_stride;       // elements between pages (ragged: between tokens)
  int64_t head_stride;       // elements between KV heads
  int32_t row_stride;        // elements between consecutive slots of a page
  int32_t num_qo_heads;
  int32_t group;             // Hq / Hkv
  int32_t page_size;
  int32_t page_shift;        // log2(page_size) when a power of two, else -1
  int32_t out_fp32;
  float scale_log2;          // sm_scale * log2(e): logits in base-2 units
};

// Arguments of the split-KV merge that follows an attention launch.
struct MergeArgs {
  const float* part_o;       // float workspace (partial lse found via the image header)
  const int32_t* ws;         // int workspace: the plan image
  void* o;
  float* lse;
  int32_t num_qo_heads;
  int32_t group;
  int32_t out_fp32;
};

// Arguments of the standalone merge of attention states.  State s of row i,
// head h: v + i * v_row_stride + s * v_state_stride + h * D (D floats) and
// s + i * s_row_stride + s * s_state_stride + h; by default [n, S, H, D] and
// [n, S, H].
struct MergeStatesArgs {
  const float* v;
  const float* s;
  int64_t v_row_stride;
  int64_t v_state_stride;
  int64_t s_row_stride;
  int64_t s_state_stride;
  void* v_out;               // [n, H, D]
  float* s_out;              // [n, H] or null
  int64_t n;
  int32_t num_states;
  int32_t num_heads;
  int32_t head_dim;
  int32_t out_fp32;
};

// Arguments of the test-only page gather.
struct GatherArgs {
  const uint16_t* pool;
  uint16_t* k_out;
  uint16_t* v_out;
  const int32_t* req;
  const int32_t* kv_indices;
  int64_t page_stride;
  int64_t v_offset;
  int32_t row_stride;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t head_dim;
};

// Arguments of get_batch_indices_positions.
struct BatchPosArgs {
  const int32_t* append_indptr;  // [batch + 1]
  const int32_t* seq_lens;       // [batch], KV lengths after the append
  int32_t* batch_indices;        // [nnz]
  int32_t* positions;            // [nnz]
  int32_t batch;
  int32_t nnz;
};

// Arguments of the paged-KV append.  Element offsets count bf16 elements.
struct AppendArgs {
  const uint16_t* append_k;      // [nnz, Hkv, D]
  const uint16_t* append_v;      // [nnz, Hkv, D]
  const int32_t* batch_indices;  // [nnz]
  const int32_t* positions;      // [nnz]
  uint16_t* paged_kv;            // [num_pages, 2, ps, Hkv, D]
  const int32_t* kv_indices;     // [kv_indptr[batch]]
  const int32_t* kv_indptr;      // [batch + 1]
  int32_t nnz;
  int32_t batch;
  int32_t num_pages;
  int32_t page_size;
  int32_t page_shift;            // log2(page_size) when a power of two, else -1
  int32_t row_elems;             // Hkv * D
};

}  // namespace pka
