/*
 * pka.h - batch attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * The operation (FlashInfer 0.2 release blog, "flexible block sparsity and
 * vector sparsity"): PageAttention is block-sparse attention whose block
 * width is page_size; page_size = 1 is per-token (vector) sparsity.  For each
 * request r of a ragged batch, the query rows q[qo_indptr[r] .. qo_indptr[r+1])
 * attend over the request's kv_len keys, read through a flat page table
 * (flashinfer-trace discussion #15, "Notes on fa3_gqa_prefill_v1":
 * kv_indices + kv_indptr + kv_last_page_len; Q ragged as
 * [total_q, num_qo_heads, head_dim]).  Every call returns O and a base-2
 * log-sum-exp (same passage), and states of disjoint KV parts merge into the
 * state of the whole (FlashInfer documentation, "Attention States and
 * Recursive Attention", "Merge Attention States").
 *
 * Semantics fixed by this library where the pages are silent:
 *   kv_len      = (npages - 1) * page_size + kv_last_page_len[r], 0 if npages == 0.
 *   GQA         query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *   causal      bottom-right: query i sees key j iff j <= i + kv_len - qo_len.
 *   s_j         = sm_scale * q . k_j,  sm_scale <= 0 selects 1/sqrt(head_dim).
 *   lse         = log2 sum_j exp(s_j) over the visible keys.
 *   no key      a row that sees no key gets o = 0 and lse = -inf.
 *
 * Layouts (all row-major, contiguous):
 *   q           bf16 [total_q, num_qo_heads, head_dim]
 *   paged_kv    bf16 [num_pages, 2, page_size, num_kv_heads, head_dim]  (NHD; 0 = K, 1 = V)
 *   k, v        bf16 [total_kv, num_kv_heads, head_dim]  (ragged dense form)
 *   o           bf16 (default) or fp32 (PKA_OUT_FP32) [total_q, num_qo_heads, head_dim]
 *   lse         fp32 [total_q, num_qo_heads]
 *
 * Plan / run split (FlashInfer 0.2 release blog, "faster plan function"): the
 * plan reads its index arrays from HOST memory, copies what the kernels need
 * into a caller-owned device workspace with an asynchronous host-to-device
 * copy on the caller's stream, and never waits for the device.  The copy
 * reads pinned staging buffers that the library keeps in a process-wide pool:
 * once the pool holds buffers of the sizes in use, creating, updating and
 * destroying plans allocates and frees no pinned memory (the first plans of a
 * process allocate it, which HIP may serialise with device work).  One plan
 * may be run many times (for instance once per layer) on any q / KV of the
 * planned shape.
 *
 * Errors: every int-returning call returns PKA_OK (0) or a PKA_ERR_* code and
 * records a message readable with pka_last_error() (per thread).  No call
 * aborts, and no C++ exception crosses this interface.
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (hipStream_t); NULL means the null stream. */
typedef struct ihipStream_t* pka_stream_t;

/* Opaque plan, owned by the library (pka_plan_destroy frees it). */
typedef struct pka_plan pka_plan;

/* Opaque multi-level cascade, owned by the library (pka_cascade_destroy frees it). */
typedef struct pka_cascade pka_cascade;

enum {
  PKA_OK = 0,
  PKA_ERR_INVALID_ARG = 1, /* malformed arrays, null pointers, mismatched plan  */
  PKA_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, Hq % Hkv != 0, page_size outside [1,128] */
  PKA_ERR_WORKSPACE = 3,   /* a workspace is smaller than pka_plan_workspace_size asks */
  PKA_ERR_HIP = 4          /* the HIP runtime reported an error (message has its text)    */
};

/* Plan flags. */
#define PKA_DISABLE_SPLIT_KV 0x1u /* never split one request's KV over several work units */
#define PKA_OUT_FP32 0x2u         /* o is fp32 instead of bf16                               */
#define PKA_RAGGED_KV 0x4u        /* K/V are ragged dense tensors: kv_indptr counts tokens,
                                     kv_indices and kv_last_page_len are unused (may be NULL),
                                     page_size is ignored; run with pka_run_ragged           */
#define PKA_GRAPH_STABLE 0x8u     /* every run enqueues the same launches whatever the batch, so
                                     a run captured into a HIP graph can be replayed after
                                     pka_plan_update has planned another batch into the same
                                     workspaces (FlashInfer 0.2 release blog, "CUDAGraph
                                     compatibility for variable-length inputs")              */
#define PKA_MIXED_BATCH 0x10u     /* a batch with both prefill requests (qo_len > 1) and decode
                                     requests (qo_len == 1) runs as one persistent launch whose
                                     workgroups serve both kinds, one after the other: those of
                                     the compute units that a cost model (the algorithmic work
                                     of each side) gives decode start with decode units, the
                                     others with prefill units, and whichever kind runs out
                                     first, its workgroups move on to the other.  (Prefill and
                                     decode in one kernel for chunked prefill: "[Roadmap]
                                     FlashInfer v0.2 to v0.3", milestone "POD-Attention
                                     Integration"; FlashInfer documentation contents,
                                     "flashinfer.pod".)  A batch of one kind plans as without
                                     the flag.  Not with PKA_GRAPH_STABLE; not for
                                     pka_debug_gather.                                          */
#define PKA_MIXED_TWO_LAUNCHES 0x20u /* with PKA_MIXED_BATCH: two persistent launches side by side
                                     instead of one: the prefill kernel on the compute units
                                     the cost model gives prefill and the decode kernel, on a
                                     side stream the plan holds (drawn from a library-wide
                                     pool), on the rest; the caller's stream waits for both
                                     (attention on a subset of the compute units: "[Roadmap]
                                     FlashInfer v0.2 to v0.3", milestone "Nanoflow
                                     Parallelism").  Without PKA_MIXED_BATCH it is an invalid
                                     argument.                                                 */

/* Which attention kernel a plan launches. */
enum { PKA_KERNEL_PREFILL = 0, PKA_KERNEL_DECODE = 1, PKA_KERNEL_MIXED = 2 };

/* Summary of a plan (all counts are exact for the planned batch). */
typedef struct pka_plan_info {
  int32_t kernel;           /* PKA_KERNEL_PREFILL, PKA_KERNEL_DECODE or PKA_KERNEL_MIXED  */
  int32_t num_units;        /* work units (decode: one workgroup each)                      */
  int32_t num_merge_groups; /* split (request, kv head, row block) groups merged afterwards */
  int32_t num_partial_rows; /* fp32 partial-state rows held in the float workspace          */
  int32_t block_rows;       /* packed query rows (token x group head) per work unit         */
  int32_t kv_chunk;         /* keys per split chunk, 0 when no unit is split                */
  int32_t batch;
  int32_t nnz_pages;
  int64_t total_q;
  int64_t total_kv;         /* sum of kv_len over the batch                                 */
  int64_t int_ws_bytes;     /* bytes of the int workspace image the plan uploads            */
  int64_t float_ws_bytes;   /* bytes of float workspace the runs need                       */
  int32_t num_workers;      /* workgroups of the persistent attention launch (prefill: each
                               takes units from its XCD's queue, then from the others; a
                               mixed batch in one launch: the workgroups serving both kinds) */
  int32_t num_queues;       /* unit queues: one per XCD for prefill, one for decode          */
  int32_t prefill_cus;      /* mixed batch: compute units whose workgroups start with prefill
                               units (two launches: the prefill launch's compute units)      */
  int32_t decode_cus;       /* mixed batch: compute units whose workgroups start with decode
                               units (two launches: the decode launch's compute units)       */
} pka_plan_info;

/* Message for the last failed call on this thread ("" if none). */
const char* pka_last_error(void);

/*
 * Workspace sizes for a plan of this batch, so that the caller can allocate
 * them before planning (FlashInfer 0.2 release blog, "CUDAGraph compatibility
 * for variable-length inputs": the workspaces a plan writes are sized up
 * front; a graph-stable caller sizes them once for its largest batch).  Pure
 * host call; reads host arrays qo_indptr[batch+1], kv_indptr[batch+1] and
 * (paged) kv_last_page_len[batch].  Writes the byte counts the two device
 * workspaces of pka_plan_create need for exactly this batch.  The work
 * decomposition it computes is kept (per thread) and reused by the next
 * pka_plan_create of the same batch on this thread, so that the pair plans
 * once.  Errors as pka_plan_create (except the page-id checks, which need
 * kv_indices).
 */
int pka_plan_workspace_size(const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_last_page_len, int32_t batch,
                            int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t causal, uint32_t flags,
                            size_t* int_ws_bytes, size_t* float_ws_bytes);

/*
 * Plan a batch.
 *   qo_indptr[batch+1], kv_indptr[batch+1], kv_indices[nnz_pages],
 *   kv_last_page_len[batch]: HOST int32 arrays, read during the call only.
 *   num_pages_in_pool: pages in paged_kv; every kv_indices entry must lie in
 *   [0, num_pages_in_pool).  Ids may repeat (shared read-only pages).
 *   int_ws / float_ws: caller-owned DEVICE buffers of at least the sizes
 *   pka_plan_workspace_size reports; they must stay valid, and be used by no
 *   other plan, while this plan is in use.
 *   stream: the plan's host-to-device copy is enqueued on it; a run on another
 *   stream must be ordered after it by the caller.
 *   *out receives a library-owned plan.  The pinned staging its copy reads
 *   is held by the plan until pka_plan_destroy, so the plan must outlive
 *   that copy.
 * PKA_ERR_WORKSPACE when a workspace is smaller than this batch needs; the
 * sizes are checked before anything is allocated or enqueued.
 * Validation (PKA_ERR_INVALID_ARG): indptr arrays start at 0 and never
 * decrease; kv_indptr[batch] == nnz_pages; for a request with pages,
 * 1 <= kv_last_page_len <= page_size, and 0 when it has none; ids in range.
 */
int pka_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len,
                    int32_t batch, int32_t nnz_pages, int32_t num_pages_in_pool,
                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t page_size, int32_t causal, float sm_scale, uint32_t flags,
                    void* int_ws, size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes,
                    pka_stream_t stream, pka_plan** out);

/* Counts and sizes of a plan. */
int pka_plan_get_info(const pka_plan* plan, pka_plan_info* info);

/*
 * Host-only planning: the same validation and work decomposition as
 * pka_plan_create, but the int workspace image is written to host memory
 * `image` (capacity image_bytes; NULL to query the size through info) instead
 * of being uploaded.  pka_plan_create uploads exactly these bytes.
 */
int pka_plan_host_image(const int32_t* qo_indptr, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const int32_t* kv_last_page_len,
                        int32_t batch, int32_t nnz_pages, int32_t num_pages_in_pool,
                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, int32_t causal, uint32_t flags,
                        void* image, size_t image_bytes, pka_plan_info* info);

/*
 * Attention over the paged KV cache (plan made without PKA_RAGGED_KV).
 * q, paged_kv, o, lse: caller-owned DEVICE memory in the layouts above; lse
 * may be NULL.  Enqueued on `stream` after the plan's copy; returns without
 * waiting.  The run writes every row of o and lse.
 */
int pka_run(const pka_plan* plan, const void* q, const void* paged_kv, void* o, float* lse,
            pka_stream_t stream);

/*
 * pka_run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, but the split-KV partial states go to a static
 * device scratch array of the library (64 MiB per GPU, held from the first
 * load of the library on that GPU until the process ends) instead of the
 * plan's float workspace, which this call never touches.  The call itself
 * allocates nothing.  Arguments, layouts and ownership as pka_run.
 * PKA_ERR_WORKSPACE when the plan's partial states (pka_plan_info
 * float_ws_bytes) exceed 64 MiB.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (on different streams, or from
 * several threads without ordering) race and give wrong results.
 */
int pka_run_noalloc(const pka_plan* plan, const void* q, const void* paged_kv, void* o, float* lse,
                    pka_stream_t stream);

/*
 * Attention over a paged KV cache stored with arbitrary strides (plan made
 * without PKA_RAGGED_KV): the HND page layout [num_pages, 2, Hkv, ps, D],
 * separate K and V pools, or pages spaced apart in a larger buffer
 * (FlashInfer documentation, "KV-Cache Layout in FlashInfer / Layout:
 * NHD/HND"; FlashInfer 0.2 release blog, "non-contiguous KV-cache").
 * The K row of (page, slot, KV head) starts at element
 *   k_cache + page * page_stride + slot * slot_stride + head * head_stride
 * and holds head_dim contiguous bf16; its V row is at the same offset from
 * v_cache.  Strides count bf16 elements and must be positive multiples of 8;
 * page_stride < 2^31, slot_stride < 2^24; k_cache and v_cache 16-byte
 * aligned (PKA_ERR_INVALID_ARG / PKA_ERR_UNSUPPORTED otherwise).  pka_run
 * is this call with page_stride = 2*ps*Hkv*D, slot_stride = Hkv*D,
 * head_stride = D and v_cache = k_cache + ps*Hkv*D.
 */
int pka_run_paged_strided(const pka_plan* plan, const void* q, const void* k_cache,
                          const void* v_cache, int64_t page_stride, int64_t slot_stride,
                          int64_t head_stride, void* o, float* lse, pka_stream_t stream);

/*
 * Attention over ragged dense K/V (plan made with PKA_RAGGED_KV): the dense
 * variable-length problem that paged attention with page_size = 1 must match
 * (FlashInfer 0.2 release blog, "performance benchmark": the vector-sparse
 * kernel is compared with dense variable-length attention on the same
 * inputs; "flexible block sparsity and vector sparsity": both run one kernel
 * that differs only in where K/V rows are read).  Request r's keys are rows
 * kv_indptr[r] .. kv_indptr[r+1]-1 of k and v, bf16 [total_kv, Hkv, D];
 * q, o, lse and errors as pka_run.
 */
int pka_run_ragged(const pka_plan* plan, const void* q, const void* k, const void* v, void* o,
                   float* lse, pka_stream_t stream);

/*
 * Merge attention states (FlashInfer documentation, "Merge Attention States").
 *   v   fp32 [n, num_states, num_heads, head_dim],  s fp32 [n, num_states, num_heads] (base 2)
 *   v_out bf16 (default) or fp32 (PKA_OUT_FP32) [n, num_heads, head_dim], s_out fp32 [n, num_heads]
 * With M = max_s s_s and w_s = 2^(s_s - M): s_out = M + log2 sum_s w_s and
 * v_out = sum_s w_s v_s / sum_s w_s; states with s = -inf weigh 0, and a row
 * whose states are all empty gets (0, -inf).  All pointers are device memory;
 * s_out may be NULL.  head_dim must be a multiple of 4 and at most 1024.
 */
int pka_merge_states(const float* v, const float* s, int64_t n, int32_t num_states,
                     int32_t num_heads, int32_t head_dim, void* v_out, float* s_out,
                     uint32_t flags, pka_stream_t stream);

/*
 * pka_merge_states over states at arbitrary strides (counted in floats):
 * state s of row i, head h is v[i*v_row_stride + s*v_state_stride + h*D ..]
 * and s[i*s_row_stride + s*s_state_stride + h].  Used by cascade attention,
 * whose levels write their states as [S, n, H, D] (FlashInfer documentation,
 * "flashinfer.cascade: Cascade Attention"; the merge is the one above).
 * v strides must be multiples of 4; v and v_out 16-byte aligned.
 */
int pka_merge_states_strided(const float* v, const float* s, int64_t n, int32_t num_states,
                             int32_t num_heads, int32_t head_dim, int64_t v_row_stride,
                             int64_t v_state_stride, int64_t s_row_stride, int64_t s_state_stride,
                             void* v_out, float* s_out, uint32_t flags, pka_stream_t stream);

/*
 * Test aid: copy the keys and values the page table selects into dense
 * k_dense / v_dense bf16 [total_kv, num_kv_heads, head_dim] (requests in
 * order, each kv_len rows), exactly as the attention kernels address them.
 */
int pka_debug_gather(const pka_plan* plan, const void* paged_kv, void* k_dense, void* v_dense,
                     pka_stream_t stream);

/*
 * Request and position of every appended token, for a per-element append
 * (FlashInfer 0.2 release blog, "KV-cache append optimisation":
 * get_batch_indices_positions).
 *   append_indptr [batch+1]: DEVICE int32; request r appends the tokens
 *     append_indptr[r] .. append_indptr[r+1]-1 of the appended tensors;
 *   seq_lens [batch]: DEVICE int32, each request's KV length AFTER the
 *     append; its n_r appended tokens are its last n_r tokens;
 *   nnz = append_indptr[batch], given by the caller;
 *   batch_indices, positions [nnz]: DEVICE int32 outputs, token i of
 *     request r getting r and seq_lens[r] - n_r + (i - append_indptr[r]).
 * Asynchronous on `stream`.  Null pointers or negative sizes ->
 * PKA_ERR_INVALID_ARG; the device arrays themselves are not validated.
 */
int pka_get_batch_indices_positions(const int32_t* append_indptr, const int32_t* seq_lens,
                                    int32_t batch, int32_t nnz, int32_t* batch_indices,
                                    int32_t* positions, pka_stream_t stream);

/*
 * Write appended K/V rows into the paged cache (FlashInfer documentation,
 * "flashinfer.page: Append new K/V tensors to Paged KV-Cache").
 *   append_k, append_v: DEVICE bf16 [nnz, num_kv_heads, head_dim];
 *   batch_indices, positions: DEVICE int32 [nnz] (see above);
 *   paged_kv: DEVICE bf16 [num_pages, 2, page_size, num_kv_heads, head_dim]
 *     (NHD; 0 = K, 1 = V), updated in place;
 *   kv_indptr [batch+1], kv_indices [kv_indptr[batch]]: DEVICE int32 page
 *     table already covering the lengths after the append.
 * Token i goes to page kv_indices[kv_indptr[b] + p / page_size], slot
 * p % page_size, with b = batch_indices[i], p = positions[i] -- the slot the
 * attention kernels read position p from.  A token whose b is outside
 * [0, batch), whose p is negative or past the request's pages, or whose page
 * id is outside [0, num_pages) is skipped: nothing is written for it.
 * Tokens that map to the same slot race.  head_dim must be 64 or 128 and
 * page_size in [1, 128] (PKA_ERR_UNSUPPORTED otherwise); the K/V tensors must
 * be 16-byte aligned (PKA_ERR_INVALID_ARG).  Asynchronous on `stream`.
 */
int pka_append_paged_kv(const void* append_k, const void* append_v, const int32_t* batch_indices,
                        const int32_t* positions, int32_t nnz, void* paged_kv, int32_t num_pages,
                        int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                        const int32_t* kv_indices, const int32_t* kv_indptr, int32_t batch,
                        pka_stream_t stream);

/*
 * Plan another batch into an existing plan's workspaces (same heads,
 * head_dim, page_size, pool, causal flag, sm_scale and flags; host arrays as
 * for pka_plan_create).  The new image is uploaded on `stream`; runs ordered
 * after it on that stream see the new batch, and a graph-stable plan's
 * captured runs replay it.  The call never waits for the device: it stages
 * the image in one of the plan's two pinned buffers whose previous copy has
 * completed (an event query), or in another buffer from the pool when both
 * are still being read.  The workspaces given at creation must be large
 * enough (PKA_ERR_WORKSPACE); a graph-stable plan cannot move between prefill
 * and decode batches (PKA_ERR_INVALID_ARG).
 */
int pka_plan_update(pka_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_indices, const int32_t* kv_last_page_len, int32_t batch,
                    int32_t nnz_pages, pka_stream_t stream);

/*
 * Cascade attention (FlashInfer documentation, "flashinfer.cascade: Cascade
 * Attention" and "Multi-level Cascade Inference Data Layout"): the query rows
 * of a batch attend to keys stored in num_levels levels.  Level l groups the
 * same total_q query rows into batch[l] contiguous groups (qo_indptr[l],
 * batch[l] + 1 entries) that share the keys of that level's flat page table
 * (kv_indptr[l], kv_indices[l], kv_last_page_len[l]; nnz_pages[l] ids), all
 * in one paged_kv pool.  A query attends to the concatenation of its groups'
 * keys, level 0 first, and the result equals attention over that
 * concatenation (the recursive-attention identity: FlashInfer documentation,
 * "Attention States and Recursive Attention").  Only the last level is
 * causally masked (bottom-right, when causal != 0): the keys of the earlier
 * levels precede every query of their groups, so each request's last-level
 * group must hold at least its own query tokens (a causal last-level group
 * with fewer keys than query rows is PKA_ERR_INVALID_ARG).
 *
 * Every level is planned like pka_plan_create (host arrays, validation,
 * split-KV unless PKA_DISABLE_SPLIT_KV) into its share of the two
 * caller-owned device workspaces; a run attends to each level into fp32
 * states held in the float workspace and merges them (pka_merge_states) into
 * o (bf16, or fp32 with PKA_OUT_FP32) and lse.  flags: PKA_OUT_FP32,
 * PKA_DISABLE_SPLIT_KV; anything else is PKA_ERR_INVALID_ARG.  All levels must
 * cover the same number of query rows (PKA_ERR_INVALID_ARG).
 * pka_cascade_workspace_size reports the two workspace sizes (pure host,
 * kv_indices not needed).  Ownership and stream rules are those of a plan:
 * the workspaces must outlive the cascade and its runs, and the caller must
 * make sure every run has completed before pka_cascade_destroy.  num_levels
 * is at most 64.
 */
int pka_cascade_workspace_size(int32_t num_levels, const int32_t* const* qo_indptr,
                               const int32_t* const* kv_indptr, const int32_t* const* kv_last_page_len,
                               const int32_t* batch, int32_t num_qo_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t page_size, int32_t causal, uint32_t flags,
                               size_t* int_ws_bytes, size_t* float_ws_bytes);

int pka_cascade_create(int32_t num_levels, const int32_t* const* qo_indptr,
                       const int32_t* const* kv_indptr, const int32_t* const* kv_indices,
                       const int32_t* const* kv_last_page_len, const int32_t* batch,
                       const int32_t* nnz_pages, int32_t num_pages_in_pool, int32_t num_qo_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                       float sm_scale, uint32_t flags, void* int_ws, size_t int_ws_bytes,
                       void* float_ws, size_t float_ws_bytes, pka_stream_t stream, pka_cascade** out);

/* Cascade attention of q bf16 [total_q, Hq, D] over paged_kv (layouts as
 * pka_run) into o and lse (lse may be NULL).  Asynchronous on `stream`. */
int pka_cascade_run(const pka_cascade* cascade, const void* q, const void* paged_kv, void* o,
                    float* lse, pka_stream_t stream);

/* Free a cascade and its level plans (NULL is a no-op). */
void pka_cascade_destroy(pka_cascade* cascade);

/* Free a plan.  The caller must first make sure every run using it has
 * completed (for example by synchronising the stream).  Its staging buffers
 * return to the library's pool with the events of their last copies (a
 * buffer is reused only once its copy has completed), so destroying a plan
 * frees no pinned memory and does not wait.  The side stream and events of a
 * PKA_MIXED_TWO_LAUNCHES plan go back to a library-wide pool in the same way
 * (creating a stream costs milliseconds).  NULL is a no-op. */
void pka_plan_destroy(pka_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* PKA_H */
