// Prefill / append attention over a paged (or ragged dense) KV cache, gfx950:
// the persistent workgroup's work (prefill_worker), used by the prefill kernel
// and by the one-grid mixed kernel.
//
// A work unit is (request r, KV head hk, block of packed query rows, key
// range [kv_lo, kv_hi)); a block is 32 rows per wave, 8 waves (256 rows) at
// D=128 and 4 waves (128 rows) at D=64.  Packed row p of a request is token
// p / G and query head hk * G + p % G, so the G query heads that share a KV
// head share every K/V tile the workgroup loads.  The launch is persistent:
// one workgroup per resident slot, each taking units from its XCD's queue
// and, once that is empty, from the other queues.
//
// PageAttention is block-sparse attention with page_size-wide blocks
// (FlashInfer 0.2 release blog, "flexible block sparsity and vector
// sparsity"), and the paged form differs from dense attention only in where
// the K/V rows are read from (same blog, "FlashAttention-3 template with
// block/vector sparsity": the gather sits in the producer's memory load).  The
// same holds here: the page-table lookup happens in the tile loader; the
// contraction and softmax code is shared by the paged and ragged variants.
//
// Per 64-key tile:
//   loader   each thread fetches KPT keys x one 16-byte chunk of K and V,
//            issued one tile ahead (page ids two tiles ahead); K goes to LDS
//            row-major in padded rows, V is transposed in registers and
//            stored as V^T so that the P.V operand is one 16-byte LDS read.
//   S^T      = K . Q^T with v_mfma_f32_32x32x16_bf16: each wave owns 32 query
//            rows as MFMA columns, so a lane holds 16 of a row's 32 scores per
//            32-key block and the other 16 sit in lane l ^ 32.
//   softmax  online, fp32, base 2 (sm_scale * log2 e folded into one FMA)
//            against a reference max that moves only when a tile's max
//            exceeds it by more than kSlack; each lane compares its half of
//            the row with a per-row bound, and the halves' max is exchanged
//            (v_permlane32_swap) only when some row moves.  The row sum adds
//            the bf16-rounded p that multiply V, two per v_dot2, and stays
//            per lane until the end.
//   O^T     += V^T . P^T with the same MFMA; P^T is the S^T accumulator
//            rounded to bf16 in place (no data movement), V^T comes from LDS.
#pragma once

#include "args.h"
#include "device.h"
#include "planner.h"

namespace pka {
namespace {

constexpr int kBN = 64;   // keys per tile
// Headroom (base-2 units) the running max may lag a row's true max by before
// O is rescaled (see the online softmax below).
constexpr float kSlack = 8.f;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// lo + hi of a packed bf16 pair, added to acc in fp32 (v_dot2c_f32_bf16 with 1.0).
__device__ __forceinline__ float sum_bf16x2(uint32_t x, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}
// Position of key k (0..63) of a tile inside a V^T row.  Within each group of
// 16 keys the order is 0-3, 8-11, 4-7, 12-15: exactly the key order in which
// a lane of the S^T accumulator holds its scores, so P^T needs no shuffle.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) + 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3);
}
// LDS layouts, chosen so that the MFMA operand reads are bank-conflict free
// for 16 lanes per LDS cycle.  K rows are padded by one 16-byte chunk (row
// stride D + 8 elements): 16 consecutive keys then start in 16 different
// chunk slots, and a lane's eight K reads differ only by immediate offsets.
// V^T rows (by d) use an XOR swizzle of their 16-byte chunks.
template <int D>
constexpr int k_stride() { return D + 8; }
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// How K/V rows are found: a dense ragged array, pages whose power-of-two size
// is at least one loader thread's run of keys (one page id per thread per
// tile), smaller power-of-two pages (one id per key, shifts and masks), or
// pages of any other size (one id per key, division).
enum KvMode : int { kKvRagged = 0, kKvPagedRun = 1, kKvPagedPow2 = 2, kKvPagedAny = 3 };

// What the kernel reads about one work unit; every field is wave-uniform.
struct UnitInfo {
  int r, hk, row_begin, row_end, kv_lo, kv_hi, prow;
  int qo_begin, qo_len, kv_base, kv_len;
};

__device__ __forceinline__ UnitInfo load_unit(const PlanView& pv, int ui) {
  const int32_t* u = pv.units + static_cast<int64_t>(ui) * kUnitWords;
  UnitInfo x;
  x.r = u[kUnitRequest];
  x.hk = u[kUnitKvHead];
  x.row_begin = u[kUnitRowBegin];
  x.row_end = u[kUnitRowEnd];
  x.kv_lo = u[kUnitKvBegin];
  x.kv_hi = u[kUnitKvEnd];
  x.prow = u[kUnitPartialRow];
  x.qo_begin = u[kUnitQoBegin];
  x.qo_len = u[kUnitQoLen];
  x.kv_base = u[kUnitKvBase];
  x.kv_len = u[kUnitKvLen];
  return x;
}

// The work of one persistent prefill workgroup: units from the plan's queues
// until every queue is empty.  The prefill kernel is this alone; the
// one-grid mixed kernel runs it and then the decode worker.
template <int D, int MODE, bool CAUSAL>
__device__ __forceinline__ void prefill_worker(const AttnArgs a) {
  constexpr int kThreads = 64 * prefill_waves(D);  // 32 packed query rows per wave
  constexpr bool PAGED = MODE != kKvRagged;
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int KPT = kBN * CPR / kThreads;  // keys per loader thread: 2
  constexpr int DS = D / 16;                 // k-steps of the S^T MFMA
  constexpr int DB = D / 32;                 // 32-row d blocks of O^T
  static_assert(KPT == 2 || KPT == 4, "tile shape");

  constexpr int KS = k_stride<D>();
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * kBN];
  __shared__ int s_unit[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int qcol = lane & 31, half = lane >> 5;  // this lane's query row (MFMA column) and half
  const int lc = tid % CPR;                      // loader: 16-byte chunk of the row
  const int lj = tid / CPR;                      // loader: keys KPT*lj .. KPT*lj + KPT-1
  const int G = a.group, Hq = a.num_qo_heads;
  const int ps = a.page_size, pshift = a.page_shift;
  // Byte offsets: a page's base is one 32x32 -> 64-bit multiply-add.
  const uint32_t page_bytes = static_cast<uint32_t>(a.page_stride) * 2u;
  const uint32_t row_bytes = static_cast<uint32_t>(a.row_stride) * 2u;
  // A power-of-two page_size >= KPT keeps a thread's KPT keys (KPT-aligned,
  // tiles start 64-aligned) in one page: one page id per thread per tile.
  constexpr bool one_page = MODE == kKvPagedRun;
  // With such pages the slot of a loader thread's first key is a lane part
  // (below) plus a tile part, since tiles start at multiples of 64 keys.
  // (opaque, so that the compiler does not fold the two parts' products
  // back into one multiply per tile)
  uint32_t lane_slot_bytes = 0;
  if constexpr (one_page) {
    lane_slot_bytes = static_cast<uint32_t>((KPT * lj) & (min(ps, kBN) - 1)) * row_bytes;
    asm volatile("" : "+v"(lane_slot_bytes));
  }
  // Single-key pages with KPT == 2: the two lanes of a pair load one page id
  // each and swap them with one DPP move.
  constexpr bool pair_ids = MODE == kKvPagedPow2 && KPT == 2;
  constexpr int NID = (one_page || pair_ids) ? 1 : KPT;
  constexpr bool pow2 = MODE != kKvPagedAny;

  // Persistent: the next unit is claimed during the current unit's last
  // tile, and its Q and first K/V tile are in flight while the current unit
  // writes its output.
  const PlanView pv = plan_view(a.ws);
  // A worker serves its own queue (one per XCD, whose units share K/V in
  // that XCD's L2) and, once it is empty, the other queues in turn, so that
  // no worker idles while units remain anywhere.  A claim gives a unit
  // index, or -1 once every queue has been found empty.
  const int n_queues = pv.num_queues;
  int q_cur = blockIdx.x % n_queues;  // (thread 0 only)
  int q_left = n_queues;
  auto claim = [&](int slot) {
    if (tid == 0) {
      int u = -1;
      while (q_left > 0) {
        int32_t* sq = pv.sched + q_cur * kSchedWords;
        const int v = sq[kSchedBegin] + __hip_atomic_fetch_add(sq + kSchedNext, 1, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
        if (v < sq[kSchedEnd]) {
          u = v;
          break;
        }
        --q_left;
        q_cur = q_cur + 1 == n_queues ? 0 : q_cur + 1;
      }
      s_unit[slot] = u;
    }
  };

  // ---- per-unit lane facts -----------------------------------------------
  struct Lane {
    int my_row, tok, head, lim;
    bool row_ok;
  };
  auto lane_of = [&](const UnitInfo& U) {
    Lane L;
    const int wrow0 = U.row_begin + wave * 32;
    L.my_row = wrow0 + qcol;
    L.row_ok = L.my_row < U.row_end;
    const int row = L.row_ok ? L.my_row : wrow0;
    L.tok = row / G;
    L.head = U.hk * G + (row - L.tok * G);
    L.lim = L.tok + U.kv_len - U.qo_len;  // last visible key (causal)
    return L;
  };

  // ---- loader ----------------------------------------------------------------
  u32x4 kreg[KPT], vreg[KPT];
  int ids_a[NID], ids_b[NID];
  bf16x8 qreg[DS];

  auto page_of = [&](int key) { return pow2 ? (key >> pshift) : (key / ps); };
  auto slot_of = [&](int key) { return pow2 ? (key & (ps - 1)) : (key - (key / ps) * ps); };
  // Keys past the unit's range (the last tile's tail) are read as the
  // range's last key: real, finite rows whose scores the mask removes, so
  // that no load needs a branch.  kv_hi > kv_lo wherever a tile is fetched.
  auto fetch_ids = [&](const UnitInfo& U, int k0, int* ids) {
    if constexpr (PAGED) {
      const int32_t* idx = pv.kv_indices + U.kv_base;
      const int key0 = k0 + KPT * lj, last = U.kv_hi - 1;
      if constexpr (one_page) {
        ids[0] = idx[min(key0, last) >> pshift];  // a clamped run stays in its page
      } else if constexpr (pair_ids) {
        ids[0] = idx[min(key0 + (lc & 1), last)];  // page_size 1: page = key
      } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) ids[i < NID ? i : 0] = idx[page_of(min(key0 + i, last))];
      }
    }
  };
  // byte offset of key's K row, given the page id
  auto row_off = [&](const UnitInfo& U, int key, int pid) -> uint64_t {
    if constexpr (PAGED) {
      return static_cast<uint64_t>(static_cast<uint32_t>(pid)) * page_bytes +
             static_cast<uint32_t>(slot_of(key)) * row_bytes;
    } else {
      return static_cast<uint64_t>(static_cast<uint32_t>(U.kv_base + key)) * page_bytes;
    }
  };
  auto fetch_data = [&](const UnitInfo& U, int k0, const int* ids_in) {
    int pair[2];
    const int* ids = ids_in;
    if constexpr (pair_ids) {
      // quad_perm [1, 0, 3, 2]: the partner lane's id (lanes 2m, 2m + 1 share lj)
      const int other = __builtin_amdgcn_mov_dpp(ids_in[0], 0xB1, 0xF, 0xF, true);
      pair[0] = (lc & 1) ? other : ids_in[0];
      pair[1] = (lc & 1) ? ids_in[0] : other;
      ids = pair;
    }
    const char* kbase = reinterpret_cast<const char*>(a.k + U.hk * a.head_stride + 8 * lc);
    const char* vbase = reinterpret_cast<const char*>(a.v + U.hk * a.head_stride + 8 * lc);
    const int key0 = k0 + KPT * lj;
    if (k0 + kBN <= U.kv_hi) {  // uniform: the whole tile is in range
      if constexpr (one_page) {
        const uint32_t slot_bytes = lane_slot_bytes + static_cast<uint32_t>(k0 & (ps - 1) & ~(kBN - 1)) * row_bytes;
        const uint64_t off0 = static_cast<uint64_t>(static_cast<uint32_t>(ids[0])) * page_bytes + slot_bytes;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          kreg[i] = *reinterpret_cast<const u32x4*>(kbase + off0 + i * row_bytes);
          vreg[i] = *reinterpret_cast<const u32x4*>(vbase + off0 + i * row_bytes);
        }
      } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const uint64_t off = row_off(U, key0 + i, ids[(i < NID || pair_ids) ? i : 0]);
          kreg[i] = *reinterpret_cast<const u32x4*>(kbase + off);
          vreg[i] = *reinterpret_cast<const u32x4*>(vbase + off);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint64_t off = row_off(U, min(key0 + i, U.kv_hi - 1), ids[one_page ? 0 : i]);  // pair_ids: ids = pair
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + off);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = KPT * lj + i;
      st16(Ks + key * KS + lc * 8, kreg[i]);
    }
    const int p0 = vt_pos(KPT * lj);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      uint16_t* dst = Vt + d * kBN + (((p0 >> 3) ^ vt_swz(d)) * 8) + (p0 & 7);
      const int w = e >> 1;
      if constexpr (KPT == 4) {
        u32x2 pk;
        pk[0] = (e & 1) ? pack_hi16(vreg[0][w], vreg[1][w]) : pack_lo16(vreg[0][w], vreg[1][w]);
        pk[1] = (e & 1) ? pack_hi16(vreg[2][w], vreg[3][w]) : pack_lo16(vreg[2][w], vreg[3][w]);
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) =
            (e & 1) ? pack_hi16(vreg[0][w], vreg[1][w]) : pack_lo16(vreg[0][w], vreg[1][w]);
      }
    }
  };
  // Q rows of the unit into the MFMA B operand, and its first K/V tile
  auto start_unit = [&](const UnitInfo& U) {
    const Lane L = lane_of(U);
    const uint16_t* qp = a.q + (static_cast<int64_t>(U.qo_begin + L.tok) * Hq + L.head) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = as_bf16x8(L.row_ok ? ld16(qp + 16 * s) : u32x4{0, 0, 0, 0});
    if (U.kv_hi > U.kv_lo) {
      fetch_ids(U, U.kv_lo, ids_a);
      fetch_data(U, U.kv_lo, ids_a);
      if (U.kv_lo + kBN < U.kv_hi) fetch_ids(U, U.kv_lo + kBN, ids_b);
    }
  };

  claim(0);
  __syncthreads();
  int ui = __builtin_amdgcn_readfirstlane(s_unit[0]);
  int slot = 0;
  UnitInfo U{};
  if (ui >= 0) {
    U = load_unit(pv, ui);
    start_unit(U);
  }

  while (ui >= 0) {
    const int lim = lane_of(U).lim;
    const int wrow0 = U.row_begin + wave * 32;
    const bool wave_active = wrow0 < U.row_end;
    const int wave_lim = wrow0 / G + U.kv_len - U.qo_len;  // smallest limit in the wave
    // keys any row of the wave can see end before wave_hi
    const int wave_hi =
        CAUSAL ? min(U.kv_hi, (min(wrow0 + 32, U.row_end) - 1) / G + U.kv_len - U.qo_len + 1) : U.kv_hi;
    const int kv_lo = U.kv_lo, kv_hi = U.kv_hi;

    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x16{};
    // per row (lane): the reference max m_run (base 2), -m_run for the
    // exponentials (0 before the row's first visible key), and thr, the raw
    // score above which the reference moves (sm_scale > 0)
    float m_run = -INFINITY, l_run = 0.f;
    float neg_m = 0.f, thr = -INFINITY;
    const float sl2 = a.scale_log2, inv_sl2 = 1.f / sl2;

    const int n_tiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kBN - 1) / kBN : 0;
    if (n_tiles == 0) {
      claim(slot ^ 1);
      __syncthreads();
    }
    for (int t = 0; t < n_tiles; ++t) {
      const int k0 = kv_lo + t * kBN;
      store_tile();
      __syncthreads();
      if (t + 1 < n_tiles) {
        fetch_data(U, k0 + kBN, ids_b);
        if (t + 2 < n_tiles) fetch_ids(U, k0 + 2 * kBN, ids_b);
      } else {
        claim(slot ^ 1);  // visible to all after this tile's closing barrier
      }

      if (wave_active && k0 < wave_hi) {  // tiles past every row of the wave are skipped
        // S^T = K . Q^T for two 32-key blocks.  The two blocks' accumulation
        // chains alternate so that consecutive MFMAs are independent, and the
        // K operands of step st + 1 are read while step st multiplies.
        f32x16 s[2] = {f32x16{}, f32x16{}};
        const uint16_t* kp = Ks + qcol * KS + half * 8;
        bf16x8 ka[2][2];
        ka[0][0] = as_bf16x8(ld16(kp));
        ka[0][1] = as_bf16x8(ld16(kp + 32 * KS));
#pragma unroll
        for (int st = 0; st < DS; ++st) {
          if (st + 1 < DS) {
            ka[(st + 1) & 1][0] = as_bf16x8(ld16(kp + (st + 1) * 16));
            ka[(st + 1) & 1][1] = as_bf16x8(ld16(kp + 32 * KS + (st + 1) * 16));
          }
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1][0], qreg[st], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1][1], qreg[st], s[1], 0, 0, 0);
        }
        // issue order: four K reads, then (two MFMAs, two K reads) per step,
        // so that two steps of operands are in flight
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int st = 0; st + 2 < DS; ++st) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
        // mask: keys past the unit's range, and (causal) keys past the row's
        // limit; lim_t = last visible key offset in this tile for the lane's row
        const bool need_mask = (k0 + kBN > kv_hi) || (CAUSAL && k0 + kBN - 1 > wave_lim);
        if (need_mask) {
          const int lim_t = (CAUSAL ? min(lim, kv_hi - 1) : kv_hi - 1) - k0 - 4 * half;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim_t) s[kb][i] = -INFINITY;
        }
        // online softmax in base 2: the max of this lane's half of the row
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        // The reference max moves only when this tile's max exceeds it by
        // more than kSlack (base-2 units): p then stays below 2^kSlack and
        // the O rescale below is rare after a row's first tile.  Either half
        // shows whether a row moves; the row max (lanes l and l ^ 32) is
        // taken only then.
        float alpha = 1.f;
        if (__any(mx > thr)) {  // the reference moves for some row of this wave
          mx = xor32_max(mx);
          const bool bump = mx > thr;
          const float m_new = bump ? mx * sl2 : m_run;
          alpha = (bump && m_run != -INFINITY) ? fast_exp2(m_run - m_new) : 1.f;
          m_run = m_new;
          neg_m = m_new == -INFINITY ? 0.f : -m_new;
          thr = (m_new + kSlack) * inv_sl2;
          if (__any(alpha != 1.f)) {
#pragma unroll
            for (int b = 0; b < DB; ++b) o[b] *= alpha;
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], sl2, neg_m));

        // O^T += V^T . P^T, 16 keys per step.  The row sum is taken from the
        // same bf16-rounded p that multiply V, two per v_dot2 (each packed
        // word is summed as its own value, before it joins the MFMA operand).
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kb = u >> 1, i0 = 8 * (u & 1);
          u32x4 pw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = pack_bf16(s[kb][i0 + 2 * w], s[kb][i0 + 2 * w + 1]);
            rs = sum_bf16x2(x, rs);
            pw[w] = x;
          }
          const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
          for (int b = 0; b < DB; ++b) {
            const int d = b * 32 + qcol;
            const int ch = 2 * u + half;
            const bf16x8 va = as_bf16x8(ld16(Vt + d * kBN + ((ch ^ vt_swz(d)) * 8)));
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[b], 0, 0, 0);
          }
        }
        l_run = l_run * alpha + rs;
      }
      __syncthreads();
    }

    // ---- next unit: start its loads, then finish this one -------------------
    // Both s_unit slots alternate: the slot claimed here was last read one
    // unit ago, before barriers every thread has since passed.
    const int un = __builtin_amdgcn_readfirstlane(s_unit[slot ^ 1]);
    const UnitInfo Uc = U;
    if (un >= 0) {
      U = load_unit(pv, un);
      start_unit(U);
    }
    ui = un;
    slot ^= 1;

    // ---- epilogue of unit Uc --------------------------------------------------
    if (wave_active) {
      const Lane L = lane_of(Uc);
      // opaque copy: output addresses are formed here, not kept across units
      int hf = half;
      asm volatile("" : "+v"(hf));
      const float l_tot = xor32_sum(l_run);
      if (L.row_ok) {
        const bool seen = l_tot > 0.f;
        const float inv = seen ? 1.f / l_tot : 0.f;
        const float lse = seen ? m_run + __log2f(l_tot) : -INFINITY;
        if (Uc.prow < 0) {
          const int64_t orow = static_cast<int64_t>(Uc.qo_begin + L.tok) * Hq + L.head;
          if (a.out_fp32) {
            float* op = static_cast<float*>(a.o) + orow * D;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int d0 = b * 32 + 8 * g + 4 * hf;
                *reinterpret_cast<f32x4*>(op + d0) =
                    f32x4{o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv};
              }
          } else {
            uint16_t* op = static_cast<uint16_t*>(a.o) + orow * D;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int d0 = b * 32 + 8 * g + 4 * hf;
                u32x2 pk;
                pk[0] = pack_bf16(o[b][4 * g] * inv, o[b][4 * g + 1] * inv);
                pk[1] = pack_bf16(o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(op + d0) = pk;
              }
          }
          if (a.lse && hf == 0) a.lse[orow] = lse;
        } else {
          const int64_t prow_i = Uc.prow + (L.my_row - Uc.row_begin);
          float* op = a.part_o + prow_i * D;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int d0 = b * 32 + 8 * g + 4 * hf;
              *reinterpret_cast<f32x4*>(op + d0) =
                  f32x4{o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv};
            }
          if (hf == 0) a.part_o[pv.partial_lse + prow_i] = lse;
        }
      }
    }
  }

  // Workers take units from every queue, so the launch's last worker to get
  // here (counted on queue 0's record) resets every queue's counter for the
  // next run; acq_rel orders every worker's final takes before the reset.
  if (tid == 0) {
    int32_t* s0 = pv.sched;
    const int done = __hip_atomic_fetch_add(s0 + kSchedDone, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == static_cast<int>(gridDim.x) - 1) {
      for (int q = 0; q < n_queues; ++q)
        __hip_atomic_store(pv.sched + q * kSchedWords + kSchedNext, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(s0 + kSchedDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace
}  // namespace pka
