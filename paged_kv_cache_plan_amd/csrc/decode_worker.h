// Single-token decode attention over a paged (or ragged dense) KV cache, gfx950:
// the persistent workgroup's work (decode_worker), used by the decode kernel
// and by the one-grid mixed kernel.
//
// A work unit is (request r, KV head hk, key range [kv_lo, kv_hi)).  The G
// query heads that share KV head hk are processed together so each K/V byte
// is read from HBM once.  The launch is persistent: one workgroup per
// resident slot takes units, longest first, from one queue and starts
// loading its next unit while it merges and writes the current one.  The
// waves (four in the decode kernel) take interleaved 32-key steps of the
// range and keep independent online-softmax states, merged through LDS at
// the end (the recursive-attention identity: FlashInfer documentation,
// "Attention States and Recursive Attention").
//
// Loads run two steps ahead of the math: a step issues the page ids of the
// step after next, then the K/V rows of the next step (nontemporal: each
// byte is read once), then computes on its own rows, which arrived during
// the previous step.  Every load is unconditional (keys past a unit's end
// read its last row and are masked), so the compiler's wait counts stay
// exact and a step never waits for the loads queued behind its own.
//
// Per 32-key step of one wave:
//   K        loaded from global straight into the A operand of
//            v_mfma_f32_16x16x32_bf16 (lane: key l % 16, 8 consecutive d);
//   S^T      = K . Q^T, query heads as MFMA columns (up to 16);
//   softmax  fp32, base 2, row max over the four 16-lane rows with
//            v_permlane16_swap / v_permlane32_swap;
//   V        loaded 16 bytes per key, transposed in registers into a
//            wave-private V^T tile in LDS, whose key order matches the order
//            in which the S^T accumulator holds the scores, so P^T is the
//            accumulator itself rounded to bf16;
//   O^T     += V^T . P^T.
// The kernel is bound by HBM bandwidth; the MFMA padding of G < 16 heads to
// 16 columns costs matrix-core time that is otherwise idle.
#pragma once

#include <type_traits>

#include "args.h"
#include "device.h"
#include "planner.h"

namespace pka {
namespace {

constexpr int kTK = 32;  // keys per wave step
constexpr int kDecodeWaves = 4;  // waves of a decode workgroup

// V^T row chunk swizzle (4 chunks of 8 keys per 32-key row).
__device__ __forceinline__ int dvt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }

// How a step finds its K/V rows: ragged dense tensors, a page table whose
// page_size is a power of two >= 16 (each 16-key half of a step lies in one
// page, so the whole wave shares two page ids), or any other page table (one
// page id per row).
enum IdMode : int { kRagged = 0, kPagedUniform = 1, kPagedLane = 2, kPagedLaneDiv = 3 };

// The work of one persistent decode workgroup of NW waves: units from the
// plan's queue until it is empty.  The decode kernel runs it with 4 waves;
// the one-grid mixed kernel, after the prefill worker, with the prefill
// workgroup's waves.
template <int D, int MODE, int NW>
__device__ __forceinline__ void decode_worker(const AttnArgs a) {
  constexpr int kWaves = NW;
  constexpr int kThreads = 64 * NW;
  constexpr bool PAGED = MODE != kRagged;
  constexpr bool LANE = MODE == kPagedLane || MODE == kPagedLaneDiv;  // page ids per lane
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int DS = D / 32;   // k-steps of the S^T MFMA
  constexpr int DB = D / 16;   // 16-row d blocks of O^T
  constexpr int VT_ELEMS = D * kTK;               // per-wave V^T tile (bf16)
  constexpr int MERGE_BYTES = kWaves * 16 * (D + 2) * 4;
  constexpr int VT_BYTES = kWaves * VT_ELEMS * 2;
  constexpr int SMEM = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

  __shared__ int s_unit[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int G = a.group, Hq = a.num_qo_heads;
  const PlanView pv = plan_view(a.ws);

  const int col = lane & 15;  // query head within the group (MFMA column)
  const int g4 = lane >> 4;   // 16-lane row
  const bool col_ok = col < G;

  int32_t* sched = pv.sched + (blockIdx.x % pv.num_queues) * kSchedWords;
  const int q_begin = sched[kSchedBegin], q_end = sched[kSchedEnd];
  auto claim = [&](int slot) {
    if (tid == 0)
      s_unit[slot] = q_begin + __hip_atomic_fetch_add(sched + kSchedNext, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
  };
  // fields of a unit and of its request (wave-uniform)
  struct Unit { int hk, kv_lo, kv_hi, prow, qo_begin, kv_base; };
  auto load_unit = [&](int ui) {
    const int32_t* u = pv.units + static_cast<int64_t>(ui) * kUnitWords;
    // read as wave-uniform values, so that no later wait is left pending on
    // these loads (a join with a path that never used them would keep one)
    auto rd = [&](int w) { return __builtin_amdgcn_readfirstlane(u[w]); };
    Unit x;
    x.hk = rd(kUnitKvHead);
    x.kv_lo = rd(kUnitKvBegin);
    x.kv_hi = rd(kUnitKvEnd);
    x.prow = rd(kUnitPartialRow);
    x.qo_begin = rd(kUnitQoBegin);
    x.kv_base = rd(kUnitKvBase);
    return x;
  };

  bf16x8 qreg[DS];
  const int ps = a.page_size, pshift = a.page_shift;
  int hk = 0, kv_hi = 0, kv_base = 0;  // of the unit being loaded
  const uint16_t* kb_ptr = a.k;
  const uint16_t* vb_ptr = a.v;
  auto bind = [&](const Unit& U) {
    hk = U.hk;
    kv_hi = U.kv_hi;
    kv_base = U.kv_base;
    kb_ptr = a.k + U.hk * a.head_stride;
    vb_ptr = a.v + U.hk * a.head_stride;
  };

  // V loader: a V^T row (one d, 32 keys) holds four 8-key slots; slot vg
  // holds keys 4 vg + j (j < 4) and 16 + 4 vg + j - 4 (j >= 4).  At D=128
  // (16 chunks a row) lane (vc, vg) loads chunk vc of all 8 keys of slot vg;
  // at D=64 (8 chunks a row) lane (vc, vh, vg) loads chunk vc of the half vh
  // of slot vg (VJ = 4 keys), so that every lane loads only rows it uses.
  constexpr int VJ = CPR == 16 ? 8 : 4;
  static_assert(CPR == 16 || CPR == 8, "head_dim 128 or 64");
  const int vc = lane % CPR;
  const int vg = (lane / CPR) & 3, vh = CPR == 16 ? 0 : lane / (4 * CPR);
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * VT_ELEMS;

  // Keys of one step handled by this lane: K rows 16 kb + col (kb = 0, 1);
  // V rows: element j of the lane's part of slot vg.
  auto v_key = [&](int j) {
    const int jj = j + 4 * vh;
    return jj < 4 ? 4 * vg + jj : 16 + 4 * vg + (jj - 4);
  };

  // Page ids of a step.
  struct IdsUniform { int s[2]; };
  struct IdsLane { int key; };  // lane l: the page id of key k0 + (l % 32)
  struct IdsNone {};
  using Ids = typename std::conditional<MODE == kPagedUniform, IdsUniform,
                typename std::conditional<LANE, IdsLane, IdsNone>::type>::type;
  // page of a key; the page size is a compile-time choice between a power of
  // two and not, so no id load sits behind a branch
  auto page_of = [&](int key) -> int {  // (keys are never negative)
    return MODE == kPagedLaneDiv ? static_cast<unsigned>(key) / static_cast<unsigned>(ps) : key >> pshift;
  };
  // Keys past the unit's range read the row of its last key instead: a
  // valid row whose score the mask sets to -inf, so its P is exactly zero.
  // No load is then predicated, and no load result is copied or read as a
  // wave-uniform value before its use, which would wait for every load in
  // flight (the next step's prefetch included).
  auto fetch_ids = [&](int k0, Ids& id) {
    const int last = kv_hi - 1;
    if constexpr (MODE == kPagedUniform) {
      // per-lane copies of the two ids (VGPRs, not SGPRs)
      int z = 0;
      asm volatile("" : "+v"(z));
      id.s[0] = pv.kv_indices[kv_base + (min(k0, last) >> pshift) + z];
      id.s[1] = pv.kv_indices[kv_base + (min(k0 + 16, last) >> pshift) + z];
    } else if constexpr (LANE) {
      // one id load per lane; the K and V rows' lanes fetch theirs from the
      // lane that holds them (ds_bpermute) when the data loads are formed
      const int key = min(k0 + (lane & 31), last);
      id.key = pv.kv_indices[kv_base + page_of(key)];
    }
  };
  auto row_off = [&](int key, int pid) -> int64_t {  // element offset of the K row of `key`
    if constexpr (PAGED) {
      const int slot = MODE == kPagedLaneDiv ? static_cast<int>(static_cast<unsigned>(key) % static_cast<unsigned>(ps))
                                            : (key & (ps - 1));
      return static_cast<int64_t>(pid) * a.page_stride + static_cast<int64_t>(slot) * a.row_stride;
    } else {
      return static_cast<int64_t>(kv_base + key) * a.page_stride;
    }
  };
  struct Data { u32x4 k[2][DS]; u32x4 v[VJ]; };
  auto fetch_data = [&](int k0, const Ids& id, Data& x) {
    const int last = kv_hi - 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(k0 + 16 * kb + col, last);
      int pid = 0;
      if constexpr (MODE == kPagedUniform) pid = id.s[kb];
      if constexpr (LANE) pid = __builtin_amdgcn_ds_bpermute((16 * kb + col) * 4, id.key);
      const uint16_t* p = kb_ptr + row_off(key, pid) + 8 * g4;
#pragma unroll
      for (int s = 0; s < DS; ++s) x.k[kb][s] = ld16_stream(p + 32 * s);
    }
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const int key = min(k0 + v_key(j), last);
      int pid = 0;
      if constexpr (MODE == kPagedUniform) pid = (j + 4 * vh) < 4 ? id.s[0] : id.s[1];  // key half of the step
      if constexpr (LANE) pid = __builtin_amdgcn_ds_bpermute(v_key(j) * 4, id.key);
      x.v[j] = ld16_stream(vb_ptr + row_off(key, pid) + 8 * vc);
    }
  };

  // Steps t = wave, wave + 4, ...: page ids two steps ahead, data one ahead,
  // each in two buffers that alternate from step to step (the first step of
  // a unit reads buf_a, and ids_b holds the ids of its second step).
  Ids ids_a{}, ids_b{};
  Data buf_a{}, buf_b{};
  auto start_unit = [&](const Unit& U) {
    bind(U);
    const uint16_t* qp = a.q + (static_cast<int64_t>(U.qo_begin) * Hq + U.hk * G + (col_ok ? col : 0)) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = as_bf16x8(col_ok ? ld16(qp + 32 * s) : u32x4{0, 0, 0, 0});
    if (U.kv_hi > U.kv_lo) {
      // ids of the first two steps before the first data, so that waiting
      // for the second step's ids does not wait for the first step's data
      fetch_ids(U.kv_lo + wave * kTK, ids_a);
      fetch_ids(U.kv_lo + (wave + kWaves) * kTK, ids_b);
      fetch_data(U.kv_lo + wave * kTK, ids_a, buf_a);
    }
  };

  claim(0);
  __syncthreads();
  int ui = __builtin_amdgcn_readfirstlane(s_unit[0]);
  int slot = 0;
  Unit U{};
  if (ui < q_end) {
    U = load_unit(ui);
    start_unit(U);
  }
  while (ui < q_end) {
  const int kv_lo = U.kv_lo, prow = U.prow, qo_begin = U.qo_begin;
  f32x4 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  const int n_tiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kTK - 1) / kTK : 0;
  // Thread 0 takes the next unit as its wave starts its last step (at once
  // if it has none) and writes the id to LDS after the steps (the first
  // merge barrier publishes it), so the atomic's return is awaited only there.
  int next_claim = 0;
  // Every step issues the same loads (past the unit's end they are clamped,
  // unused reads), so the compiler's load accounting stays exact and a step
  // waits only for its own data, not for the prefetch behind it.
  // The ids two steps ahead are issued before the next step's data, so the
  // wait for the ids that data needs leaves that step's own data in flight.
  auto step = [&](int t, Data& cur, Data& nxt, const Ids& ids_use, Ids& ids_fill) {
    const int k0 = kv_lo + t * kTK;
    fetch_ids(k0 + 2 * kWaves * kTK, ids_fill);
    fetch_data(k0 + kWaves * kTK, ids_use, nxt);
    // keep this step's work on `cur` below the loads (hoisted above them, it
    // would wait for `cur` before they issue)
    __builtin_amdgcn_sched_barrier(0);

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int st = 0; st < DS; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[kb][st]), qreg[st], s[kb], 0, 0, 0);
    }

    // transpose V into the wave's V^T tile
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // (an empty use by every lane, so that no path past the branch below
    // sees these loads as still pending: a later write to their registers
    // would wait for the newest loads)
#pragma unroll
    for (int j = 0; j < VJ; ++j) __asm__ volatile("" ::"v"(cur.v[j]));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vc + e;
      const int w = e >> 1;
      uint16_t* dst = vt + d * kTK + ((vg ^ dvt_swz(d)) * 8) + 4 * vh;
      if constexpr (VJ == 8) {
        u32x4 pk;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pk[h] = (e & 1) ? pack_hi16(cur.v[2 * h][w], cur.v[2 * h + 1][w])
                          : pack_lo16(cur.v[2 * h][w], cur.v[2 * h + 1][w]);
        st16(dst, pk);
      } else {
        u32x2 pk;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pk[h] = (e & 1) ? pack_hi16(cur.v[2 * h][w], cur.v[2 * h + 1][w])
                          : pack_lo16(cur.v[2 * h][w], cur.v[2 * h + 1][w]);
        *reinterpret_cast<u32x2*>(dst) = pk;
      }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // mask keys past the range; S^T lane holds keys 16 kb + 4 g4 + i
    if (k0 + kTK > kv_hi) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 16 * kb + 4 * g4 + i >= kv_hi) s[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][i], sl2, -m_use));
        s[kb][i] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
    }

    u32x4 pw;
    pw[0] = pack_bf16(s[0][0], s[0][1]);
    pw[1] = pack_bf16(s[0][2], s[0][3]);
    pw[2] = pack_bf16(s[1][0], s[1][1]);
    pw[3] = pack_bf16(s[1][2], s[1][3]);
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int d = 16 * b + col;
      const bf16x8 va = as_bf16x8(ld16(vt + d * kTK + ((g4 ^ dvt_swz(d)) * 8)));
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[b], 0, 0, 0);
    }
  };
  // pairs of steps, then an odd last one: no path runs a step twice in a
  // row on one buffer, which would leave its prefetch looking unfinished
  const int my_steps = wave < n_tiles ? (n_tiles - 1 - wave) / kWaves + 1 : 0;
  auto claim_at = [&](int i) {
    if (tid == 0 && i == my_steps - 1)
      next_claim = __hip_atomic_fetch_add(sched + kSchedNext, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (my_steps == 0) claim_at(-1);
  int t = wave;
  for (int i = 0; i < (my_steps >> 1); ++i, t += 2 * kWaves) {
    claim_at(2 * i);
    step(t, buf_a, buf_b, ids_b, ids_a);
    claim_at(2 * i + 1);
    step(t + kWaves, buf_b, buf_a, ids_a, ids_b);
  }
  if (my_steps & 1) {
    claim_at(my_steps - 1);
    step(t, buf_a, buf_b, ids_b, ids_a);
  }

  // ---- merge the waves' states ------------------------------------------
  __asm__ volatile("" ::"v"(next_claim));  // awaited here by every lane, not only in the branch
  if (tid == 0) s_unit[slot ^ 1] = q_begin + next_claim;
  float l_tot = xor32_sum(xor16_sum(l_run));
  __syncthreads();  // every wave is done with its V^T tile; publishes the claim
  // the next unit's Q, page ids and first K/V step load during this merge;
  // the s_unit slot claimed now was last read one unit ago, before barriers
  // every thread has since passed
  const int un = __builtin_amdgcn_readfirstlane(s_unit[slot ^ 1]);
  const int c_hk = hk;
  if (un < q_end) {
    U = load_unit(un);
    start_unit(U);
  }
  ui = un;
  slot ^= 1;
  float* wo = reinterpret_cast<float*>(smem);            // [wave][16][D]
  float* wm = wo + kWaves * 16 * D;                       // [wave][16]
  float* wl = wm + kWaves * 16;                           // [wave][16]
  if (g4 == 0) {
    wm[wave * 16 + col] = m_run;
    wl[wave * 16 + col] = l_tot;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) wo[(wave * 16 + col) * D + 16 * b + 4 * g4 + i] = o[b][i];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int c = idx / D, d = idx - c * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * 16 + c]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = fast_exp2(wm[w * 16 + c] - M);
        L += sc * wl[w * 16 + c];
        acc += sc * wo[(w * 16 + c) * D + d];
      }
    }
    const bool seen = L > 0.f;
    const float val = seen ? acc / L : 0.f;
    const float lse = seen ? M + __log2f(L) : -INFINITY;
    if (prow < 0) {
      const int64_t orow = static_cast<int64_t>(qo_begin) * Hq + c_hk * G + c;
      if (a.out_fp32)
        static_cast<float*>(a.o)[orow * D + d] = val;
      else
        static_cast<__bf16*>(a.o)[orow * D + d] = static_cast<__bf16>(val);
      if (a.lse && d == 0) a.lse[orow] = lse;
    } else {
      a.part_o[static_cast<int64_t>(prow + c) * D + d] = val;
      if (d == 0) a.part_o[pv.partial_lse + prow + c] = lse;
    }
  }
  __syncthreads();  // the next unit's V^T tiles reuse the merge buffers
  }

  // The last worker of the queue to get here resets its counters for the
  // next run; acq_rel orders every worker's final take before the reset.
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(sched + kSchedDone, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == sched[kSchedWorkers] - 1) {
      __hip_atomic_store(sched + kSchedNext, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sched + kSchedDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace
}  // namespace pka
