// Device helpers for the gfx950 attention kernels: vector types, 16-byte
// loads and stores, wave-half exchanges and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "planner.h"

namespace pka {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// A streaming load of data read once (nontemporal: it does not displace
// cached data that is read again).
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Sum / max of x over the two lanes l and l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum / max over lanes l and l ^ 16 (v_permlane16_swap).
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round two floats to bf16 (round to nearest even) and pack them, lo first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Low / high 16-bit halves of two words, packed (v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The sections of a plan image in device memory, read from its header
// (wave-uniform scalar loads), so that kernel arguments do not depend on the
// batch that was planned.
struct PlanView {
  const int32_t* units;
  const int32_t* req;
  const int32_t* kv_indices;
  const int32_t* merge;
  int32_t* sched;
  int32_t num_queues;
  int32_t num_merge;
  int32_t merge_slices;  // workgroup slices of the largest merge group
  int32_t partial_lse;   // float index of the partial lse in the float workspace
};
__device__ __forceinline__ PlanView plan_view(const int32_t* ws) {
  PlanView v;
  v.units = ws + ws[kHdrOffUnits];
  v.req = ws + ws[kHdrOffReq];
  v.kv_indices = ws + ws[kHdrOffIndices];
  v.merge = ws + ws[kHdrOffMerge];
  v.sched = const_cast<int32_t*>(ws) + ws[kHdrOffSched];
  v.num_queues = ws[kHdrNumQueues];
  v.num_merge = ws[kHdrNumMerge];
  v.merge_slices = ws[kHdrMergeSlices];
  v.partial_lse = ws[kHdrPartialLse];
  return v;
}

}  // namespace pka
