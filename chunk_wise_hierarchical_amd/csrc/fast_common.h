// Shared pieces of the bf16 MFMA fast path (d = 128, S = 64, gfx950 wave64).
#pragma once
#include "hils_device.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace fastp {

constexpr int D = 128;
constexpr int S = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t ld_bf16x8(const bf16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ uint4 ld_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st_u4(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the bare v_exp_f32 (results below 2^-126 flush to zero, which is
// harmless for softmax weights; exp2(-inf) = 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lanes l, l^16 (resp. l^32) with the gfx950 row-swap
// instructions (VALU, no LDS round trip).  permlane16_swap(v, v) yields, in
// every lane, the pair {v[l], v[l^16]} ordered lower lane first, so max/sum of
// the pair is the xor-16 reduction; permlane32_swap likewise for xor-32.
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of lane l ^ stride within the wavefront, for stride in {1,...,32}
// (a compile-time constant after unrolling).  Strides 1-8 use DPP row
// patterns (quad_perm, row_half_mirror, row_mirror), 16 and 32 the row-swap
// instructions: VALU only, no LDS round trip.
__device__ __forceinline__ uint32_t xshfl(uint32_t v, int stride) {
  if (stride == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  if (stride == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  if (stride == 4) {
    const int t = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false);
  }
  if (stride == 8) {
    const int t = __builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, false);
  }
  if (stride == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  }
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float xshfl_f(float v, int stride) {
  return __uint_as_float(xshfl(__float_as_uint(v), stride));
}
__device__ __forceinline__ uint64_t xshfl_u64(uint64_t v, int stride) {
  return ((uint64_t)xshfl((uint32_t)(v >> 32), stride) << 32) | xshfl((uint32_t)v, stride);
}
// maximum / sum over all 64 lanes (xor butterfly: every lane gets the same value)
__device__ __forceinline__ float wmax64(float v) {
  v = fmaxf(v, xshfl_f(v, 1));
  v = fmaxf(v, xshfl_f(v, 2));
  v = fmaxf(v, xshfl_f(v, 4));
  v = fmaxf(v, xshfl_f(v, 8));
  return max_x32(max_x16(v));
}
__device__ __forceinline__ float wsum64(float v) {
  v += xshfl_f(v, 1);
  v += xshfl_f(v, 2);
  v += xshfl_f(v, 4);
  v += xshfl_f(v, 8);
  return sum_x32(sum_x16(v));
}

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// workgroup id.  xcd_work maps workgroup blk of a grid of at least
// NXCD * ceil(nwork / NXCD) workgroups to a work index such that XCD x takes
// the contiguous range [x * per, (x + 1) * per), per = ceil(nwork / NXCD), in
// order: neighbouring work items, which share data through L2, run on one
// XCD.  Workgroups without a work item get -1.
constexpr int NXCD = 8;
__device__ __forceinline__ long long xcd_work(long long blk, long long nwork) {
  const long long per = (nwork + NXCD - 1) / NXCD;
  const long long j = blk / NXCD;
  if (j >= per) return -1;
  const long long L = (blk % NXCD) * per + j;
  return L < nwork ? L : -1;
}
inline long long xcd_grid(long long nwork) { return NXCD * ((nwork + NXCD - 1) / NXCD); }

// value of lane 63 - l (= l ^ 63)
__device__ __forceinline__ uint32_t lane_reverse(uint32_t v) {
  const uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);   // l ^ 15
  return xshfl(xshfl(t, 16), 32);
}

// 64-bit shuffle
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace fastp
