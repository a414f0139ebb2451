// Device helpers shared by the HiLS kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

typedef uint16_t bf16_t;

// ---- element storage: bf16 (raw uint16) or fp32 ---------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// double -> bf16 with a single round-to-nearest-even from the double value
// (never through fp32, which could round twice).  The value is scaled by a
// power of two so that its 8 significant bits are the integer part, rounded
// with rint (ties to even), and scaled back; subnormal bf16 values use the
// fixed quantum 2^-133.  The rounded value is exact in fp32, so the final
// conversion to fp32 is exact and its top 16 bits are the bf16 pattern.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  if (!(x == x)) return (bf16_t)0x7fc0;
  if (x == 0.0 || isinf(x)) return f32_to_bf16((float)x);
  int e = ilogb(x);                    // |x| in [2^e, 2^(e+1))
  int sh = (e < -126) ? 133 : 7 - e;
  double r = ldexp(rint(ldexp(x, sh)), -sh);
  float f = (float)r;                  // exact, or +-inf when r >= 2^128
  return (bf16_t)(__float_as_uint(f) >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void st64(float* p, double v) { *p = (float)v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ void st64(bf16_t* p, double v) { *p = f64_to_bf16(v); }
};

// ---- window geometry (0-based; floor division) ----------------------------

// l(i) = floor((i - W + 1)/S) * S
__device__ __forceinline__ long long window_left(long long i, int W, int S) {
  long long t = i - W + 1;
  long long q = (t >= 0) ? t / S : -((-t + S - 1) / S);
  return q * S;
}
// |C_i| = max(0, l(i)/S)
__device__ __forceinline__ int n_cand(long long i, int W, int S) {
  long long l = window_left(i, W, S);
  return l > 0 ? (int)(l / S) : 0;
}
__device__ __forceinline__ long long window_start(long long i, int W, int S) {
  long long l = window_left(i, W, S);
  return l > 0 ? l : 0;
}

// Decode length of sequence b clamped to [1, cap] so that no kernel can index
// outside the cache even for an out-of-contract seqlen value.
__device__ __forceinline__ long long clamp_len(int32_t t, int cap) {
  return t < 1 ? 1 : (t > cap ? (long long)cap : (long long)t);
}

// ---- wave64 reductions ------------------------------------------------------

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// inverse of f32_order_key
__device__ __forceinline__ float order_key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// float -> uint32 key whose unsigned order is the float order (-0 mapped to +0).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
