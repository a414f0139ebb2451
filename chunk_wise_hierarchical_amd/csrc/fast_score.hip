// Fast-path chunk scoring + exact top-K selection (bf16, d = 128, S = 64).
//
// "Hierarchical Sparse Attention Done Right", section 3 routing equation
// (s_hat = q_hat . k'_c / sqrt(d) + b'_c, top-K over the candidate chunks C_i)
// and section 4.1 (GQA: per-head log-softmax over C_i, maximum over the heads
// of a group, one shared top-K).
//
// One workgroup (4 wavefronts) owns QB = 128/G query positions of one
// (batch, KV group).  k' tiles of 32 chunks x G heads stream through LDS
// (double-buffered); each wavefront computes a 32-chunk x 32-query score tile
// of one head with v_mfma_f32_32x32x16_bf16 (A = k' rows, B = q_hat).  Scores
// are kept in base-2 units (scaled by log2 e), which preserves their order.
//   pass 0 (G > 1 only): per (query, head) online log-sum-exp over C_i;
//   pass 1: group score g = max_h (s_h - L_h) (cross-head max through LDS),
//           filtered against the query's current K-th best key and appended to
//           an LDS staging list; a staging list past half full is merged into
//           the query's sorted top-K list by a wavefront-wide bitonic sort.
// Keys are 64-bit: (order-preserving bits of g) << 32 | (~chunk id), so ties
// rank the lower chunk id first and every key is unique.  The selected ids
// are written ascending, -1 padded.
#include "fast_common.h"
#include "hils_internal.h"

using namespace fastp;

namespace {

constexpr int NT = 256;
constexpr int CT = 32;         // chunks per tile
constexpr int KROW = D + 8;    // padded k' row in LDS (elements)
constexpr int XROW = CT + 4;   // padded row of the cross-head exchange buffer (floats)
constexpr int STG = 64;        // staging slots per query

template <int G>
struct Geo {
  static constexpr int QB = 32 * 4 / G;   // queries per workgroup
  static constexpr int QW = QB / 4;       // queries per wavefront in the selection layout
  static constexpr int LQ = 64 / QW;      // lanes per query
  static constexpr int CL = CT / LQ;      // chunks per lane per tile (selection layout)
};

template <int G>
struct Lds {
  size_t ktile, btile, xb, lst, stg, cnt, thr, total;
  __host__ __device__ Lds(int K) {
    size_t o = 0;
    ktile = o; o += (size_t)2 * G * CT * KROW * 2;
    btile = o; o += (size_t)2 * G * CT * 4;
    xb = o;    o += (G > 1) ? (size_t)G * Geo<G>::QB * XROW * 4 : 0;
    o = (o + 15) & ~(size_t)15;
    lst = o;   o += (size_t)Geo<G>::QB * K * 8;
    stg = o;   o += (size_t)Geo<G>::QB * STG * 8;
    cnt = o;   o += (size_t)Geo<G>::QB * 2 * 4;
    o = (o + 15) & ~(size_t)15;
    thr = o;   o += (size_t)Geo<G>::QB * 8;
    total = o;
  }
};

// wavefront-wide bitonic sort of 128 keys (2 per lane: index lane and lane+64), descending
__device__ __forceinline__ void sort128_desc(uint64_t& e0, uint64_t& e1, int lane) {
#pragma unroll
  for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 64) {
        const uint64_t mx = e0 > e1 ? e0 : e1, mn = e0 > e1 ? e1 : e0;
        e0 = mx; e1 = mn;
      } else {
        const uint64_t p0 = shfl_xor_u64(e0, stride), p1 = shfl_xor_u64(e1, stride);
        const bool lower = (lane & stride) == 0;
        const bool desc0 = ((lane & size) == 0);
        const bool desc1 = (((lane + 64) & size) == 0);
        const bool km0 = (lower == desc0), km1 = (lower == desc1);
        e0 = km0 ? (e0 > p0 ? e0 : p0) : (e0 < p0 ? e0 : p0);
        e1 = km1 ? (e1 > p1 ? e1 : p1) : (e1 < p1 ? e1 : p1);
      }
    }
  }
}

// wavefront-wide bitonic sort of 64 ints (1 per lane), ascending
__device__ __forceinline__ int sort64_asc(int v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int p = __shfl_xor(v, stride, 64);
      const bool lower = (lane & stride) == 0;
      const bool asc = (lane & size) == 0;
      v = (lower == asc) ? min(v, p) : max(v, p);
    }
  }
  return v;
}

template <int G>
__global__ void __launch_bounds__(NT)
k_score_fast(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ ksum,
             const float* __restrict__ bsum, int32_t* __restrict__ sel, int Hq, int Hkv, int N,
             int W, int K, int nC, float tau2, int nqb) {
  using GE = Geo<G>;
  constexpr int QB = GE::QB, QW = GE::QW, LQ = GE::LQ, CL = GE::CL;
  extern __shared__ __align__(16) unsigned char sm[];
  const Lds<G> L(K);
  bf16_t* ktile = reinterpret_cast<bf16_t*>(sm + L.ktile);   // [2][G][CT][KROW]
  float* btile = reinterpret_cast<float*>(sm + L.btile);     // [2][G][CT]  (b' * log2 e)
  float* xb = reinterpret_cast<float*>(sm + L.xb);           // [G][QB][XROW]
  uint64_t* lst = reinterpret_cast<uint64_t*>(sm + L.lst);   // [QB][K]
  uint64_t* stg = reinterpret_cast<uint64_t*>(sm + L.stg);   // [QB][STG]
  uint32_t* cnt_stg = reinterpret_cast<uint32_t*>(sm + L.cnt);
  uint32_t* cnt_lst = cnt_stg + QB;
  uint64_t* thr = reinterpret_cast<uint64_t*>(sm + L.thr);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int qb = nqb - 1 - (blk % nqb);            // heaviest query blocks first
  const int bg = blk / nqb;
  const int g = bg % Hkv;
  const long long b = bg / Hkv;
  const int i0 = qb * QB;
  const int i_last = min(i0 + QB, N) - 1;
  const int n_hi = n_cand(i_last, W, S);
  const int ntiles = (n_hi + CT - 1) / CT;
  const long long hb = b * Hq + (long long)g * G;  // first query head of the group
  int32_t* selg = sel + (b * Hkv + g) * (long long)N * K;

  if (ntiles == 0) {
    for (int t = tid; t < (i_last - i0 + 1) * K; t += NT) selg[(long long)i0 * K + t] = -1;
    return;
  }
  for (int t = tid; t < QB; t += NT) { cnt_stg[t] = 0; cnt_lst[t] = 0; thr[t] = 0; }

  // MFMA layout: wavefront -> (head hw, 32-query column block qw); lane -> query column
  const int hw = w % G, qw = w / G;
  const int col = lane & 31, half = lane >> 5;
  const int iq = i0 + 32 * qw + col;
  const int nq = (iq < N) ? n_cand(iq, W, S) : 0;
  bf16x8_t bq[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (iq < N) bq[ks] = ld_bf16x8(qr + ((hb + hw) * N + iq) * (long long)D + 16 * ks + 8 * half);
    else bq[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }

  // selection layout: lane -> (query qsel, CL chunks of the tile)
  const int qsel = (G == 1) ? (32 * w + col) : (w * QW + lane / LQ);
  const int cbase = (G == 1) ? 0 : CL * (lane % LQ);

  // tile staging through registers (double-buffered LDS)
  constexpr int PPT = 2 * G;               // 16-byte pieces per thread per tile
  uint4 pre[PPT];
  float bpre = 0.0f;
  auto load_tile = [&](int t) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = tid + NT * p;
      const int h = piece / (CT * 16), c = (piece / 16) % CT, part = piece % 16;
      const int cg = CT * t + c;
      pre[p] = (cg < nC) ? ld_u4(ksum + ((hb + h) * nC + cg) * (long long)D + part * 8)
                         : make_uint4(0, 0, 0, 0);
    }
    if (tid < G * CT) {
      const int h = tid / CT, cg = CT * t + tid % CT;
      bpre = (cg < nC) ? bsum[(hb + h) * nC + cg] * LOG2E : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = tid + NT * p;
      const int h = piece / (CT * 16), c = (piece / 16) % CT, part = piece % 16;
      st_u4(ktile + (((size_t)buf * G + h) * CT + c) * KROW + part * 8, pre[p]);
    }
    if (tid < G * CT) btile[buf * G * CT + tid] = bpre;
  };

  // merge query q's staging list into its sorted top-K list (whole wavefront)
  auto merge = [&](int q) {
    const int ns = (int)cnt_stg[q], nl = (int)cnt_lst[q];
    uint64_t e0 = (lane < nl) ? lst[(size_t)q * K + lane] : 0ull;
    uint64_t e1 = (lane < ns) ? stg[(size_t)q * STG + lane] : 0ull;
    sort128_desc(e0, e1, lane);
    const int tot = min(K, nl + ns);
    const uint32_t klo = __shfl((uint32_t)e0, K - 1, 64);
    const uint32_t khi = __shfl((uint32_t)(e0 >> 32), K - 1, 64);
    if (lane < K) lst[(size_t)q * K + lane] = (lane < tot) ? e0 : 0ull;
    if (lane == 0) {
      cnt_lst[q] = tot;
      cnt_stg[q] = 0;
      thr[q] = (tot >= K) ? (((uint64_t)khi << 32) | klo) : 0ull;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };

  float L2 = 0.0f;
  for (int pass = (G > 1 ? 0 : 1); pass < 2; ++pass) {
    float m = -INFINITY, ssum = 0.0f;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) load_tile(t + 1);
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const bf16_t* kb = ktile + (((size_t)buf * G + hw) * CT + col) * KROW + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) acc = mfma32(ld_bf16x8(kb + 16 * ks), bq[ks], acc);
      const float* bt = btile + ((size_t)buf * G + hw) * CT;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cl = 8 * (i >> 2) + 4 * half + (i & 3);
        x[i] = (CT * t + cl < nq) ? fmaf(acc[i], tau2, bt[cl]) : -INFINITY;
      }
      if (pass == 0) {
        float mt = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, x[i]);
        if (mt > m) { ssum = (m == -INFINITY) ? 0.0f : ssum * exp2f(m - mt); m = mt; }
        if (m != -INFINITY) {
#pragma unroll
          for (int i = 0; i < 16; ++i) ssum += exp2f(x[i] - m);
        }
      } else {
        float gs[CL];
        int cid0;
        if (G > 1) {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = (x[i] == -INFINITY) ? -INFINITY : x[i] - L2;
          float* xr = xb + ((size_t)hw * QB + 32 * qw + col) * XROW;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float4 v4 = make_float4(x[4 * gq], x[4 * gq + 1], x[4 * gq + 2], x[4 * gq + 3]);
            *reinterpret_cast<float4*>(xr + 8 * gq + 4 * half) = v4;
          }
          __syncthreads();
#pragma unroll
          for (int j = 0; j < CL; j += 4) {
            float4 mx = *reinterpret_cast<const float4*>(xb + ((size_t)0 * QB + qsel) * XROW + cbase + j);
#pragma unroll
            for (int h = 1; h < G; ++h) {
              const float4 v = *reinterpret_cast<const float4*>(xb + ((size_t)h * QB + qsel) * XROW + cbase + j);
              mx.x = fmaxf(mx.x, v.x); mx.y = fmaxf(mx.y, v.y);
              mx.z = fmaxf(mx.z, v.z); mx.w = fmaxf(mx.w, v.w);
            }
            gs[j] = mx.x; gs[j + 1] = mx.y; gs[j + 2] = mx.z; gs[j + 3] = mx.w;
          }
          cid0 = CT * t + cbase;
        } else {
#pragma unroll
          for (int i = 0; i < CL; ++i) gs[i] = x[i];
          cid0 = CT * t;
        }
        // filter against the query's current K-th best key and stage the survivors
        const uint64_t th = thr[qsel];
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          const int cid = (G == 1) ? (cid0 + 8 * (j >> 2) + 4 * half + (j & 3)) : (cid0 + j);
          if (gs[j] != -INFINITY) {
            const uint64_t key = ((uint64_t)f32_order_key(gs[j]) << 32) |
                                 (uint64_t)(0xffffffffu - (uint32_t)cid);
            if (key > th) {
              const uint32_t slot = atomicAdd(&cnt_stg[qsel], 1u);
              stg[(size_t)qsel * STG + slot] = key;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (int qq = 0; qq < QW; ++qq) {
          const int q = w * QW + qq;
          if (cnt_stg[q] > (uint32_t)(STG / 2)) merge(q);
        }
      }
      if (t + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }
    if (pass == 0) {
      const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(ssum, 32, 64);
      const float M = fmaxf(m, m2);
      float s = 0.0f;
      if (M != -INFINITY) {
        s = (m == -INFINITY ? 0.0f : ssum * exp2f(m - M)) + (m2 == -INFINITY ? 0.0f : s2 * exp2f(m2 - M));
      }
      L2 = M + log2f(s);
    }
  }

  // final merge, ascending ids, write the selection
  for (int qq = 0; qq < QW; ++qq) {
    const int q = w * QW + qq;
    if (cnt_stg[q] > 0) merge(q);
    const int tot = (int)cnt_lst[q];
    const uint64_t e = (lane < tot) ? lst[(size_t)q * K + lane] : 0ull;
    int id = (lane < tot) ? (int)(0xffffffffu - (uint32_t)e) : 0x7fffffff;
    id = sort64_asc(id, lane);
    const int i = i0 + q;
    if (i < N && lane < K) selg[(long long)i * K + lane] = (lane < tot) ? id : -1;
  }
}

template <int G>
hipError_t launch_score(const HilsShape& s, const void* qr, const void* ksum, const float* bsum,
                        int32_t* sel, hipStream_t st) {
  const int QB = Geo<G>::QB;
  const int nqb = (s.N + QB - 1) / QB;
  const Lds<G> L(s.K);
  auto f = k_score_fast<G>;
  hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
  const float tau2 = (float)(s.tau * 1.4426950408889634);
  { HilsProfScope ps_("k_score_fast", st); hipLaunchKernelGGL(f, dim3((unsigned)((long long)s.B * s.Hkv * nqb)), dim3(NT), L.total, st,
                     (const bf16_t*)qr, (const bf16_t*)ksum, bsum, sel, s.Hq, s.Hkv, s.N, s.W, s.K,
                     s.nC, tau2, nqb); }
  return hipGetLastError();
}

}  // namespace

size_t hils_fast_score_lds(int G, int K) {
  switch (G) {
    case 1: return Lds<1>(K).total;
    case 2: return Lds<2>(K).total;
    case 4: return Lds<4>(K).total;
  }
  return 0;
}

hipError_t hils_launch_score_fast(const HilsShape& s, const void* qr, const void* ksum,
                                  const float* bsum, int32_t* sel, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_score<1>(s, qr, ksum, bsum, sel, st);
    case 2: return launch_score<2>(s, qr, ksum, bsum, sel, st);
    case 4: return launch_score<4>(s, qr, ksum, bsum, sel, st);
  }
  return hipErrorInvalidValue;
}
