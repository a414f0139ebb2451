// Fast-path prefill attention, organised by selected chunk ("pair-sorted"),
// bf16, d = 128, S = 64.
//
// "Hierarchical Sparse Attention Done Right", section 3 (hierarchical
// softmax): a query's output is the window attention plus, for each selected
// chunk c, an attention over that chunk's S keys alone, mixed by a softmax
// over {s_hat_c} U {log Z_swa}.  Once the window pass has fixed log Z_swa and
// the fusion weights alpha_c, every (query, selected chunk) pair is an
// independent S-key attention scaled by alpha_c.
//
// Section 4.2 of the pages packs adjacent queries and loads the union of their
// chunks; when adjacent queries route to different chunks that re-reads every
// chunk's K/V for almost every query.  Here the pairs of a slice of queries are
// bucketed by chunk instead, so each chunk's K/V is staged in LDS once per
// slice and every pair that selected it is computed against it:
//   1. k_pair_count / k_pair_bsum / k_pair_scan / k_pair_tiles / k_pair_scatter: counting
//      sort of the slice's (query, slot) pairs by (KV group, chunk), cut into
//      tiles of 64/G pairs (64 MFMA rows with the G heads of a group);
//   2. k_pair_attn: per tile, gather the 64 query rows, form the fusion logit
//      s_hat = scale q_hat.k'_c + b'_c of each row, S^T = K Q^T and
//      O^T = V^T P^T on MFMA; writes o_c (normalised, bf16) and s_hat per pair;
//   3. k_win_fuse: window attention (online softmax over the window tiles),
//      then alpha = softmax over {s_hat_c} U {log Z_swa} and
//      out = alpha_swa o_swa + sum_c alpha_c o_c, in slot order (deterministic;
//      the order of pairs inside a bucket never changes a result, since MFMA
//      rows are independent).  The window's compute overlaps the per-chunk
//      outputs' reads across the workgroups of a CU.
#include <algorithm>
#include <type_traits>

#include "fast_common.h"
#include "hils_internal.h"

using namespace fastp;

namespace {

// Streaming (non-temporal) access to the per-pair outputs, which are written
// once and read once: the bf16 partial rows (whole 128-byte lines per store
// instruction), the scattered 4-byte fusion logits and the reduction's reads,
// so that none of them displaces cached query rows and K/V.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_u4_nt(const void* p) {
  nt_u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ void st_u4_nt(void* p, uint4 v) {
  const nt_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x4*>(p));
}

constexpr int NT = 256;
constexpr int KSTR = D;       // K tile row stride (elements); 16-byte parts XOR-swizzled per row
constexpr int VSTR = S + 8;   // V^T tile row stride (elements)
constexpr int PQ = 512;       // queries per list-building workgroup
constexpr int PTPW = HILS_PAIR_TPW;   // tiles per pair-attention workgroup
constexpr int SB = HILS_PAIR_SB;      // buckets per scan workgroup
constexpr int KSS = D + 8;    // k'_c row stride in LDS (elements)
constexpr int OSTR = 17;      // output patch row stride (16-byte pieces; one of padding)

__device__ __forceinline__ int kswz(int r, int p) { return p ^ (((r >> 1) & 12) | (r & 3)); }

constexpr size_t KT_BYTES = (size_t)S * KSTR * 2;
constexpr size_t VT_BYTES = (size_t)D * VSTR * 2;

// ---------------------------------------------------------------------------
// pair lists

__global__ void __launch_bounds__(NT)
k_fill_u32(uint32_t* __restrict__ p, long long n, uint32_t v) {
  for (long long t = (long long)blockIdx.x * NT + threadIdx.x; t < n; t += (long long)gridDim.x * NT)
    p[t] = v;
}

// per (KV group, chunk): number of pairs of the slice that selected it
__global__ void __launch_bounds__(NT)
k_pair_count(const int32_t* __restrict__ sel, uint32_t* __restrict__ cnt, int N, int K, int nC,
             int i0, int qs) {
  extern __shared__ uint32_t hist[];   // [nC]
  const int bg = blockIdx.x;
  const int q0 = blockIdx.y * PQ;
  const int qn = min(PQ, qs - q0);
  for (int c = threadIdx.x; c < nC; c += NT) hist[c] = 0;
  __syncthreads();
  const int32_t* sb = sel + ((long long)bg * N + i0 + q0) * K;
  for (int t = threadIdx.x; t < qn * K; t += NT) {
    const int c = sb[t];
    if (c >= 0 && c < nC) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  uint32_t* cg = cnt + (long long)bg * nC;
  for (int c = threadIdx.x; c < nC; c += NT)
    if (hist[c]) atomicAdd(&cg[c], hist[c]);
}

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// per scan workgroup (SB buckets): number of pairs and of tiles
__global__ void __launch_bounds__(NT)
k_pair_bsum(const uint32_t* __restrict__ cnt, uint32_t* __restrict__ bsa,
            uint32_t* __restrict__ bsb, int F, int TQ) {
  __shared__ uint32_t sa, sb;
  if (threadIdx.x == 0) { sa = 0; sb = 0; }
  __syncthreads();
  const long long f0 = (long long)blockIdx.x * SB;
  uint32_t a = 0, b = 0;
  for (int t = threadIdx.x; t < SB; t += NT) {
    const long long f = f0 + t;
    if (f < F) {
      const uint32_t n = cnt[f];
      a += n;
      b += (n + (uint32_t)TQ - 1u) / (uint32_t)TQ;
    }
  }
  atomicAdd(&sa, a);
  atomicAdd(&sb, b);
  __syncthreads();
  if (threadIdx.x == 0) { bsa[blockIdx.x] = sa; bsb[blockIdx.x] = sb; }
}

// exclusive prefix sums over the buckets f = bg * nC + c of the bucket
// sizes (list offsets, also the scatter cursors) and of their tile counts;
// each workgroup adds up the totals of the workgroups before it, then scans
// its SB buckets, 16 consecutive ones per thread.  The last workgroup writes
// tot[0] = pairs, tot[1] = tiles.
__global__ void __launch_bounds__(NT)
k_pair_scan(const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ bsa,
            const uint32_t* __restrict__ bsb, uint32_t* __restrict__ loff,
            uint32_t* __restrict__ toff, uint32_t* __restrict__ cur, uint32_t* __restrict__ tot,
            int F, int TQ) {
  static_assert(SB == 16 * NT, "16 buckets per thread");
  __shared__ uint32_t wa[NT / 64], wb[NT / 64], ba, bb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) { ba = 0; bb = 0; }
  __syncthreads();
  {
    uint32_t a = 0, b = 0;
    for (int i = tid; i < (int)blockIdx.x; i += NT) { a += bsa[i]; b += bsb[i]; }
    atomicAdd(&ba, a);
    atomicAdd(&bb, b);
  }
  const long long f0 = (long long)blockIdx.x * SB + 16 * tid;
  uint32_t na[16], ta = 0, tb = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    na[e] = (f0 + e < F) ? cnt[f0 + e] : 0u;
    ta += na[e];
    tb += (na[e] + (uint32_t)TQ - 1u) / (uint32_t)TQ;
  }
  const uint32_t ia = wave_incl_scan_u32(ta, lane), ib = wave_incl_scan_u32(tb, lane);
  if (lane == 63) { wa[w] = ia; wb[w] = ib; }
  __syncthreads();
  uint32_t pa = ba, pb = bb, sa = 0, sb2 = 0;
#pragma unroll
  for (int u = 0; u < NT / 64; ++u) {
    if (u < w) { pa += wa[u]; pb += wb[u]; }
    sa += wa[u];
    sb2 += wb[u];
  }
  pa += ia - ta;
  pb += ib - tb;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (f0 + e < F) {
      loff[f0 + e] = pa;
      cur[f0 + e] = pa;
      toff[f0 + e] = pb;
    }
    pa += na[e];
    pb += (na[e] + (uint32_t)TQ - 1u) / (uint32_t)TQ;
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) { tot[0] = ba + sa; tot[1] = bb + sb2; }
}

// tile t (one thread per tile): {f << 7 | pairs in the tile, first list
// position}, f the bucket holding it = the last bucket whose first tile is
// <= t (buckets without pairs share their first tile with the next one)
__global__ void __launch_bounds__(NT)
k_pair_tiles(const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ loff,
             const uint32_t* __restrict__ toff, const uint32_t* __restrict__ tot,
             uint2* __restrict__ tinfo, int F, int TQ) {
  const uint32_t t = (uint32_t)blockIdx.x * NT + threadIdx.x;
  if (t >= tot[1]) return;
  int lo = 0, hi = F;   // toff[lo] <= t < toff[hi] (toff[F] read as +inf)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (toff[mid] <= t) lo = mid; else hi = mid;
  }
  const uint32_t u = t - toff[lo], n = cnt[lo];
  const uint32_t m = min((uint32_t)TQ, n - u * (uint32_t)TQ);
  tinfo[t] = make_uint2(((uint32_t)lo << 7) | m, loff[lo] + u * (uint32_t)TQ);
}

// list entries (local query << 7 | slot), bucketed by chunk; the order inside
// a bucket depends on atomics and does not affect any result
__global__ void __launch_bounds__(NT)
k_pair_scatter(const int32_t* __restrict__ sel, uint32_t* __restrict__ cur,
               uint32_t* __restrict__ list, int N, int K, int nC, int i0, int qs) {
  extern __shared__ uint32_t lc[];   // [nC]: local count, then next global position
  const int bg = blockIdx.x;
  const int q0 = blockIdx.y * PQ;
  const int qn = min(PQ, qs - q0);
  for (int c = threadIdx.x; c < nC; c += NT) lc[c] = 0;
  __syncthreads();
  const int32_t* sb = sel + ((long long)bg * N + i0 + q0) * K;
  for (int t = threadIdx.x; t < qn * K; t += NT) {
    const int c = sb[t];
    if (c >= 0 && c < nC) atomicAdd(&lc[c], 1u);
  }
  __syncthreads();
  uint32_t* cg = cur + (long long)bg * nC;
  for (int c = threadIdx.x; c < nC; c += NT) {
    const uint32_t n = lc[c];
    if (n) lc[c] = atomicAdd(&cg[c], n);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < qn * K; t += NT) {
    const int c = sb[t];
    if (c >= 0 && c < nC) {
      const uint32_t pos = atomicAdd(&lc[c], 1u);
      list[pos] = ((uint32_t)(q0 + t / K) << 7) | (uint32_t)(t % K);
    }
  }
}

// ---------------------------------------------------------------------------
// window attention + fusion weights

// One workgroup per 128/G consecutive queries of one (batch, KV group): 128
// MFMA rows, each wavefront owning two 16-row blocks, so every K / V^T
// fragment a wavefront reads from LDS feeds two MFMAs.
template <int G>
__global__ void __launch_bounds__(NT, 2)
k_win_fuse(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
           const bf16_t* __restrict__ vt, const float* __restrict__ lamb,
           const bf16_t* __restrict__ part, bf16_t* __restrict__ out, int Hq, int Hkv, int N,
           int W, int K, int nCc, float tau2, int i0, int qs, int nqb, int nbg) {
  constexpr int QA = 128 / G;
  extern __shared__ __align__(16) unsigned char sm[];
  bf16_t* ktile = reinterpret_cast<bf16_t*>(sm);
  bf16_t* vtile = reinterpret_cast<bf16_t*>(sm + KT_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // consecutive query blocks, whose windows overlap, run on one XCD
  const long long wk = xcd_work(blockIdx.x, (long long)nbg * nqb);
  if (wk < 0) return;
  const int blk = (int)wk;
  const int qb = blk % nqb;
  const int bg = blk / nqb;
  const int g = bg % Hkv;
  const long long b = bg / Hkv;
  const int ib0 = i0 + qb * QA;
  const int qcount = min(QA, i0 + qs - ib0);
  const long long hb = b * Hq + (long long)g * G;
  const long long kvbase = bg;

  // row block rb of this wavefront: rows 32 w + 16 rb + (lane & 15) = (query qa, head h)
  const int h = (lane & 15) % G;
  const int lq = lane >> 4;
  // positions fit 32 bits here (the fast path caps N at 2^20)
  bool vcol[2];
  int iq[2], wlo[2];
  bf16x8_t bq[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int qa = (32 * w + 16 * rb + (lane & 15)) / G;
    vcol[rb] = qa < qcount;
    iq[rb] = ib0 + qa;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (vcol[rb]) bq[rb][ks] = ld_bf16x8(q + ((hb + h) * N + iq[rb]) * (long long)D + 32 * ks + 8 * lq);
      else bq[rb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    }
    wlo[rb] = vcol[rb] ? (int)window_start(iq[rb], W, S) : 0;
  }

  // rows past N read row N-1 (masked); V^T is zero there
  auto load_chunk = [&](uint4* r, int c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 16, part = piece % 16;
      const long long t = min((long long)c * S + row, (long long)N - 1);
      r[p] = ld_u4(k + (kvbase * N + t) * D + part * 8);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 8, part = piece % 8;
      r[4 + p] = ld_u4(vt + ((kvbase * nCc + c) * D + row) * (long long)S + part * 8);
    }
  };
  auto store_chunk = [&](const uint4* r) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 16, part = piece % 16;
      st_u4(ktile + row * KSTR + kswz(row, part) * 8, r[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 8, part = piece % 8;
      st_u4(vtile + row * VSTR + part * 8, r[4 + p]);
    }
  };
  f32x4_t acc[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rb][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // running row reference in raw score units (logit = tau2 * raw, base 2) and
  // this lane's part of the row's exp sum relative to it (the four lanes of a
  // row add up at the end)
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  const float mslack = 8.0f / tau2;

  // full: the tile lies inside the window of every row of the workgroup, so
  // no score needs a mask
  auto window_tile = [&](int c, auto full_tag) {
    constexpr bool full = decltype(full_tag)::value;
    f32x4_t s[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int mm = lane & 15;
      const int key = 32 * (kt >> 1) + 8 * (mm >> 2) + 4 * (kt & 1) + (mm & 3);
      s[0][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      s[1][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t kf = ld_bf16x8(ktile + key * KSTR + kswz(key, 4 * ks + lq) * 8);
        s[0][kt] = mfma16(kf, bq[0][ks], s[0][kt]);
        s[1][kt] = mfma16(kf, bq[1][ks], s[1][kt]);
      }
    }
    bf16x8_t pb[2][2];
    float scale[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float x[16];
      float mt = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = s[rb][kt][e];
          if constexpr (!full) {
            const int j = c * S + 32 * (kt >> 1) + 8 * lq + 4 * (kt & 1) + e;
            v = (vcol[rb] && j >= wlo[rb] && j <= iq[rb]) ? v : -INFINITY;
          }
          x[kt * 4 + e] = v;
          mt = fmaxf(mt, v);
        }
      mt = max_x32(max_x16(mt));
      // the row's reference m moves only when the tile's maximum passes it by
      // more than 8 in base-2 logit units (always on the first finite tile):
      // the weights stay below 2^8, and the outputs are rescaled rarely.  A
      // row without a finite score yet keeps m = -inf and weights 0.
      const float mnew = (m[rb] == -INFINITY || mt > m[rb] + mslack) ? mt : m[rb];
      scale[rb] = (mnew == m[rb]) ? 1.0f : fast_exp2((m[rb] - mnew) * tau2);
      const float mneg = (mnew == -INFINITY) ? 0.0f : -mnew * tau2;
      float p[16];
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t) { p[t] = fast_exp2(fmaf(x[t], tau2, mneg)); ps += p[t]; }
      l[rb] = l[rb] * scale[rb] + ps;
      m[rb] = mnew;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float* pp = p + 8 * kb;
        const uint4 u = make_uint4(pack_bf16x2(pp[0], pp[1]), pack_bf16x2(pp[2], pp[3]),
                                   pack_bf16x2(pp[4], pp[5]), pack_bf16x2(pp[6], pp[7]));
        pb[rb][kb] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
    // rescale the outputs only when some row's reference moved
    if (__ballot(scale[0] != 1.0f || scale[1] != 1.0f)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[rb][dt] *= scale[rb];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t vf = ld_bf16x8(vtile + (16 * dt + (lane & 15)) * VSTR + 32 * kb + 8 * lq);
        acc[0][dt] = mfma16(vf, pb[0][kb], acc[0][dt]);
        acc[1][dt] = mfma16(vf, pb[1][kb], acc[1][dt]);
      }
  };

  // Chunk-level fusion (section 3, hierarchical softmax): each row (query,
  // head) mixes its window output with the per-chunk outputs o_c the pair
  // kernel stored for its selected chunks: alpha = softmax over {s_hat_c} U
  // {log Z_swa} (base 2 throughout), out = alpha_swa o_swa + sum_c alpha_c o_c.
  // The chunk part is accumulated first against the row's largest chunk
  // logit m_c: P = sum_c 2^(s_hat_c - m_c) o_c (slot order) and
  // E = sum_c 2^(s_hat_c - m_c); with M = max(m_c, log Z_swa) the output is
  //   (2^(m_c - M) P + 2^(log Z_swa - M) o_swa) / (2^(m_c - M) E + 2^(log Z_swa - M)).
  // So the chunk part does not wait for the window: workgroups of odd work
  // index take row block 0's chunk part before their window tiles, even ones
  // after, which keeps the per-chunk output reads of some workgroups of a CU
  // running while others compute their window.  A row's four lanes (lq)
  // share its weights through this wavefront's part of the LDS, free outside
  // the tile loop.
  float* al = reinterpret_cast<float*>(sm) + (size_t)w * 32 * (K + 1);
  // chunk part of row block rb into pa (with its m_c and E)
  auto chunk_part = [&](int rb, float (&pa)[8][4], float& pmx, float& pse) __attribute__((always_inline)) {
    const int kk = vcol[rb] ? min(K, n_cand(iq[rb], W, S)) : 0;
    const long long qrow = (long long)bg * qs + (iq[rb] - i0);
    float* ar = al + (16 * rb + (lane & 15)) * (K + 1);
    const float* lrow = lamb + qrow * K * G + h;    // slot kx at lrow[kx * G]
    float mx = -INFINITY;
    for (int kx = lq; kx < kk; kx += 4) {
      const float x = lrow[(long long)kx * G];
      ar[kx] = x;
      mx = fmaxf(mx, x);
    }
    mx = max_x32(max_x16(mx));
    float se = 0.0f;
    for (int kx = lq; kx < kk; kx += 4) {
      const float e = fast_exp2(ar[kx] - mx);
      ar[kx] = e;
      se += e;
    }
    pse = sum_x32(sum_x16(se));
    pmx = mx;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // the row's weights, from its four lanes
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) pa[dt][e] = 0.0f;
    // piece 4j + lq of head h's row (16 bytes at element 32 (G j + h) + 8 lq
    // of the pair's block) holds the elements 32j + 4lq + {0..3} (acc block
    // 2j) and 32j + 16 + 4lq + {0..3} (block 2j + 1) of this lane; for G > 1
    // one load instruction reads whole 128-byte lines (the 4 lq lanes of two
    // heads), non-temporal
    const bf16_t* pp = part + qrow * K * G * D + 32 * h + 8 * lq;
    constexpr int RU = 8;                 // slots whose pieces are in flight together
    for (int kx = 0; kx < kk; kx += RU) {
      uint4 u[RU][4];
#pragma unroll
      for (int t = 0; t < RU; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)   // a slot past kk reads slot kk - 1 again, unused
          {  // G = 1 reads half lines per instruction: cached, so the line's other half hits
            const bf16_t* src = pp + (long long)min(kx + t, kk - 1) * G * D + 32 * G * jj;
            u[t][jj] = (G == 1) ? ld_u4(src) : ld_u4_nt(src);
          }
#pragma unroll
      for (int t = 0; t < RU; ++t) {
        if (kx + t < kk) {
          const float wt = ar[kx + t];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t uv[4] = {u[t][jj].x, u[t][jj].y, u[t][jj].z, u[t][jj].w};
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              pa[2 * jj][2 * t2] = fmaf(wt, __uint_as_float(uv[t2] << 16), pa[2 * jj][2 * t2]);
              pa[2 * jj][2 * t2 + 1] =
                  fmaf(wt, __uint_as_float(uv[t2] & 0xffff0000u), pa[2 * jj][2 * t2 + 1]);
              pa[2 * jj + 1][2 * t2] = fmaf(wt, __uint_as_float(uv[2 + t2] << 16), pa[2 * jj + 1][2 * t2]);
              pa[2 * jj + 1][2 * t2 + 1] =
                  fmaf(wt, __uint_as_float(uv[2 + t2] & 0xffff0000u), pa[2 * jj + 1][2 * t2 + 1]);
            }
          }
        }
      }
    }
  };
  // the output rows of block rb: window state (m, l, acc) with the chunk part
  auto finish = [&](int rb, const float (&pa)[8][4], float pmx, float pse) __attribute__((always_inline)) {
    const float lr = sum_x32(sum_x16(l[rb]));      // the row's four lanes
    if (!vcol[rb]) return;
    // every valid row has its own position in the window: lr >= 1
    const float lzr = m[rb] * tau2 + log2f(lr);
    const float M2 = fmaxf(pmx, lzr);
    const float sc = fast_exp2(pmx - M2);          // 0 without selected chunks (pmx = -inf)
    const float es = fast_exp2(lzr - M2);
    const float iz = 1.0f / (sc * pse + es);
    const float cw = sc * iz, ww = es * iz / lr;
    bf16_t* op = out + ((hb + h) * N + iq[rb]) * (long long)D + 4 * lq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = fmaf(cw, pa[dt][e], ww * acc[rb][dt][e]);
      *reinterpret_cast<uint2*>(op + 16 * dt) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  };
  // row block 0's chunk part of a part-first workgroup waits in LDS (past the
  // tiles), lane-interleaved 16-byte pieces: the tile loop needs the registers
  const bool part_first = (wk & 1) != 0;
  float4* p0s = reinterpret_cast<float4*>(sm + KT_BYTES + VT_BYTES) + (size_t)w * 8 * 64 + lane;
  float m0 = -INFINITY, e0 = 0.0f;
  if (part_first) {
    float pa[8][4];
    chunk_part(0, pa, m0, e0);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) p0s[dt * 64] = make_float4(pa[dt][0], pa[dt][1], pa[dt][2], pa[dt][3]);
    __syncthreads();             // the LDS weights are read; the tile loop takes that LDS
  }

  const int cw_lo = (int)(window_start(ib0, W, S) / S);
  const int cw_hi = (ib0 + qcount - 1) / S;
  const int nw = cw_hi - cw_lo + 1;
  // tiles [full_lo, full_hi] lie inside every row's window [window_start(i), i]
  const long long full_lo = (window_start(ib0 + qcount - 1, W, S) + S - 1) / S;
  const long long full_hi = (ib0 + 1) / S - 1;
  // one register buffer: tile idx + 1 is loaded while tile idx is scored
  uint4 ra[8];
  load_chunk(ra, cw_lo);
  store_chunk(ra);
  __syncthreads();
  for (int idx = 0; idx < nw; ++idx) {
    const int c = cw_lo + idx;
    load_chunk(ra, cw_lo + min(idx + 1, nw - 1));
    if (qcount == QA && c >= full_lo && c <= full_hi) window_tile(c, std::true_type{});
    else window_tile(c, std::false_type{});
    __syncthreads();
    store_chunk(ra);             // past the last tile: rewrites the last tile, unused
    __syncthreads();
  }
  if (part_first) {
    float pa[8][4];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 v = p0s[dt * 64];
      pa[dt][0] = v.x; pa[dt][1] = v.y; pa[dt][2] = v.z; pa[dt][3] = v.w;
    }
    finish(0, pa, m0, e0);
  } else {
    float pa[8][4], pm, pe;
    chunk_part(0, pa, pm, pe);
    finish(0, pa, pm, pe);
  }
  {
    float pa[8][4], pm, pe;
    chunk_part(1, pa, pm, pe);
    finish(1, pa, pm, pe);
  }
}

// ---------------------------------------------------------------------------
// per-chunk attention of the bucketed pairs

template <int G, bool QR>
__global__ void __launch_bounds__(NT, 2)
k_pair_attn(const bf16_t* __restrict__ q, const bf16_t* __restrict__ qr,
            const bf16_t* __restrict__ k, const bf16_t* __restrict__ vt,
            const bf16_t* __restrict__ ksum, const float* __restrict__ bsum,
            const uint32_t* __restrict__ list, const uint2* __restrict__ tinfo,
            const uint32_t* __restrict__ tot, float* __restrict__ lamb, bf16_t* __restrict__ part,
            int Hq, int Hkv, int N, int K, int nC, int nCc, float tau2, int i0, int qs) {
  extern __shared__ __align__(16) unsigned char sm[];
  bf16_t* ktile = reinterpret_cast<bf16_t*>(sm);
  bf16_t* vtile = reinterpret_cast<bf16_t*>(sm + KT_BYTES);
  bf16_t* kstile = reinterpret_cast<bf16_t*>(sm + KT_BYTES + VT_BYTES);   // [G + 1][KSS] k'_c, zero row
  __shared__ float bst[G];
  __shared__ uint2 tl[PTPW];
  __shared__ uint4 ostg[4 * 16 * OSTR];   // per wavefront: 16 output rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t T = tot[1];
  const uint32_t t0 = (uint32_t)blockIdx.x * PTPW;
  if (t0 >= T) return;
  const int nt = (int)min((uint32_t)PTPW, T - t0);
  if (tid < nt) tl[tid] = tinfo[t0 + tid];
  if (tid < 16) st_u4(kstile + G * KSS + tid * 8, make_uint4(0, 0, 0, 0));
  __syncthreads();
  const int colr = 16 * w + (lane & 15);
  const int jr = colr / G, h = colr % G;
  const int lq = lane >> 4;

  // list entry of this lane's row in tile u (rows past the tile's pairs repeat
  // its last pair: loads stay valid, results are not stored)
  auto entry = [&](int u) {
    const uint2 ti = tl[min(u, nt - 1)];
    const int mcount = (int)(ti.x & 127u);
    return list[ti.y + min(jr, mcount - 1)];
  };
  auto qrow = [&](uint32_t ent, int u) {
    const int f = (int)(tl[min(u, nt - 1)].x >> 7);
    const int bg = f / nC;
    const int b = bg / Hkv, g = bg - b * Hkv;
    return (((long long)b * Hq + (long long)g * G + h) * N + i0 + (int)(ent >> 7)) * D;
  };
  auto load_q = [&](const bf16_t* src, long long off, bf16x8_t* r) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r[ks] = ld_bf16x8(src + off + 32 * ks + 8 * lq);
  };

  // prefetch: list entries three tiles ahead, query rows two tiles ahead
  uint32_t e0 = entry(0), e1 = entry(1), e2 = entry(2);
  bf16x8_t bq0[4], bq1[4], bq2[4], br0[4], br1[4], br2[4];
  load_q(q, qrow(e0, 0), bq0);
  load_q(q, qrow(e1, 1), bq1);
  if (QR) {
    load_q(qr, qrow(e0, 0), br0);
    load_q(qr, qrow(e1, 1), br1);
  }
  int cur = -1;
  // A operand of the fusion logits: rows 0..G-1 the group's k'_c, the other
  // rows read the zero row G
  const bf16_t* kar = kstile + min(lane & 15, G) * KSS + 8 * lq;
  for (int u = 0; u < nt; ++u) {
    const uint2 ti = tl[u];
    const int f = (int)(ti.x >> 7), mcount = (int)(ti.x & 127u);
    const int bg = f / nC, c = f - bg * nC;
    const uint32_t e3 = entry(u + 3);
    {
      const long long off = qrow(e2, u + 2);
      load_q(q, off, bq2);
      if (QR) load_q(qr, off, br2);
    }
    if (f != cur) {            // stage the chunk's K (swizzled), V^T and the group's k'_c, b'_c
      __syncthreads();
      uint4 r[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int piece = tid + NT * p, row = piece / 16, pt = piece % 16;
        r[p] = ld_u4(k + ((long long)bg * N + (long long)c * S + row) * D + pt * 8);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int piece = tid + NT * p, row = piece / 8, pt = piece % 8;
        r[4 + p] = ld_u4(vt + (((long long)bg * nCc + c) * D + row) * (long long)S + pt * 8);
      }
      const int b = bg / Hkv, g = bg - b * Hkv;
      const long long hs = (long long)b * Hq + (long long)g * G;
      uint4 rk = make_uint4(0, 0, 0, 0);
      if (tid < G * 16) rk = ld_u4(ksum + ((hs + tid / 16) * nC + c) * (long long)D + (tid % 16) * 8);
      float rb = 0.0f;
      if (tid < G) rb = bsum[(hs + tid) * nC + c];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int piece = tid + NT * p, row = piece / 16, pt = piece % 16;
        st_u4(ktile + row * KSTR + kswz(row, pt) * 8, r[p]);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int piece = tid + NT * p, row = piece / 8, pt = piece % 8;
        st_u4(vtile + row * VSTR + pt * 8, r[4 + p]);
      }
      if (tid < G * 16) st_u4(kstile + (tid / 16) * KSS + (tid % 16) * 8, rk);
      if (tid < G) bst[tid] = rb;
      __syncthreads();
      cur = f;
    }
    const bool valid = jr < mcount;
    const int qi = (int)(e0 >> 7), kx = (int)(e0 & 127u);
    const long long prow = ((long long)bg * qs + qi) * K + kx;   // pair index

    // fusion logit of the row (base 2) on the matrix cores: output element
    // (h', row) of k'·q^T is the dot product of head h' with the row's query,
    // and the row's own head h < 4 sits in element h of its lq = 0 lane
    float lam;
    {
      const bf16x8_t* src = QR ? br0 : bq0;
      f32x4_t a5 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a5 = mfma16(ld_bf16x8(kar + 32 * ks), src[ks], a5);
      const float d01 = (h & 1) ? a5[1] : a5[0], d23 = (h & 1) ? a5[3] : a5[2];
      const float dp = (h & 2) ? d23 : d01;
      lam = fmaf(dp, tau2, bst[h] * LOG2E);
    }

    f32x4_t s4[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int mm = lane & 15;
      const int key = 32 * (kt >> 1) + 8 * (mm >> 2) + 4 * (kt & 1) + (mm & 3);
      f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a4 = mfma16(ld_bf16x8(ktile + key * KSTR + kswz(key, 4 * ks + lq) * 8), bq0[ks], a4);
      s4[kt] = a4;
    }
    // every key of a selected chunk is visible: no mask.  The maximum is taken
    // on the raw products (the scale is positive) and scaled once.
    float mr = s4[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mr = fmaxf(mr, s4[kt][e]);
    const float nmt = -max_x32(max_x16(mr)) * tau2;
    float p[16];
    float ps = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[kt * 4 + e] = fast_exp2(fmaf(s4[kt][e], tau2, nmt));
        ps += p[kt * 4 + e];
      }
    ps = sum_x32(sum_x16(ps));
    const float coef = __builtin_amdgcn_rcpf(ps);   // ps >= 1; the weights are rounded to bf16
    bf16x8_t pb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pk[8];
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) pk[t2] = p[(2 * kb + (t2 >> 2)) * 4 + (t2 & 3)] * coef;
      const uint4 uu = make_uint4(pack_bf16x2(pk[0], pk[1]), pack_bf16x2(pk[2], pk[3]),
                                  pack_bf16x2(pk[4], pk[5]), pack_bf16x2(pk[6], pk[7]));
      pb[kb] = __builtin_bit_cast(bf16x8_t, uu);
    }
    f32x4_t acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      acc[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc[dt] = mfma16(ld_bf16x8(vtile + (16 * dt + (lane & 15)) * VSTR + 32 * kb + 8 * lq),
                         pb[kb], acc[dt]);
    }
    {
      // Each lane holds a 64-byte slice of its row (piece 4j + lq holds
      // elements 32j + 4lq + {0..3} and 32j + 16 + 4lq + {0..3}).  The rows go
      // through the wavefront's LDS patch so that every store instruction
      // writes whole 128-byte lines: 8 lanes per line, two rows per 8-lane
      // group.  Whole-line non-temporal stores neither split lines nor push
      // reused query rows and K/V out of the caches.
      uint4* ow = ostg + w * (16 * OSTR);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 uu = make_uint4(pack_bf16x2(acc[2 * j][0], acc[2 * j][1]),
                                    pack_bf16x2(acc[2 * j][2], acc[2 * j][3]),
                                    pack_bf16x2(acc[2 * j + 1][0], acc[2 * j + 1][1]),
                                    pack_bf16x2(acc[2 * j + 1][2], acc[2 * j + 1][3]));
        ow[(lane & 15) * OSTR + 4 * j + lq] = uu;
      }
      if (valid && lq == 0) __builtin_nontemporal_store(lam, lamb + prow * G + h);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      // Stored layout of a pair's G rows (G D elements): piece 4j + lq of
      // head h at element 32 (G j + h) + 8 lq, so that the pieces 4j .. 4j + 3
      // of two neighbouring heads fill one 128-byte line (G = 1: the row in
      // order).  Line ln of this wavefront's 16 rows: 8 lanes, 16 bytes each.
      const int sl = lane & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ln = 8 * i + (lane >> 3);
        int rr, pc, eo;                                     // patch row, piece, element offset
        if constexpr (G == 1) {
          rr = ln >> 1;
          pc = 8 * (ln & 1) + sl;
          eo = 64 * (ln & 1) + 8 * sl;
        } else {
          const int pw = ln / (2 * G), rem = ln % (2 * G);
          const int jj = rem / (G / 2), hp = rem % (G / 2);
          rr = pw * G + 2 * hp + (sl >> 2);
          pc = 4 * jj + (sl & 3);
          eo = 32 * (G * jj + 2 * hp) + 8 * sl;
        }
        const int rp0 = rr - rr % G;                        // first row of the pair
        const uint32_t er = (uint32_t)__shfl((int)e0, rp0); // its list entry
        const int jrr = (16 * w + rp0) / G;
        const long long pr = ((long long)bg * qs + (int)(er >> 7)) * K + (int)(er & 127u);
        const uint4 u = ow[rr * OSTR + pc];
        if (jrr < mcount) st_u4_nt(part + pr * G * D + eo, u);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // patch reads before the next tile's writes
    }
    e0 = e1;
    e1 = e2;
    e2 = e3;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bq0[ks] = bq1[ks];
      bq1[ks] = bq2[ks];
      if (QR) {
        br0[ks] = br1[ks];
        br1[ks] = br2[ks];
      }
    }
  }
}

template <int G>
hipError_t launch_pairs(const HilsShape& s, const void* q, const void* qr, const void* k,
                        const void* vt, const void* ksum, const float* bsum, const int32_t* sel,
                        void* out, const HilsPairBufs& pb, hipStream_t st) {
  constexpr int QA = 128 / G;   // queries per window workgroup
  constexpr int TQ = 64 / G;
  const int F = s.B * s.Hkv * s.nC;
  const float tau2 = (float)(s.tau * 1.4426950408889634);
  const size_t hshm = (size_t)(s.nC > 0 ? s.nC : 1) * 4;
  // window tiles during the tile loop (per wavefront 32 rows of fusion weights
  // outside it), then the part-first workgroups' row block 0 chunk parts
  const size_t wshm = std::max(KT_BYTES + VT_BYTES, (size_t)4 * 32 * (s.K + 1) * 4) +
                      (size_t)4 * 8 * 64 * 16;
  const size_t ashm = KT_BYTES + VT_BYTES + (size_t)(G + 1) * KSS * 2;
  hils_allow_lds((const void*)k_pair_count, hshm);
  hils_allow_lds((const void*)k_pair_scatter, hshm);
  hils_allow_lds((const void*)k_win_fuse<G>, wshm);
  hils_allow_lds((const void*)k_pair_attn<G, false>, ashm);
  hils_allow_lds((const void*)k_pair_attn<G, true>, ashm);
  const bf16_t* qb = (const bf16_t*)q;
  const bf16_t* qrb = (qr == q) ? nullptr : (const bf16_t*)qr;
  const int nsb = (F + SB - 1) / SB;        // scan workgroups
  for (int i0 = 0; i0 < s.N; i0 += pb.qs_max) {
    const int qs = min(pb.qs_max, s.N - i0);
    const int nqb = (qs + QA - 1) / QA;
    if (F > 0) {
      { HilsProfScope ps_("k_pair_lists", st);
        hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)min(1024, (F + NT - 1) / NT)), dim3(NT), 0, st,
                           pb.cnt, (long long)F, 0u);
        hipLaunchKernelGGL(k_pair_count, dim3(s.B * s.Hkv, (qs + PQ - 1) / PQ), dim3(NT), hshm, st,
                           sel, pb.cnt, s.N, s.K, s.nC, i0, qs);
        hipLaunchKernelGGL(k_pair_bsum, dim3(nsb), dim3(NT), 0, st, pb.cnt, pb.bsum, pb.bsum + nsb,
                           F, TQ);
        hipLaunchKernelGGL(k_pair_scan, dim3(nsb), dim3(NT), 0, st, pb.cnt, pb.bsum, pb.bsum + nsb,
                           pb.loff, pb.toff, pb.cur, pb.tot, F, TQ);
        hipLaunchKernelGGL(k_pair_tiles, dim3((unsigned)((hils_pair_tiles_max(s, qs) + NT - 1) / NT)),
                           dim3(NT), 0, st, pb.cnt, pb.loff, pb.toff, pb.tot, pb.tinfo, F, TQ);
        hipLaunchKernelGGL(k_pair_scatter, dim3(s.B * s.Hkv, (qs + PQ - 1) / PQ), dim3(NT), hshm, st,
                           sel, pb.cur, pb.list, s.N, s.K, s.nC, i0, qs); }
    }
    if (F > 0) {
      const long long tmax = hils_pair_tiles_max(s, qs);
      const unsigned grid = (unsigned)((tmax + PTPW - 1) / PTPW);
      { HilsProfScope ps_("k_pair_attn", st);
        auto kf = qrb ? k_pair_attn<G, true> : k_pair_attn<G, false>;
        hipLaunchKernelGGL(kf, dim3(grid), dim3(NT), ashm, st, qb, qrb,
                           (const bf16_t*)k, (const bf16_t*)vt, (const bf16_t*)ksum, bsum, pb.list,
                           pb.tinfo, pb.tot, pb.lam, (bf16_t*)pb.part, s.Hq, s.Hkv, s.N, s.K, s.nC,
                           s.nCc, tau2, i0, qs); }
    }
    // window attention, then the fusion with the slice's per-chunk outputs
    { HilsProfScope ps_("k_win_fuse", st);
      hipLaunchKernelGGL(k_win_fuse<G>, dim3((unsigned)xcd_grid((long long)s.B * s.Hkv * nqb)),
                         dim3(NT), wshm, st, qb, (const bf16_t*)k, (const bf16_t*)vt, pb.lam,
                         (const bf16_t*)pb.part, (bf16_t*)out, s.Hq, s.Hkv, s.N, s.W, s.K, s.nCc,
                         tau2, i0, qs, nqb, s.B * s.Hkv); }
  }
  return hipGetLastError();
}

}  // namespace

long long hils_pair_tiles_max(const HilsShape& s, int qs) {
  const long long TQ = 64 / s.G;
  const long long pairs = (long long)s.B * s.Hkv * qs * s.K;
  return (pairs + TQ - 1) / TQ + (long long)s.B * s.Hkv * s.nC;
}

hipError_t hils_launch_attn_pairs(const HilsShape& s, const void* q, const void* qr, const void* k,
                                  const void* vt, const void* ksum, const float* bsum,
                                  const int32_t* sel, void* out, const HilsPairBufs& pb,
                                  hipStream_t st) {
  switch (s.G) {
    case 1: return launch_pairs<1>(s, q, qr, k, vt, ksum, bsum, sel, out, pb, st);
    case 2: return launch_pairs<2>(s, q, qr, k, vt, ksum, bsum, sel, out, pb, st);
    case 4: return launch_pairs<4>(s, q, qr, k, vt, ksum, bsum, sel, out, pb, st);
  }
  return hipErrorInvalidValue;
}
