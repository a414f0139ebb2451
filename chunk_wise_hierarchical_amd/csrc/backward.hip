// HiLS prefill backward with the top-K selection held fixed.
//
// "Hierarchical Sparse Attention Done Right", section 3: out = sum_c alpha_c
// o_c + alpha_w o_w with alpha = softmax({s_hat_c} U {log Z_swa}); o_c and o_w
// are S-key and window softmax attentions; s_hat_c = tau q_hat.k'_c + b'_c;
// k'_c, b'_c come from the Proposition 3.1 summary softmax of the landmark
// query q'_c over the chunk's keys.  For L = sum(dout * out) and one (query,
// head), with g_t = dout.o_t and gbar = dout.out:
//   d s_hat_t   = alpha_t (g_t - gbar)        d log Z_swa = alpha_w (g_w - gbar)
//   chunk t:  ds_j = alpha_t p_j (dout.v_j - g_t)
//   window:   ds_j = alpha_w p_j (dout.v_j - g_w) + (d log Z_swa) p_j
//   dq += tau sum_j ds_j k_j;  dk_j += tau ds_j q;  dv_j += alpha p_j dout
//   dq_hat += tau sum_t (d s_hat_t) k'_t;  dk'_t += tau (d s_hat_t) q_hat;  db'_t += d s_hat_t
// and through the summary softmax pi = softmax(tau q'.k_j):
//   dpi_j = k_j.dk' + db' (-log pi_j - 1);  dt_j = pi_j (dpi_j - sum pi dpi)
//   dq' = tau sum_j dt_j k_j;  dk_j += tau dt_j q' + pi_j dk'.
//
// Vector-ALU kernels (fp32 inputs and the shapes the matrix-core passes of
// backward_mf.hip do not take), no floating-point atomics, deterministic:
//   k_bwd_lists — per (batch, KV group): for every chunk, the (query, slot)
//                 pairs that selected it, in query order (stable counting
//                 sort; also used by the matrix-core passes);
//   k_bwd_rows  — per (batch, KV group, query): recompute the row's softmax
//                 statistics, write dq (and dq_route) and per-pair / window
//                 statistics (alpha, log-normaliser, g, d s_hat);
//   k_bwd_cols  — per (batch, KV group, chunk): accumulate dk, dv of the
//                 chunk's tokens over the queries that selected the chunk and
//                 the queries whose window holds it, then back-propagate the
//                 chunk's summaries into dlm and dk.  Its summary-only form
//                 follows the matrix-core passes.
#include "fast_common.h"
#include "hils_internal.h"
#include "hils_bwd.h"

namespace {

constexpr int BT = 256;

// 16-byte vector access to a row of T (8 bf16 or 4 fp32 elements)
template <typename T> struct V16;
template <> struct V16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void ld(const bf16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = __uint_as_float(w[t] << 16);
      o[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
    }
  }
};
template <> struct V16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void ld(const float* p, float* o) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
};

// a (fp32, LDS) . row (T, global), d % V16<T>::N == 0
template <typename T>
__device__ __forceinline__ float dot_row(const float* a, const T* row, int d) {
  constexpr int VN = V16<T>::N;
  float acc = 0.0f;
  for (int e = 0; e < d; e += VN) {
    float x[VN];
    V16<T>::ld(row + e, x);
#pragma unroll
    for (int u = 0; u < VN; ++u) acc = fmaf(a[e + u], x[u], acc);
  }
  return acc;
}

// n (a multiple of V16<T>::N, at most 16) elements of a row into registers
template <typename T>
__device__ __forceinline__ void load_slice16(const T* p, int n, float* o) {
  constexpr int VN = V16<T>::N;
#pragma unroll
  for (int u = 0; u < 16; u += VN) {
    if (u < n) V16<T>::ld(p + u, o + u);
    else {
#pragma unroll
      for (int t = 0; t < VN; ++t) o[u + t] = 0.0f;
    }
  }
}

// n (a multiple of V16<T>::N, at most 32) elements of a row into registers
template <typename T>
__device__ __forceinline__ void load_slice(const T* p, int n, float* o) {
  constexpr int VN = V16<T>::N;
#pragma unroll
  for (int u = 0; u < 32; u += VN) {
    if (u < n) V16<T>::ld(p + u, o + u);
    else {
#pragma unroll
      for (int t = 0; t < VN; ++t) o[u + t] = 0.0f;
    }
  }
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_f(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
  for (int u = 1; u < (int)(blockDim.x >> 6); ++u) m = fmaxf(m, red[u]);
  return m;
}
__device__ __forceinline__ double block_max_d(double v, double* red) {
  v = wave_max_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double m = red[0];
  for (int u = 1; u < (int)(blockDim.x >> 6); ++u) m = fmax(m, red[u]);
  return m;
}
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int u = 0; u < (int)(blockDim.x >> 6); ++u) s += red[u];
  return s;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum_f(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
  for (int u = 0; u < (int)(blockDim.x >> 6); ++u) s += red[u];
  return s;
}

// ---------------------------------------------------------------------------
// inverse selection lists: for each chunk c of (b, g), entries (i << 8 | slot)
// at off[c] .. off[c+1], in increasing query order (a stable counting sort).
// With par set, each of the 16 wavefronts takes a contiguous sixteenth of the
// queries: it counts its own entries per chunk ([16][nC] counters in LDS), the
// scan over chunks turns the counts into per-wavefront cursors (wavefront w
// starts after wavefronts 0 .. w-1 within every chunk), and the wavefronts
// scatter their ranges in parallel.  Otherwise one wavefront scatters all
// queries ([nC] counters).  Within a wavefront the queries go in order and a
// query's slots hold distinct chunks, so its LDS atomics, processed in issue
// order, keep the query order.

__global__ void __launch_bounds__(1024)
k_bwd_lists(const int32_t* __restrict__ sel, uint32_t* __restrict__ off, uint32_t* __restrict__ ent,
            int N, int K, int nC, int par) {
  extern __shared__ uint32_t cur[];          // [par ? 16 : 1][nC] counts, then cursors
  __shared__ uint32_t wtot[16];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nw = par ? 16 : 1;
  const int32_t* sg = sel + (long long)bg * N * K;
  uint32_t* og = off + (long long)bg * (nC + 1);
  uint32_t* eg = ent + (long long)bg * N * K;
  for (int c = tid; c < nw * nC; c += 1024) cur[c] = 0;
  __syncthreads();
  // this wavefront's query range (par)
  const int qa = par ? (int)((long long)N * wv / 16) : 0;
  const int qz = par ? (int)((long long)N * (wv + 1) / 16) : 0;
  if (par) {
    uint32_t* cw = cur + (size_t)wv * nC;
    for (long long t = (long long)qa * K + lane; t < (long long)qz * K; t += 64) {
      const int c = sg[t];
      if (c >= 0 && c < nC) atomicAdd(&cw[c], 1u);
    }
  } else {
    for (long long t = tid; t < (long long)N * K; t += 1024) {
      const int c = sg[t];
      if (c >= 0 && c < nC) atomicAdd(&cur[c], 1u);
    }
  }
  __syncthreads();
  // exclusive scan of the per-chunk totals in chunks of 1024
  uint32_t carry = 0;
  for (int base = 0; base < nC; base += 1024) {
    const int c = base + tid;
    uint32_t v = 0u;
    if (c < nC)
      for (int w = 0; w < nw; ++w) v += cur[(size_t)w * nC + c];
    uint32_t x = v;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const uint32_t y = __shfl_up(x, m, 64);
      if (lane >= m) x += y;
    }
    if (lane == 63) wtot[wv] = x;
    __syncthreads();
    uint32_t before = carry;
    for (int u = 0; u < wv; ++u) before += wtot[u];
    uint32_t all = carry;
    for (int u = 0; u < 16; ++u) all += wtot[u];
    __syncthreads();
    if (c < nC) {
      uint32_t e = before + x - v;
      og[c] = e;
      for (int w = 0; w < nw; ++w) {         // cursor of wavefront w in chunk c
        const uint32_t n = cur[(size_t)w * nC + c];
        cur[(size_t)w * nC + c] = e;
        e += n;
      }
    }
    carry = all;
    __syncthreads();
  }
  if (tid == 0) og[nC] = carry;
  __syncthreads();
  if (par || wv == 0) {
    uint32_t* cw = cur + (size_t)(par ? wv : 0) * nC;
    const int i0 = par ? qa : 0, i1 = par ? qz : N;
    for (int i = i0; i < i1; ++i) {
      for (int s2 = lane; s2 < K; s2 += 64) {
        const int c = sg[(long long)i * K + s2];
        if (c >= 0 && c < nC) {
          const uint32_t pos = atomicAdd(&cw[c], 1u);
          eg[pos] = ((uint32_t)i << 8) | (uint32_t)s2;
        }
      }
    }
  }
}

// The same lists built by P workgroups per (batch, KV group), for long
// sequences: sub-range r = 16 p + w (workgroup p, wavefront w) of R = 16 P
// takes queries [N r / R, N (r + 1) / R).  k_bwd_lcount writes every
// sub-range's per-chunk counts to cnt [B*Hkv][R][nC]; k_bwd_lscan turns them
// into the list offsets and, in place, each sub-range's cursors (sub-range r
// starts after sub-ranges 0 .. r-1 within every chunk); k_bwd_lscatter
// scatters each sub-range in query order as above.  Needs 16 nC counters in
// LDS.

__global__ void __launch_bounds__(1024)
k_bwd_lcount(const int32_t* __restrict__ sel, uint32_t* __restrict__ cnt, int N, int K, int nC,
             int P) {
  extern __shared__ uint32_t lc[];           // [16][nC]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long bg = blockIdx.x;
  const int R = 16 * P, r = 16 * (int)blockIdx.y + wv;
  const int32_t* sg = sel + bg * N * (long long)K;
  for (int t = tid; t < 16 * nC; t += 1024) lc[t] = 0u;
  __syncthreads();
  const long long qa = (long long)N * r / R, qz = (long long)N * (r + 1) / R;
  uint32_t* cw = lc + (size_t)wv * nC;
  for (long long t = qa * K + lane; t < qz * K; t += 64) {
    const int c = sg[t];
    if (c >= 0 && c < nC) atomicAdd(&cw[c], 1u);
  }
  __syncthreads();
  uint32_t* cg = cnt + (bg * R + 16 * (long long)blockIdx.y) * nC;
  for (int t = tid; t < 16 * nC; t += 1024) cg[t] = lc[t];
}

__global__ void __launch_bounds__(1024)
k_bwd_lscan(uint32_t* __restrict__ cnt, uint32_t* __restrict__ off, int nC, int R) {
  __shared__ uint32_t wtot[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long bg = blockIdx.x;
  uint32_t* cg = cnt + bg * R * (long long)nC;
  uint32_t* og = off + bg * (long long)(nC + 1);
  uint32_t carry = 0;
  for (int base = 0; base < nC; base += 1024) {
    const int c = base + tid;
    uint32_t v = 0u;
    if (c < nC)
      for (int r = 0; r < R; ++r) v += cg[(size_t)r * nC + c];
    uint32_t x = v;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const uint32_t y = __shfl_up(x, m, 64);
      if (lane >= m) x += y;
    }
    if (lane == 63) wtot[wv] = x;
    __syncthreads();
    uint32_t before = carry;
    for (int u = 0; u < wv; ++u) before += wtot[u];
    uint32_t all = carry;
    for (int u = 0; u < 16; ++u) all += wtot[u];
    __syncthreads();
    if (c < nC) {
      uint32_t e = before + x - v;
      og[c] = e;
      for (int r = 0; r < R; ++r) {          // cursor of sub-range r in chunk c
        const uint32_t n = cg[(size_t)r * nC + c];
        cg[(size_t)r * nC + c] = e;
        e += n;
      }
    }
    carry = all;
    __syncthreads();
  }
  if (tid == 0) og[nC] = carry;
}

__global__ void __launch_bounds__(1024)
k_bwd_lscatter(const int32_t* __restrict__ sel, const uint32_t* __restrict__ cnt,
               uint32_t* __restrict__ ent, int N, int K, int nC, int P) {
  extern __shared__ uint32_t lc[];           // [16][nC] cursors
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long bg = blockIdx.x;
  const int R = 16 * P, r = 16 * (int)blockIdx.y + wv;
  const int32_t* sg = sel + bg * N * (long long)K;
  uint32_t* eg = ent + bg * N * (long long)K;
  const uint32_t* cg = cnt + (bg * R + 16 * (long long)blockIdx.y) * nC;
  for (int t = tid; t < 16 * nC; t += 1024) lc[t] = cg[t];
  __syncthreads();
  uint32_t* cw = lc + (size_t)wv * nC;
  const int qa = (int)((long long)N * r / R), qz = (int)((long long)N * (r + 1) / R);
  for (int i = qa; i < qz; ++i) {
    for (int s2 = lane; s2 < K; s2 += 64) {
      const int c = sg[(long long)i * K + s2];
      if (c >= 0 && c < nC) {
        const uint32_t pos = atomicAdd(&cw[c], 1u);
        eg[pos] = ((uint32_t)i << 8) | (uint32_t)s2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// per query row: statistics and dq

template <typename T>
__global__ void __launch_bounds__(BT)
k_bwd_rows(const T* __restrict__ q, const T* __restrict__ qr, const T* __restrict__ k,
           const T* __restrict__ v, const T* __restrict__ ksum, const float* __restrict__ bsum,
           const T* __restrict__ dout, const int32_t* __restrict__ sel, float* __restrict__ dq,
           float* __restrict__ dqr, float* __restrict__ pstat, float* __restrict__ wstat, int Hq,
           int Hkv, int G, int N, int d, int S, int W, int K, int nC, float tau, int route_sep) {
  extern __shared__ __align__(16) float smr[];
  const int tid = threadIdx.x;
  const long long row = blockIdx.x;                  // (b, g, i)
  const int i = (int)(row % N);
  const long long bg = row / N;
  const int g = (int)(bg % Hkv);
  const long long b = bg / Hkv;
  const long long hb = b * Hq + (long long)g * G;    // first query head of the group
  const int w0 = (int)window_start(i, W, S);
  const int L = i - w0 + 1;
  const int Lp = (L + 3) & ~3;
  float* qs = smr;                                   // [G][d]
  float* qh = qs + G * d;                            // [G][d]
  float* go = qh + G * d;                            // [G][d]
  float* acc = go + G * d;                           // [G][d] dq accumulator
  float* wp = acc + G * d;                           // [G][Lp] window probabilities
  float* wu = wp + G * Lp;                           // [G][Lp] dout.v_j on the window
  float* cs = wu + G * Lp;                           // [G][S]  chunk p_j (u_j - g_t)
  float* cu = cs + G * S;                            // [G][S]
  float* st = cu + G * S;                            // [K][G][4] alpha, lse, g, dlam per slot
  float* sw = st + K * G * 4;                        // [G][4]
  float* red = sw + G * 4;                           // [4]
  __shared__ int ssel[128];
  __shared__ int sorg[128];                          // slot of each valid selection
  __shared__ int skk;

  for (int t = tid; t < G * d; t += BT) {
    const int r = t / d, e = t - r * d;
    const long long o = ((hb + r) * N + i) * (long long)d + e;
    qs[t] = Elt<T>::ld(q + o);
    qh[t] = Elt<T>::ld(qr + o);
    go[t] = Elt<T>::ld(dout + o);
    acc[t] = 0.0f;
  }
  if (tid == 0) {
    int kk = 0;
    for (int t = 0; t < K; ++t) {
      const int c = sel[row * K + t];
      if (c >= 0 && c < nC) {
        sorg[kk] = t;
        ssel[kk++] = c;
      }
    }
    skk = kk;
  }
  __syncthreads();
  const int kk = skk;
  const T* kb = k + bg * (long long)N * d;
  const T* vb = v + bg * (long long)N * d;

  // chunk scores s_hat_t (routing query) per (slot, head)
  for (int t = tid; t < kk * G; t += BT) {
    const int s2 = t / G, r = t - s2 * G, c = ssel[s2];
    const T* kp = ksum + ((hb + r) * nC + c) * (long long)d;
    const float a = dot_row<T>(qh + r * d, kp, d);
    st[(s2 * G + r) * 4 + 0] = fmaf(tau, a, bsum[(hb + r) * nC + c]);
  }
  // window logits and dout.v_j
  for (int t = tid; t < G * L; t += BT) {
    const int r = t / L, j = t - r * L;
    const T* kr = kb + (long long)(w0 + j) * d;
    const T* vr = vb + (long long)(w0 + j) * d;
    wp[r * Lp + j] = tau * dot_row<T>(qs + r * d, kr, d);
    wu[r * Lp + j] = dot_row<T>(go + r * d, vr, d);
  }
  __syncthreads();
  // per head: window log-mass, probabilities, g_w; fusion weights
  for (int r = 0; r < G; ++r) {
    float m = -INFINITY;
    for (int j = tid; j < L; j += BT) m = fmaxf(m, wp[r * Lp + j]);
    m = block_max(m, red);
    float z = 0.0f;
    for (int j = tid; j < L; j += BT) z += __expf(wp[r * Lp + j] - m);
    z = block_sum(z, red);
    const float lse = m + __logf(z);
    float gw = 0.0f;
    for (int j = tid; j < L; j += BT) {
      const float p = __expf(wp[r * Lp + j] - lse);
      wp[r * Lp + j] = p;
      gw = fmaf(p, wu[r * Lp + j], gw);
    }
    gw = block_sum(gw, red);
    if (tid == 0) {
      float M = lse;
      for (int s2 = 0; s2 < kk; ++s2) M = fmaxf(M, st[(s2 * G + r) * 4]);
      float Z = __expf(lse - M);
      for (int s2 = 0; s2 < kk; ++s2) Z += __expf(st[(s2 * G + r) * 4] - M);
      for (int s2 = 0; s2 < kk; ++s2) st[(s2 * G + r) * 4] = __expf(st[(s2 * G + r) * 4] - M) / Z;
      sw[r * 4 + 0] = __expf(lse - M) / Z;
      sw[r * 4 + 1] = lse;
      sw[r * 4 + 2] = gw;
    }
    __syncthreads();
  }
  // selected chunks: p, dout.v_j, g_t; dq += tau alpha_t sum_j p_j (u_j - g_t) k_j
  for (int s2 = 0; s2 < kk; ++s2) {
    const int c = ssel[s2];
    const T* kc = kb + (long long)c * S * d;
    const T* vc = vb + (long long)c * S * d;
    for (int t = tid; t < G * S; t += BT) {
      const int r = t / S, j = t - r * S;
      cs[t] = tau * dot_row<T>(qs + r * d, kc + (long long)j * d, d);
      cu[t] = dot_row<T>(go + r * d, vc + (long long)j * d, d);
    }
    __syncthreads();
    for (int r = 0; r < G; ++r) {
      float m = -INFINITY;
      for (int j = tid; j < S; j += BT) m = fmaxf(m, cs[r * S + j]);
      m = block_max(m, red);
      float z = 0.0f;
      for (int j = tid; j < S; j += BT) z += __expf(cs[r * S + j] - m);
      z = block_sum(z, red);
      const float lse = m + __logf(z);
      float gt = 0.0f;
      for (int j = tid; j < S; j += BT) gt = fmaf(__expf(cs[r * S + j] - lse), cu[r * S + j], gt);
      gt = block_sum(gt, red);
      for (int j = tid; j < S; j += BT) {
        const float p = __expf(cs[r * S + j] - lse);
        cs[r * S + j] = p * (cu[r * S + j] - gt);
      }
      if (tid == 0) {
        st[(s2 * G + r) * 4 + 1] = lse;
        st[(s2 * G + r) * 4 + 2] = gt;
      }
      __syncthreads();
    }
    for (int t = tid; t < G * d; t += BT) {
      const int r = t / d, e = t - r * d;
      float a = 0.0f;
      for (int j = 0; j < S; ++j) a = fmaf(cs[r * S + j], Elt<T>::ld(kc + (long long)j * d + e), a);
      acc[t] = fmaf(tau * st[(s2 * G + r) * 4], a, acc[t]);
    }
    __syncthreads();
  }
  // gbar, d s_hat, window gradient
  if (tid < G) {
    const int r = tid;
    float gbar = sw[r * 4] * sw[r * 4 + 2];
    for (int s2 = 0; s2 < kk; ++s2) gbar = fmaf(st[(s2 * G + r) * 4], st[(s2 * G + r) * 4 + 2], gbar);
    for (int s2 = 0; s2 < kk; ++s2)
      st[(s2 * G + r) * 4 + 3] = st[(s2 * G + r) * 4] * (st[(s2 * G + r) * 4 + 2] - gbar);
    sw[r * 4 + 3] = sw[r * 4] * (sw[r * 4 + 2] - gbar);
  }
  __syncthreads();
  for (int t = tid; t < G * L; t += BT) {
    const int r = t / L, j = t - r * L;
    const float p = wp[r * Lp + j];
    wu[r * Lp + j] = sw[r * 4] * p * (wu[r * Lp + j] - sw[r * 4 + 2]) + sw[r * 4 + 3] * p;
  }
  __syncthreads();
  for (int t = tid; t < G * d; t += BT) {
    const int r = t / d, e = t - r * d;
    float a = 0.0f;
    for (int j = 0; j < L; ++j) a = fmaf(wu[r * Lp + j], Elt<T>::ld(kb + (long long)(w0 + j) * d + e), a);
    float dqv = fmaf(tau, a, acc[t]);
    // routing query: tau sum_t d s_hat_t k'_t
    float dh = 0.0f;
    for (int s2 = 0; s2 < kk; ++s2)
      dh = fmaf(st[(s2 * G + r) * 4 + 3], Elt<T>::ld(ksum + ((hb + r) * nC + ssel[s2]) * (long long)d + e), dh);
    dh *= tau;
    const long long o = ((hb + r) * N + i) * (long long)d + e;
    if (route_sep) {
      dq[o] = dqv;
      dqr[o] = dh;
    } else {
      dq[o] = dqv + dh;
    }
  }
  // statistics for the column pass, per selection slot (the column pass finds
  // a pair's statistics by its slot)
  for (int t = tid; t < kk * G * 4; t += BT) {
    const int s2 = t / (G * 4);
    pstat[(row * K + sorg[s2]) * G * 4 + (t - s2 * G * 4)] = st[t];
  }
  for (int t = tid; t < G * 4; t += BT) {
    const int r = t / 4, f = t - r * 4;
    wstat[((hb + r) * N + i) * 4 + f] = sw[t];
  }
}

// ---------------------------------------------------------------------------
// per query row, all attended keys at once (used when their logits fit LDS):
// the same statistics and dq as k_bwd_rows, with the work spread so that no
// phase waits on a block-wide reduction per chunk:
//   1. every attended key's logit and dout.v (chunk keys in slot order, then
//      the window), one (key, head) per thread;
//   2. softmax statistics, one wavefront per (slot, head) and per window head;
//   3. fusion weights per head; 4. each key's dq weight;
//   5. dq = sum over keys of weight x k_j: thread (head, 16-byte group, key
//      subset) with vector loads of the key rows, subsets summed in LDS.
template <typename T>
__global__ void __launch_bounds__(BT)
k_bwd_rows2(const T* __restrict__ q, const T* __restrict__ qr, const T* __restrict__ k,
            const T* __restrict__ v, const T* __restrict__ ksum, const float* __restrict__ bsum,
            const T* __restrict__ dout, const int32_t* __restrict__ sel, float* __restrict__ dq,
            float* __restrict__ dqr, float* __restrict__ pstat, float* __restrict__ wstat, int Hq,
            int Hkv, int G, int N, int d, int S, int W, int K, int nC, float tau, int route_sep) {
  extern __shared__ __align__(16) float smr[];
  constexpr int VN = V16<T>::N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long row = blockIdx.x;                  // (b, g, i)
  const int i = (int)(row % N);
  const long long bg = row / N;
  const int g = (int)(bg % Hkv);
  const long long b = bg / Hkv;
  const long long hb = b * Hq + (long long)g * G;
  const int w0 = (int)window_start(i, W, S);
  const int L = i - w0 + 1;
  const int LW = W + S - 1;                          // longest window
  const int NCK = K * S;                             // chunk key columns
  const int RL = NCK + ((LW + 3) & ~3);              // columns per head
  float* qs = smr;                                   // [G][d]
  float* qh = qs + G * d;                            // [G][d]
  float* go = qh + G * d;                            // [G][d]
  float* lw = go + G * d;                            // [G][RL] logits -> weights
  float* du = lw + G * RL;                           // [G][RL] dout.v_j
  float* st = du + G * RL;                           // [K][G][4] alpha, lse, g, d s_hat
  float* sw = st + K * G * 4;                        // [G][4] alpha_w, lse_w, g_w, d log Z
  float* dqp = sw + G * 4;                           // [BT * VN] dq partials by key subset
  __shared__ int ssel[128];
  __shared__ int sorg[128];                          // slot of each valid selection
  __shared__ int skk;

  for (int t = tid; t < G * d; t += BT) {
    const int r = t / d, e = t - r * d;
    const long long o = ((hb + r) * N + i) * (long long)d + e;
    qs[t] = Elt<T>::ld(q + o);
    qh[t] = Elt<T>::ld(qr + o);
    go[t] = Elt<T>::ld(dout + o);
  }
  if (tid == 0) {
    int kk = 0;
    for (int t = 0; t < K; ++t) {
      const int c = sel[row * K + t];
      if (c >= 0 && c < nC) {
        sorg[kk] = t;
        ssel[kk++] = c;
      }
    }
    skk = kk;
  }
  __syncthreads();
  const int kk = skk;
  const int nk = kk * S + L;                         // attended keys
  const T* kb = k + bg * (long long)N * d;
  const T* vb = v + bg * (long long)N * d;
  // key f: chunk key (slot f / S, offset f % S) or window key f - kk S
  auto key_pos = [&](int f) -> long long {
    return (f < kk * S) ? (long long)ssel[f / S] * S + (f % S) : (long long)(w0 + f - kk * S);
  };
  auto key_col = [&](int f) { return (f < kk * S) ? f : NCK + (f - kk * S); };

  // 1. chunk scores s_hat (routing query) and every key's logit and dout.v
  for (int t = tid; t < kk * G; t += BT) {
    const int s2 = t / G, r = t - s2 * G, c = ssel[s2];
    const T* kp = ksum + ((hb + r) * nC + c) * (long long)d;
    st[(s2 * G + r) * 4 + 0] = fmaf(tau, dot_row<T>(qh + r * d, kp, d), bsum[(hb + r) * nC + c]);
  }
  // four lanes per (key, head): each load instruction reads 64 contiguous bytes
  // of a key row (the quad's four 16-byte pieces), the quad's partial dots
  // meet by DPP
  {
    const int l4 = tid & 3;
    for (int t = tid >> 2; t < nk * G; t += BT / 4) {
      const int f = t / G, r = t - f * G;
      const long long pos = key_pos(f);
      const T* kr = kb + pos * d;
      const T* vr = vb + pos * d;
      const float* qq = qs + r * d;
      const float* gg = go + r * d;
      float a = 0.0f, u2 = 0.0f;
      for (int e = VN * l4; e < d; e += 4 * VN) {
        float kv[VN], vv[VN];
        V16<T>::ld(kr + e, kv);
        V16<T>::ld(vr + e, vv);
#pragma unroll
        for (int u = 0; u < VN; ++u) {
          a = fmaf(qq[e + u], kv[u], a);
          u2 = fmaf(gg[e + u], vv[u], u2);
        }
      }
      a += fastp::xshfl_f(a, 1);
      u2 += fastp::xshfl_f(u2, 1);
      a += fastp::xshfl_f(a, 2);
      u2 += fastp::xshfl_f(u2, 2);
      if (l4 == 0) {
        const int col = key_col(f);
        lw[r * RL + col] = tau * a;
        du[r * RL + col] = u2;
      }
    }
  }
  __syncthreads();
  // 2. softmax statistics: items 0 .. G-1 are the window heads, then (slot, head)
  for (int it = wv; it < G + kk * G; it += BT / 64) {
    if (it < G) {
      const int r = it;
      float* x = lw + r * RL + NCK;
      const float* u = du + r * RL + NCK;
      float m = -INFINITY;
      for (int j = lane; j < L; j += 64) m = fmaxf(m, x[j]);
      m = wave_max_f(m);
      float z = 0.0f;
      for (int j = lane; j < L; j += 64) z += __expf(x[j] - m);
      z = wave_sum_f(z);
      const float lse = m + __logf(z);
      float gw = 0.0f;
      for (int j = lane; j < L; j += 64) {
        const float p = __expf(x[j] - lse);
        x[j] = p;
        gw = fmaf(p, u[j], gw);
      }
      gw = wave_sum_f(gw);
      if (lane == 0) { sw[r * 4 + 1] = lse; sw[r * 4 + 2] = gw; }
    } else {
      const int s2 = (it - G) / G, r = (it - G) - s2 * G;
      float* x = lw + r * RL + s2 * S;
      const float* u = du + r * RL + s2 * S;
      const float xv = (lane < S) ? x[lane] : -INFINITY;
      const float m = wave_max_f(xv);
      const float z = wave_sum_f((lane < S) ? __expf(xv - m) : 0.0f);
      const float lse = m + __logf(z);
      const float p = (lane < S) ? __expf(xv - lse) : 0.0f;
      const float uv = (lane < S) ? u[lane] : 0.0f;
      const float gt = wave_sum_f(p * uv);
      if (lane < S) x[lane] = p * (uv - gt);
      if (lane == 0) { st[(s2 * G + r) * 4 + 1] = lse; st[(s2 * G + r) * 4 + 2] = gt; }
    }
  }
  __syncthreads();
  // 3. fusion weights, gbar, d s_hat and d log Z_swa per head
  if (tid < G) {
    const int r = tid;
    const float lse = sw[r * 4 + 1];
    float M = lse;
    for (int s2 = 0; s2 < kk; ++s2) M = fmaxf(M, st[(s2 * G + r) * 4]);
    float Z = __expf(lse - M);
    for (int s2 = 0; s2 < kk; ++s2) Z += __expf(st[(s2 * G + r) * 4] - M);
    for (int s2 = 0; s2 < kk; ++s2) st[(s2 * G + r) * 4] = __expf(st[(s2 * G + r) * 4] - M) / Z;
    sw[r * 4 + 0] = __expf(lse - M) / Z;
    float gbar = sw[r * 4] * sw[r * 4 + 2];
    for (int s2 = 0; s2 < kk; ++s2) gbar = fmaf(st[(s2 * G + r) * 4], st[(s2 * G + r) * 4 + 2], gbar);
    for (int s2 = 0; s2 < kk; ++s2)
      st[(s2 * G + r) * 4 + 3] = st[(s2 * G + r) * 4] * (st[(s2 * G + r) * 4 + 2] - gbar);
    sw[r * 4 + 3] = sw[r * 4] * (sw[r * 4 + 2] - gbar);
  }
  __syncthreads();
  // 4. dq weight of every key: tau alpha_t p_j (u_j - g_t) on a chunk,
  //    tau (alpha_w p_j (u_j - g_w) + d log Z_swa p_j) on the window
  for (int t = tid; t < nk * G; t += BT) {
    const int f = t / G, r = t - f * G;
    const int col = key_col(f);
    float* x = lw + r * RL + col;
    if (f < kk * S) {
      *x = tau * st[((f / S) * G + r) * 4] * *x;
    } else {
      const float p = *x;
      *x = tau * (sw[r * 4] * p * (du[r * RL + col] - sw[r * 4 + 2]) + sw[r * 4 + 3] * p);
    }
  }
  __syncthreads();
  // 5. dq: thread (head r, 16-byte group eg, key subset sub)
  const int ngh = d / VN, ngr = G * ngh, nsub = BT / ngr;
  {
    const int grp = tid % ngr, sub = tid / ngr;
    const int r = grp / ngh, eg = grp - r * ngh;
    float a[VN];
#pragma unroll
    for (int u = 0; u < VN; ++u) a[u] = 0.0f;
    if (sub < nsub) {
      for (int f = sub; f < nk; f += nsub) {
        const float wgt = lw[r * RL + key_col(f)];
        float kv[VN];
        V16<T>::ld(kb + key_pos(f) * d + eg * VN, kv);
#pragma unroll
        for (int u = 0; u < VN; ++u) a[u] = fmaf(wgt, kv[u], a[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < VN; ++u) dqp[tid * VN + u] = a[u];
  }
  __syncthreads();
  for (int t = tid; t < G * d; t += BT) {
    const int r = t / d, e = t - r * d;
    const int grp = r * ngh + e / VN, u = e % VN;
    float dqv = 0.0f;
    for (int sub = 0; sub < nsub; ++sub) dqv += dqp[(sub * ngr + grp) * VN + u];
    // routing query: tau sum_t d s_hat_t k'_t
    float dh = 0.0f;
    for (int s2 = 0; s2 < kk; ++s2)
      dh = fmaf(st[(s2 * G + r) * 4 + 3], Elt<T>::ld(ksum + ((hb + r) * nC + ssel[s2]) * (long long)d + e), dh);
    dh *= tau;
    const long long o = ((hb + r) * N + i) * (long long)d + e;
    if (route_sep) {
      dq[o] = dqv;
      dqr[o] = dh;
    } else {
      dq[o] = dqv + dh;
    }
  }
  // statistics for the column pass (window probabilities are recomputed
  // there), per selection slot (the column pass finds a pair's statistics by
  // its slot)
  for (int t = tid; t < kk * G * 4; t += BT) {
    const int s2 = t / (G * 4);
    pstat[(row * K + sorg[s2]) * G * 4 + (t - s2 * G * 4)] = st[t];
  }
  for (int t = tid; t < G * 4; t += BT) {
    const int r = t / 4, f = t - r * 4;
    wstat[((hb + r) * N + i) * 4 + f] = sw[t];
  }
}

size_t bwd_rows2_lds(const HilsShape& s) {
  const int LW = s.W + s.S - 1;
  const size_t RL = (size_t)s.K * s.S + ((LW + 3) & ~3);
  const int vn = (s.dtype == 0) ? 8 : 4;
  return sizeof(float) * (3 * (size_t)s.G * s.d + 2 * (size_t)s.G * RL + (size_t)s.K * s.G * 4 +
                          (size_t)s.G * 4 + (size_t)BT * vn);
}

// ---------------------------------------------------------------------------
// per chunk: dk, dv of its tokens; summary backward
//
// 512 threads: thread (token jt = tid / 8, eighth qd = tid % 8) owns d/8
// elements of the token's k, v, dk, dv.  Contributions (query, head) are
// described in LDS in batches (query, head, alpha, log-normaliser, g, and the
// window term), and the next contribution's q and dout slices are loaded while
// the current one is applied.

constexpr int CT = 512;
constexpr int CBATCH = 512;                          // contributions described per batch
constexpr int CE = 16;                               // elements per thread (d <= 128)
// contributions whose q, dout and routing-query rows are staged in LDS
// together (two buffers): 48 KB for d = 128 in either precision
template <typename T> struct ColStage { static constexpr int NB = (sizeof(T) == 2) ? 32 : 16; };

// bytes of the column kernel's staging area (also the summary backward's
// scratch of one d-row of doubles per wavefront, used after the contributions)
// (the summary-only variant stages no rows)
template <typename T, bool SUMONLY>
__host__ __device__ inline size_t col_stage_bytes(int d, int S) {
  (void)S;
  const size_t st = SUMONLY ? 0 : (size_t)2 * 3 * ColStage<T>::NB * d * sizeof(T);
  const size_t sc = (size_t)(CT / 64) * d * sizeof(double);
  return ((st > sc ? st : sc) + 15) & ~(size_t)15;
}

// (the summary-only variant at two workgroups per CU: its row reads are
// latency-bound, and it fits 128 registers)
template <typename T, bool SUMONLY, int GT = 0>
__global__ void __launch_bounds__(CT, SUMONLY ? 4 : 1)
k_bwd_cols(const T* __restrict__ q, const T* __restrict__ qr, const T* __restrict__ k,
           const T* __restrict__ v, const T* __restrict__ lm, const T* __restrict__ dout,
           const uint32_t* __restrict__ off, const uint32_t* __restrict__ ent,
           const float* __restrict__ pstat, const float* __restrict__ wstat, float* __restrict__ dk,
           float* __restrict__ dv, float* __restrict__ dlm, int Hq, int Hkv, int G, int N, int d,
           int S, int W, int K, int nC, int nCc, float tau, int mode) {
  extern __shared__ __align__(16) float smc[];
  const int tid = threadIdx.x;
  // chunk-major order (c, b, g): a chunk's work (its selections) depends on
  // its position and on the routing, and neighbouring chunks of one sequence
  // tend to be alike; consecutive workgroups take one chunk of every sequence
  // and KV group, so heavy chunks spread over the chip instead of arriving
  // together on a few CUs.
  const long long blk = blockIdx.x;
  const long long nbg = gridDim.x / nCc;             // B * Hkv
  const int c = (int)(blk / nbg);
  const long long bg = blk % nbg;
  const int g = (int)(bg % Hkv);
  const long long b = bg / Hkv;
  const long long hb = b * Hq + (long long)g * G;
  const int j0 = c * S;
  const int jn = min(S, N - j0);                     // tokens of this chunk
  const int DQ = d / 8;                              // elements per thread
  const int jt = tid >> 3, qd = tid & 7;
  const bool act = jt < jn;
  const int e0 = qd * DQ;
  constexpr int NB = ColStage<T>::NB;
  // staging: [2 buffers][q, dout, routing query][NB][d] T; after the
  // contributions the same bytes hold the [CT / 64][d] double column sums.
  // dk' and db' of the chunk's summaries accumulate in double: their
  // contributions (one per selecting query and head) cancel, and the
  // summary backward below subtracts nearly equal terms.
  T* stg = reinterpret_cast<T*>(smc);
  double* tmp = reinterpret_cast<double*>(smc);
  double* dks = reinterpret_cast<double*>(reinterpret_cast<char*>(smc) + col_stage_bytes<T, SUMONLY>(d, S));
  double* dbs = dks + G * d;                         // [G]
  double* redd = dbs + G;                            // [8]
  float* red = reinterpret_cast<float*>(redd + 8);   // [8]
  int* di = reinterpret_cast<int*>(red + 8);         // [CBATCH] query << 4 | head, window flag << 31
  float* dsx = reinterpret_cast<float*>(di + CBATCH);   // [CBATCH][4] alpha, lse, g, window term
  int* dwl = reinterpret_cast<int*>(dsx + 4 * CBATCH);  // [CBATCH] window contributions: first
                                                         // token of the window, minus j0
  const T* kb = k + (bg * (long long)N + j0) * d;
  const T* vb = v + (bg * (long long)N + j0) * d;

  float kj[CE], vj[CE], dkj[CE], dvj[CE];
  const int jr = act ? jt : 0;                       // inactive tokens read row 0, zeroed
  // (the summary-only variant needs K only after its contributions)
  auto load_kv = [&]() __attribute__((always_inline)) {
    load_slice16<T>(kb + (long long)jr * d + e0, DQ, kj);
    if (!SUMONLY) load_slice16<T>(vb + (long long)jr * d + e0, DQ, vj);
#pragma unroll
    for (int u = 0; u < CE; ++u) {
      if (!act) { kj[u] = 0.0f; vj[u] = 0.0f; }
    }
  };
  if (!SUMONLY) load_kv();
#pragma unroll
  for (int u = 0; u < CE; ++u) {
    dkj[u] = 0.0f;
    dvj[u] = 0.0f;
  }
  for (int t = tid; t < G * d + G; t += CT) dks[t] = 0.0;
  // dk' and db' of the chunk's summaries: thread t takes element ea = t % 128
  // of the selecting contributions u with u % 4 == t / 128 (every wavefront a
  // quarter of them), in registers; the four quarters meet in dks / dbs after
  // the contributions
  const int ea = tid & 127, eq4 = tid >> 7;
  double dka[8], dba[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) { dka[rr] = 0.0; dba[rr] = 0.0; }
  // summary-only variant: wavefront w takes contributions 64 w .. 64 w + 63 of
  // each batch, lane the elements 2 lane, 2 lane + 1; the eight wavefronts'
  // sums meet in dks / dbs in order after the contributions
  const int wvs = tid >> 6, el = 2 * (tid & 63);
  double sa[8][2], sb[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) { sa[rr][0] = 0.0; sa[rr][1] = 0.0; sb[rr] = 0.0; }
  // With GT > 0 (the summary-only variant follows the matrix-core passes, so
  // d is 64 or 128) a row is read as PR = d / 8 pieces of 16 bytes: lane
  // (rq, pc) = (lane / PR, lane % PR) takes elements 8 pc .. 8 pc + 7 of rows
  // RPI j + rq (RPI = 64 / PR) of its wavefront's 64, whose head (RPI j + rq)
  // % GT is one of NHW per lane (slot j % NHW)
  constexpr int NHW = GT == 8 ? 2 : 1;
  const int PR = d / 8, RPI = 64 / PR;
  const int rq = (tid & 63) / PR, pc = (tid & 63) % PR;
  double sw[NHW][8], sbw[NHW];
#pragma unroll
  for (int h2 = 0; h2 < NHW; ++h2) {
    sbw[h2] = 0.0;
#pragma unroll
    for (int x = 0; x < 8; ++x) sw[h2][x] = 0.0;
  }

  const bool summ = c < nC;
  const uint32_t p0 = summ ? off[bg * (nC + 1) + c] : 0u;
  const uint32_t p1 = summ ? off[bg * (nC + 1) + c + 1] : 0u;
  const long long nsel = (long long)(p1 - p0) * G;                 // (pair, head) contributions
  const int i1 = min(N, (c + 1) * S + W - 1);
  // summaries only (dk, dv of the contributions come from the matrix-core
  // column pass): the selecting contributions' d s_hat and q_hat alone
  const long long nwin = SUMONLY ? 0 : (long long)(i1 - j0) * G;  // window (query, head)
  const uint32_t* eg = ent + bg * (long long)N * K;

  for (long long base = 0; base < nsel + nwin; base += CBATCH) {
    const int nb = (int)min((long long)CBATCH, nsel + nwin - base);
    __syncthreads();                                 // previous batch consumed
    for (int t = tid; t < nb; t += CT) {
      const long long idx = base + t;
      if (idx < nsel) {
        const uint32_t e = eg[p0 + idx / G];
        const int r = (int)(idx % G), i = (int)(e >> 8), s2 = (int)(e & 255u);
        const float* ps = pstat + (((bg * N + i) * (long long)K + s2) * G + r) * 4;
        di[t] = (i << 4) | r;
        dsx[t * 4 + 0] = ps[0];
        dsx[t * 4 + 1] = ps[1];
        dsx[t * 4 + 2] = ps[2];
        dsx[t * 4 + 3] = ps[3];                      // d s_hat (for dk', db')
      } else {
        const long long widx = idx - nsel;
        const int i = j0 + (int)(widx / G), r = (int)(widx % G);
        const float* ws = wstat + ((hb + r) * N + i) * 4;
        di[t] = (int)(0x80000000u | ((uint32_t)i << 4) | (uint32_t)r);
        dwl[t] = (int)(window_start(i, W, S) - j0);
        dsx[t * 4 + 0] = ws[0];
        dsx[t * 4 + 1] = ws[1];
        dsx[t * 4 + 2] = ws[2];
        dsx[t * 4 + 3] = ws[3];                      // d log Z_swa
      }
    }
    __syncthreads();
    if constexpr (SUMONLY) {
      static_assert(sizeof(T) == 2, "the summary-only variant reads bf16 pairs");
      // sixteen rows in flight; with the group size GT fixed at compile time
      // (u0 and ub are multiples of it) contribution ub + x has head x % GT
      const int u0 = 64 * wvs, u1 = min(nb, u0 + 64);
      if constexpr (GT > 0) {
        // the wavefront's 64 rows as 16-byte pieces, eight rows per lane in flight
        for (int jh = 0; jh < PR; jh += 8) {
          uint4 rv[8];
#pragma unroll
          for (int j2 = 0; j2 < 8; ++j2) {
            const int u = u0 + RPI * (jh + j2) + rq;
            rv[j2] = make_uint4(0u, 0u, 0u, 0u);
            if (u < u1) {
              const int dd = di[u];
              rv[j2] = *reinterpret_cast<const uint4*>(qr + ((hb + (dd & 15)) * N + (dd >> 4)) * (long long)d + 8 * pc);
            }
          }
#pragma unroll
          for (int j2 = 0; j2 < 8; ++j2) {
            const int u = u0 + RPI * (jh + j2) + rq;
            if (u < u1) {
              const double xt = (double)dsx[u * 4 + 3];
              const double tx = (double)tau * xt;
              const uint32_t w4[4] = {rv[j2].x, rv[j2].y, rv[j2].z, rv[j2].w};
              const int h2 = j2 % NHW;               // jh is a multiple of NHW
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                sw[h2][2 * t] = fma(tx, (double)__uint_as_float(w4[t] << 16), sw[h2][2 * t]);
                sw[h2][2 * t + 1] = fma(tx, (double)__uint_as_float(w4[t] & 0xffff0000u), sw[h2][2 * t + 1]);
              }
              if (pc == 0) sbw[h2] += xt;
            }
          }
        }
        continue;
      }
      for (int ub = u0; ub < u1; ub += 16) {
        uint32_t rv[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int u = ub + x;
          rv[x] = 0u;
          if (u < u1 && el < d) {
            const int dd = di[u];
            rv[x] = *reinterpret_cast<const uint32_t*>(
                qr + ((hb + (dd & 15)) * N + (dd >> 4)) * (long long)d + el);
          }
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int u = ub + x;
          if (u < u1) {
            const double xt = (double)dsx[u * 4 + 3];
            const double tx = (double)tau * xt;
            const double h0 = (double)__uint_as_float(rv[x] << 16);
            const double h1 = (double)__uint_as_float(rv[x] & 0xffff0000u);
            if constexpr (GT > 0) {
              const int rr = x % GT;
              sa[rr][0] = fma(tx, h0, sa[rr][0]);
              sa[rr][1] = fma(tx, h1, sa[rr][1]);
              sb[rr] += xt;
            } else {
              const int r = di[u] & 15;
#pragma unroll
              for (int rr = 0; rr < 8; ++rr) {
                if (rr == r) {
                  sa[rr][0] = fma(tx, h0, sa[rr][0]);
                  sa[rr][1] = fma(tx, h1, sa[rr][1]);
                  sb[rr] += xt;
                }
              }
            }
          }
        }
      }
      continue;
    }
    // the rows of sub-batch sb (NB contributions) are loaded into registers
    // while sub-batch sb - 1 is applied from LDS, then stored to the other
    // buffer.  Thread tid takes 16-byte piece tid % prow of contribution
    // tid / prow from each of the three rows (NB * prow <= CT: d <= 128).
    constexpr int VE = 16 / (int)sizeof(T);          // elements per 16-byte piece
    const int prow = d / VE;                         // pieces per row
    const int sul = tid / prow, spart = tid - sul * prow;
    const bool stager = sul < NB;
    uint4 pv0 = make_uint4(0u, 0u, 0u, 0u), pv1 = pv0, pv2 = pv0;
    auto stage_load = [&](int sb) __attribute__((always_inline)) {
      const int u = sb * NB + sul;
      if (stager && u < nb) {
        const int dd = di[u];
        const int i = (dd >> 4) & 0x7ffffff, r = dd & 15;
        const long long o = ((hb + r) * N + i) * (long long)d + spart * VE;
        pv0 = *reinterpret_cast<const uint4*>(q + o);
        pv1 = *reinterpret_cast<const uint4*>(dout + o);
        pv2 = *reinterpret_cast<const uint4*>(qr + o);
      }
    };
    auto stage_store = [&](int buf) __attribute__((always_inline)) {
      if (stager) {
        T* base = stg + ((size_t)buf * 3 * NB + sul) * d + spart * VE;
        *reinterpret_cast<uint4*>(base) = pv0;
        *reinterpret_cast<uint4*>(base + (size_t)NB * d) = pv1;
        *reinterpret_cast<uint4*>(base + (size_t)2 * NB * d) = pv2;
      }
    };
    auto apply = [&](int u, int buf) __attribute__((always_inline)) {
      const int ul = u % NB;
      float qv[CE], dv2[CE];
      load_slice16<T>(stg + (((size_t)buf * 3 + 0) * NB + ul) * d + e0, DQ, qv);
      load_slice16<T>(stg + (((size_t)buf * 3 + 1) * NB + ul) * d + e0, DQ, dv2);
      const int dd = di[u];
      const bool window = dd < 0;
      const int i = (dd >> 4) & 0x7ffffff, r = dd & 15;
      float a = 0.0f, u2 = 0.0f;
#pragma unroll
      for (int x = 0; x < CE; ++x) {
        a = fmaf(qv[x], kj[x], a);
        u2 = fmaf(dv2[x], vj[x], u2);
      }
      // the 8 lanes of a token hold its 8 slices (DPP, within one row)
      a += fastp::xshfl_f(a, 1);
      u2 += fastp::xshfl_f(u2, 1);
      a += fastp::xshfl_f(a, 2);
      u2 += fastp::xshfl_f(u2, 2);
      a += fastp::xshfl_f(a, 4);
      u2 += fastp::xshfl_f(u2, 4);
      const float alpha = dsx[u * 4], lse = dsx[u * 4 + 1], gq = dsx[u * 4 + 2], xt = dsx[u * 4 + 3];
      const int j = j0 + jt;
      bool ok = act;
      if (window) ok = ok && j <= i && jt >= dwl[u];
      const float pp = ok ? __expf(tau * a - lse) : 0.0f;
      const float ds = alpha * pp * (u2 - gq) + (window ? xt * pp : 0.0f);
      const float ap = alpha * pp;
#pragma unroll
      for (int x = 0; x < CE; ++x) {
        dkj[x] = fmaf(tau * ds, qv[x], dkj[x]);
        dvj[x] = fmaf(ap, dv2[x], dvj[x]);
      }
      // dk' += tau d s_hat q_hat, db' += d s_hat (see dka above)
      if (!window && (u & 3) == eq4 && ea < d) {
        const double hv = (double)Elt<T>::ld(stg + (((size_t)buf * 3 + 2) * NB + ul) * d + ea);
        const double txt = (double)tau * (double)xt;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (rr == r) {
            dka[rr] = fma(txt, hv, dka[rr]);
            dba[rr] += (double)xt;
          }
        }
      }
    };
    const int nsb = (nb + NB - 1) / NB;
    stage_load(0);
    stage_store(0);
    __syncthreads();
    for (int sb = 0; sb < nsb; ++sb) {
      if (sb + 1 < nsb) stage_load(sb + 1);
      const int ue = min(nb, (sb + 1) * NB);
      for (int u = sb * NB; u < ue; ++u) apply(u, sb & 1);
      // buffer (sb + 1) & 1 was last read in sub-batch sb - 1, before the
      // barrier that ended it
      if (sb + 1 < nsb) stage_store((sb + 1) & 1);
      __syncthreads();
    }
  }
  __syncthreads();
  if constexpr (SUMONLY && GT > 0) {
    // the wavefronts' sums in order; within a wavefront one row group (rq) at
    // a time, since the groups of one head share their dks elements
    for (int w = 0; w < CT / 64; ++w) {
      if (wvs == w) {
        for (int t = 0; t < RPI; ++t) {
          if (rq == t) {
#pragma unroll
            for (int h2 = 0; h2 < NHW; ++h2) {
              const int hd = (RPI * h2 + rq) % GT;
#pragma unroll
              for (int x = 0; x < 8; ++x) dks[hd * d + 8 * pc + x] += sw[h2][x];
              if (pc == 0) dbs[hd] += sbw[h2];
            }
          }
        }
      }
      __syncthreads();
    }
  } else if constexpr (SUMONLY) {
    for (int w = 0; w < CT / 64; ++w) {              // the wavefronts' sums, in order
      if (wvs == w) {
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (rr < G) {
            if (el < d) {
              dks[rr * d + el] += sa[rr][0];
              dks[rr * d + el + 1] += sa[rr][1];
            }
            if (el == 0) dbs[rr] += sb[rr];
          }
        }
      }
      __syncthreads();
    }
  } else {
    for (int p4 = 0; p4 < 4; ++p4) {                 // the quarters of dk', db', in order
      if (eq4 == p4 && ea < d) {
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (rr < G) {
            dks[rr * d + ea] += dka[rr];
            if (ea == 0) dbs[rr] += dba[rr];
          }
        }
      }
      __syncthreads();
    }
  }
  if (SUMONLY) load_kv();
  // summaries of the chunk (one per query head of the group)
  if (summ) {
    for (int r = 0; r < G; ++r) {
      const long long ho = ((hb + r) * nC + c) * (long long)d;
      if (mode == 1) {                       // landmark key: k' = q', b' = 0
        for (int e = tid; e < d; e += CT) dlm[ho + e] = (float)dks[r * d + e];
        continue;
      }
      if (mode == 3) {                       // mean pooling: k' = mean of the keys
#pragma unroll
        for (int x = 0; x < CE; ++x)
          if (x < DQ) dkj[x] = fmaf(1.0f / (float)S, (float)dks[r * d + e0 + x], dkj[x]);
        continue;
      }
      float lv[CE];
      load_slice16<T>(lm + ho + e0, DQ, lv);
      // the summary softmax and its backward in double (see dks above)
      double a = 0.0, dp = 0.0;
#pragma unroll
      for (int x = 0; x < CE; ++x) {
        a = fma((double)lv[x], (double)kj[x], a);
        dp = fma(x < DQ ? dks[r * d + e0 + x] : 0.0, (double)kj[x], dp);
      }
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      dp += __shfl_xor(dp, 4, 64);
      const double t = act ? (double)tau * a : -INFINITY;
      const double m = block_max_d((qd == 0) ? t : -INFINITY, redd);
      const double z = block_sum_d((qd == 0 && act) ? exp(t - m) : 0.0, redd);
      const double lpi = t - (m + log(z));
      const double pi = act ? exp(lpi) : 0.0;
      const double dpi = act ? dp + dbs[r] * (-lpi - 1.0) : 0.0;
      // dt = pi (dpi - sum pi dpi), centred on the dpi of a largest-weight
      // token (any reference gives the same value since sum pi = 1): the
      // differences stay small where pi is peaked, instead of cancelling
      const double rc = block_max_d((qd == 0 && act && t == m) ? dpi : -INFINITY, redd);
      const double spd = block_sum_d((qd == 0) ? pi * (dpi - rc) : 0.0, redd);
      const double dt = pi * ((dpi - rc) - spd);
      // dlm = tau sum_j dt_j k_j: column sums over the chunk's tokens, first
      // over the 8 tokens of a wavefront (lanes 8, 16 and 32 apart share an
      // element slice), then over the wavefronts in LDS
      {
        const int wv = tid >> 6, ln = tid & 63;
#pragma unroll
        for (int x = 0; x < CE; ++x) {
          double v = (act && x < DQ) ? dt * (double)kj[x] : 0.0;
          v += __shfl_xor(v, 8, 64);
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          if (ln < 8 && x < DQ) tmp[wv * d + e0 + x] = v;
        }
      }
      __syncthreads();
      for (int e = tid; e < d; e += CT) {
        double sum = 0.0;
        for (int u = 0; u < CT / 64; ++u) sum += tmp[u * d + e];
        dlm[ho + e] = (float)((double)tau * sum);
      }
#pragma unroll
      for (int x = 0; x < CE; ++x)
        if (x < DQ)
          dkj[x] += (float)((double)tau * dt * (double)lv[x] + pi * dks[r * d + e0 + x]);
      __syncthreads();
    }
  }
  if (SUMONLY) {                             // add the summaries' share to dk
    if (act && mode != 1) {
      float* dko = dk + (bg * (long long)N + j0 + jt) * d + e0;
#pragma unroll
      for (int x = 0; x < CE; ++x)
        if (x < DQ) dko[x] += dkj[x];
    }
    return;
  }
  if (act) {
    float* dko = dk + (bg * (long long)N + j0 + jt) * d + e0;
    float* dvo = dv + (bg * (long long)N + j0 + jt) * d + e0;
#pragma unroll
    for (int x = 0; x < CE; ++x) {
      if (x < DQ) {
        dko[x] = dkj[x];
        dvo[x] = dvj[x];
      }
    }
  }
}

}  // namespace

// workgroups per (sequence, KV group) of the list kernels: one per 4096
// queries (each wavefront then scatters at most 256), at most 64, one when
// the per-wavefront counters do not fit LDS
int hils_bwd_list_parts(const HilsShape& s) {
  if ((size_t)16 * s.nC * sizeof(uint32_t) > 128 * 1024 || s.nC <= 0) return 1;
  const int p = (s.N + 4095) / 4096;
  return p < 1 ? 1 : (p > 64 ? 64 : p);
}
size_t hils_bwd_list_count_bytes(const HilsShape& s) {
  const int p = hils_bwd_list_parts(s);
  return p > 1 ? (size_t)s.B * s.Hkv * 16 * p * s.nC * sizeof(uint32_t) : 0;
}

size_t hils_bwd_rows_lds(const HilsShape& s) {
  const int L = s.W + s.S - 1;
  const int Lp = (L + 3) & ~3;
  return sizeof(float) * ((size_t)4 * s.G * s.d + 2 * (size_t)s.G * Lp + 2 * (size_t)s.G * s.S +
                          (size_t)s.K * s.G * 4 + (size_t)s.G * 4 + 4);
}

hipError_t hils_launch_backward(const HilsShape& s, const void* q, const void* qr, const void* k,
                                const void* v, const void* lm, const void* dout, const int32_t* sel,
                                const void* ksum, const float* bsum, float* dq, float* dqr,
                                float* dk, float* dv, float* dlm, const HilsBwdBufs& wb,
                                hipStream_t st) {
  const float tau = (float)s.tau;
  // per-wavefront counters while they fit 128 KB of LDS; P workgroups per
  // (sequence, KV group) when the counts buffer is there
  const int lpar = (size_t)16 * s.nC * sizeof(uint32_t) <= 128 * 1024;
  const size_t lshm = sizeof(uint32_t) * (size_t)(lpar ? 16 : 1) * (size_t)(s.nC > 0 ? s.nC : 1);
  const int lP = hils_bwd_list_parts(s);
  if (lP > 1 && lpar && s.nC > 0 && wb.lcnt) {
    hils_allow_lds((const void*)k_bwd_lcount, lshm);
    hils_allow_lds((const void*)k_bwd_lscatter, lshm);
    HilsProfScope ps_("k_bwd_lists", st);
    hipLaunchKernelGGL(k_bwd_lcount, dim3((unsigned)(s.B * s.Hkv), (unsigned)lP), dim3(1024), lshm,
                       st, sel, wb.lcnt, s.N, s.K, s.nC, lP);
    hipLaunchKernelGGL(k_bwd_lscan, dim3((unsigned)(s.B * s.Hkv)), dim3(1024), 0, st, wb.lcnt,
                       wb.off, s.nC, 16 * lP);
    hipLaunchKernelGGL(k_bwd_lscatter, dim3((unsigned)(s.B * s.Hkv), (unsigned)lP), dim3(1024),
                       lshm, st, sel, wb.lcnt, wb.ent, s.N, s.K, s.nC, lP);
  } else {
    hils_allow_lds((const void*)k_bwd_lists, lshm);
    HilsProfScope ps_("k_bwd_lists", st);
    hipLaunchKernelGGL(k_bwd_lists, dim3((unsigned)(s.B * s.Hkv)), dim3(1024), lshm, st, sel,
                       wb.off, wb.ent, s.N, s.K, s.nC, lpar);
  }
  // the all-keys row kernel when every attended key's logit fits 64 KB of LDS
  const bool all_keys = bwd_rows2_lds(s) <= 65536;
  const size_t rshm = all_keys ? bwd_rows2_lds(s) : hils_bwd_rows_lds(s);
  const size_t ctail = sizeof(double) * ((size_t)s.G * s.d + s.G + 8) + sizeof(float) * 8 +
                       (size_t)CBATCH * (2 * sizeof(int) + 4 * sizeof(float));
  const size_t cshm = (s.dtype == 0 ? col_stage_bytes<bf16_t, false>(s.d, s.S)
                                    : col_stage_bytes<float, false>(s.d, s.S)) + ctail;
  const size_t sshm = col_stage_bytes<bf16_t, true>(s.d, s.S) + ctail;
  const int sep = dqr != nullptr;
  if (s.dtype == 0) {
    auto fr = all_keys ? k_bwd_rows2<bf16_t> : k_bwd_rows<bf16_t>;
    hils_allow_lds((const void*)fr, rshm);
    if (hils_bwd_mf_ok(s)) {
      // matrix-core passes, then the summaries' share of dk and dlm
      hipError_t e = hils_launch_backward_mf(s, q, qr, k, v, dout, sel, ksum, bsum, dq, dqr, dk, dv,
                                             wb, st);
      if (e != hipSuccess || s.nC <= 0) return e;
      // the group size as a template argument where it is a power of two
      auto fs = s.G == 1 ? k_bwd_cols<bf16_t, true, 1> : s.G == 2 ? k_bwd_cols<bf16_t, true, 2>
              : s.G == 4 ? k_bwd_cols<bf16_t, true, 4> : s.G == 8 ? k_bwd_cols<bf16_t, true, 8>
              : k_bwd_cols<bf16_t, true, 0>;
      hils_allow_lds((const void*)fs, sshm);
      HilsProfScope ps_("k_bwd_summ", st);
      hipLaunchKernelGGL(fs, dim3((unsigned)((long long)s.B * s.Hkv * s.nC)), dim3(CT),
                         sshm, st, (const bf16_t*)q, (const bf16_t*)qr, (const bf16_t*)k,
                         (const bf16_t*)v, (const bf16_t*)lm, (const bf16_t*)dout, wb.off, wb.ent,
                         wb.pstat, wb.wstat, dk, dv, dlm, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K,
                         s.nC, s.nC, tau, s.mode);
      return hipGetLastError();
    }
    { HilsProfScope ps_("k_bwd_rows", st);
      hipLaunchKernelGGL(fr, dim3((unsigned)((long long)s.B * s.Hkv * s.N)), dim3(BT), rshm, st,
                         (const bf16_t*)q, (const bf16_t*)qr, (const bf16_t*)k, (const bf16_t*)v,
                         (const bf16_t*)ksum, bsum, (const bf16_t*)dout, sel, dq, dqr, wb.pstat,
                         wb.wstat, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, s.nC, tau, sep); }
    hils_allow_lds((const void*)k_bwd_cols<bf16_t, false>, cshm);
    { HilsProfScope ps_("k_bwd_cols", st);
      hipLaunchKernelGGL((k_bwd_cols<bf16_t, false>), dim3((unsigned)((long long)s.B * s.Hkv * s.nCc)), dim3(CT), cshm, st,
                         (const bf16_t*)q, (const bf16_t*)qr, (const bf16_t*)k, (const bf16_t*)v,
                         (const bf16_t*)lm, (const bf16_t*)dout, wb.off, wb.ent, wb.pstat, wb.wstat,
                         dk, dv, dlm, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, s.nC, s.nCc, tau,
                         s.mode); }
  } else {
    auto fr = all_keys ? k_bwd_rows2<float> : k_bwd_rows<float>;
    hils_allow_lds((const void*)fr, rshm);
    hils_allow_lds((const void*)k_bwd_cols<float, false>, cshm);
    { HilsProfScope ps_("k_bwd_rows", st);
      hipLaunchKernelGGL(fr, dim3((unsigned)((long long)s.B * s.Hkv * s.N)), dim3(BT), rshm, st,
                         (const float*)q, (const float*)qr, (const float*)k, (const float*)v,
                         (const float*)ksum, bsum, (const float*)dout, sel, dq, dqr, wb.pstat,
                         wb.wstat, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, s.nC, tau, sep); }
    { HilsProfScope ps_("k_bwd_cols", st);
      hipLaunchKernelGGL((k_bwd_cols<float, false>), dim3((unsigned)((long long)s.B * s.Hkv * s.nCc)), dim3(CT), cshm, st,
                         (const float*)q, (const float*)qr, (const float*)k, (const float*)v,
                         (const float*)lm, (const float*)dout, wb.off, wb.ent, wb.pstat, wb.wstat,
                         dk, dv, dlm, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, s.nC, s.nCc, tau,
                         s.mode); }
  }
  return hipGetLastError();
}
