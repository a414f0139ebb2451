// HiLS decode: the prefill definition evaluated at the M newest positions
// i = T_b - M + m (M = 1: single-step decode; M > 1: a block of draft or
// verification tokens, each attending causally) ("Hierarchical Sparse
// Attention Done Right", sections 3 and 4.1; serving setup of section 7.1),
// split for bandwidth:
//   1. k_dec_score   — surrogate scores s_hat = scale*q_hat.k'_c + b'_c of every
//                      candidate chunk (a streaming read of the summary cache,
//                      the dominant HBM traffic, shared by up to 4 queries of a
//                      sequence);
//   2. k_dec_select  — per KV group: per-head log-sum-exp, max over heads, exact
//                      top-K by 32-bit radix select, ties to the lower chunk id;
//   3. k_dec_attn    — split-K attention: one workgroup per selected chunk or
//                      S-token window tile, partial (max, sum, unnormalised o);
//   4. k_dec_combine — window partials merged in the log domain, then the
//                      chunk-level softmax over {s_hat_c} U {log Z_swa}.
#include <type_traits>

#include "fast_common.h"
#include "hils_internal.h"

namespace {

// position of query m of a block of M new tokens of a sequence whose length is
// seqlen (clamped into the cache; a position below 0 is evaluated at 0)
__device__ __forceinline__ long long dec_pos(int32_t seqlen, int cap, int M, int m) {
  const long long i = clamp_len(seqlen, cap) - M + m;
  return i < 0 ? 0 : i;
}

// streaming 16-byte load (non-temporal): the summary cache is read once per
// step and should not evict the K/V tiles and scores the later kernels reuse
typedef unsigned int ntu4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt_u4(const void* p) {
  const ntu4_t w = __builtin_nontemporal_load(reinterpret_cast<const ntu4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;   // 16 bytes
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = __uint_as_float(w[t] << 16);
      o[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
    }
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
};

constexpr int SC_CPB = HILS_DEC_SCORE_ROWS;   // chunks per scoring workgroup: 16 groups x 16 rows

// Scores of 256 consecutive chunk rows of one (sequence, query head): a
// 16-lane group owns 16 consecutive rows and reads each row with 16-byte loads
// (all 16 rows in flight), the 16 row sums are reduce-scattered across the
// group so lane u ends with row u, and the workgroup also emits the
// (max, sum exp) partial of its scores for the per-head log-sum-exp.
// Requires d % Vec::N == 0 (checked on the host).
// Paged summary cache (PAGED): row (b, h, c) lives at physical page
// table[b * maxp + c] ([page][Hq][d] and [page][Hq]); page ids are clamped into
// [0, npages) so any table content stays in bounds.
struct PageMap {
  const int32_t* table;
  int maxp, npages;
  __device__ __forceinline__ long long page(int b, long long c) const {
    const int p = table[(long long)b * maxp + c];
    return (long long)min(max(p, 0), npages - 1);
  }
};

template <typename T, bool PAGED, int MT>
__global__ void __launch_bounds__(256)
k_dec_score(const T* __restrict__ qr, const T* __restrict__ ksum, const float* __restrict__ bsum,
            const int32_t* __restrict__ seqlen, float* __restrict__ scores, float* __restrict__ lsep,
            int Hq, int nC, int nmax, int nsb, int N, int d, int S, int W, float tau, int M,
            PageMap pm) {
  constexpr int V = Vec<T>::N;
  constexpr int MAXT = 256 / (16 * V) > 0 ? 256 / (16 * V) : 1;
  constexpr int R = 16;
  __shared__ float red_m[4][MT], red_s[4][MT];
  // grid x: 256-row block (fastest, so neighbouring workgroups stream adjacent
  // rows of one head), grid y: (sequence, head)
  const long long bh = blockIdx.y;
  const int b = (int)(bh / Hq);
  const int c0 = blockIdx.x * SC_CPB;
  // queries m0 .. m0 + mc - 1 of the sequence share every summary row read
  const int m0 = blockIdx.z * MT, mc = min(MT, M - m0);
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15, lane = tid & 63, wv = tid >> 6;
  auto lpart = [&](int mm) { return lsep + ((bh * M + m0 + mm) * nsb + blockIdx.x) * 2; };
  // Contiguous cache: the summary rows are read before the sequence length is
  // known (rows are clamped to the batch's longest candidate range, which the
  // cache always holds), so the loads overlap the length lookup; rows past
  // each query's candidates are discarded below.  Paged cache: the page
  // table is only defined for the sequence's own chunks, so the length comes
  // first.  The last query of the group has the most candidates.
  const int r0 = c0 + grp * R;
  const int h = (int)(bh - (long long)b * Hq);
  int cmax = nmax - 1;
  if (PAGED) {
    const int nb = n_cand(dec_pos(seqlen[b], N, M, m0 + mc - 1), W, S);
    if (c0 >= nb) {
      if (tid < mc) { lpart(tid)[0] = -INFINITY; lpart(tid)[1] = 0.0f; }
      return;
    }
    cmax = nb - 1;
  }
  auto krow = [&](int c) -> long long {
    return PAGED ? (pm.page(b, c) * Hq + h) * (long long)d : (bh * nC + c) * (long long)d;
  };
  const int cb = min(r0 + l16, cmax);
  const float bv = PAGED ? bsum[pm.page(b, cb) * Hq + h] : bsum[bh * nC + cb];
  float acc[MT][R];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int u = 0; u < R; ++u) acc[mm][u] = 0.0f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const int e = (t * 16 + l16) * V;
    if (e < d) {
      float qv[MT][V];
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)      // past the group: a valid row, result unused
        Vec<T>::load(qr + (bh * M + m0 + min(mm, mc - 1)) * d + e, qv[mm]);
      uint4 raw[R];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int c = min(r0 + u, cmax);
        raw[u] = ld_nt_u4(ksum + krow(c) + e);
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        float kv[V];
        Vec<T>::load(reinterpret_cast<const T*>(&raw[u]), kv);
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
#pragma unroll
          for (int x = 0; x < V; ++x) acc[mm][u] = fmaf(qv[mm][x], kv[x], acc[mm][u]);
      }
    }
  }
  const int nhi = n_cand(dec_pos(seqlen[b], N, M, m0 + mc - 1), W, S);
  if (c0 >= nhi) {
    if (tid < mc) { lpart(tid)[0] = -INFINITY; lpart(tid)[1] = 0.0f; }
    return;
  }
  const int c = r0 + l16;
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    if (mm < mc) {
      // reduce-scatter over the 16 lanes: after the step with mask k a lane
      // keeps the half of its rows whose index bit k matches its lane bit k
#pragma unroll
      for (int k2 = 8; k2 >= 1; k2 >>= 1) {
        const bool hi = (l16 & k2) != 0;
#pragma unroll
        for (int u = 0; u < k2; ++u) {
          const float keep = hi ? acc[mm][u + k2] : acc[mm][u];
          const float send = hi ? acc[mm][u] : acc[mm][u + k2];
          acc[mm][u] = keep + __shfl_xor(send, k2, 64);
        }
      }
      const int n = n_cand(dec_pos(seqlen[b], N, M, m0 + mm), W, S);
      const bool ok = c < n;
      const float x = ok ? fmaf(tau, acc[mm][0], bv) : -INFINITY;
      if (ok) scores[(bh * M + m0 + mm) * nmax + c] = x;
      const float m = wave_max_f(x);
      const float ex = ok ? __expf(x - m) : 0.0f;
      const float sw = wave_sum_f(ex);
      if (lane == 0) { red_m[wv][mm] = m; red_s[wv][mm] = sw; }
    }
  }
  __syncthreads();
  if (tid < mc) {
    const int mm = tid;
    float Mx = fmaxf(fmaxf(red_m[0][mm], red_m[1][mm]), fmaxf(red_m[2][mm], red_m[3][mm]));
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      L += (red_s[w][mm] > 0.0f) ? red_s[w][mm] * __expf(red_m[w][mm] - Mx) : 0.0f;
    lpart(mm)[0] = Mx;
    lpart(mm)[1] = L;
  }
}

constexpr int SEL_NT = 1024;
constexpr int SEL_NW = SEL_NT / 64;

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) { m = M; s = 0.0f; return; }
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

constexpr int SEL_LDS_KEYS = 24576;   // keys kept in LDS (96 KB) when the candidate set fits

__global__ void __launch_bounds__(SEL_NT)
k_dec_select(const float* __restrict__ scores, const float* __restrict__ lsep,
             const int32_t* __restrict__ seqlen, uint32_t* __restrict__ keys,
             int32_t* __restrict__ sel, float* __restrict__ slog, int Hq, int Hkv, int G, int nmax,
             int nsb, int N, int S, int W, int K, int M) {
  extern __shared__ uint32_t sel_keys_lds[];
  __shared__ uint32_t hist[256];
  __shared__ float Lh[8];
  __shared__ int wsum[SEL_NW];
  __shared__ int sh_digit, sh_need;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bgm = blockIdx.x;                 // (sequence, KV group, query)
  const int m = bgm % M, bg = bgm / M;
  const int b = bg / Hkv, g = bg % Hkv;
  const int n = n_cand(dec_pos(seqlen[b], N, M, m), W, S);
  const int kk = min(K, n);
  // per-head rows of this query: ((b * Hq + g * G + r) * M + m)
  auto hrow = [&](int r) { return ((long long)b * Hq + (long long)g * G + r) * M + m; };
  int32_t* so = sel + (long long)bgm * K;
  for (int t = tid; t < K; t += SEL_NT) if (t >= kk) so[t] = -1;
  for (int t = tid; t < G * K; t += SEL_NT) {
    const int r = t / K, kx = t % K;
    if (kx >= kk) slog[hrow(r) * K + kx] = 0.0f;
  }
  if (n == 0) return;
  uint32_t* ky = (n <= SEL_LDS_KEYS) ? sel_keys_lds : keys + (long long)bgm * nmax;

  if (G > 1) {
    // per-head log-sum-exp from the scoring workgroups' (max, sum exp) partials
    for (int r = wv; r < G; r += SEL_NW) {
      const float* lp = lsep + hrow(r) * nsb * 2;
      float m = -INFINITY, s = 0.0f;
      for (int t = lane; t < nsb; t += 64) lse_merge(m, s, lp[2 * t], lp[2 * t + 1]);
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float m2 = __shfl_xor(m, msk, 64), s2 = __shfl_xor(s, msk, 64);
        lse_merge(m, s, m2, s2);
      }
      if (lane == 0) Lh[r] = m + __logf(s);
    }
    __syncthreads();
  }
  constexpr int KU = 4;
  for (int base = 0; base < n; base += KU * SEL_NT) {
    float gs[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) gs[u] = -INFINITY;
    for (int r = 0; r < G; ++r) {
      const float* sr = scores + hrow(r) * nmax;
      const float lr = (G == 1) ? 0.0f : Lh[r];
      float x[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int c = base + u * SEL_NT + tid;
        x[u] = (c < n) ? sr[c] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < KU; ++u) gs[u] = fmaxf(gs[u], x[u] - lr);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int c = base + u * SEL_NT + tid;
      if (c < n) ky[c] = f32_order_key(gs[u]);
    }
  }
  if (tid == 0) sh_need = kk;
  __syncthreads();

  // MSD radix select of the kk-th largest 32-bit key
  uint32_t prefix = 0, pmask = 0;
  for (int p = 3; p >= 0; --p) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < n; c += SEL_NT) {
      const uint32_t key = ky[c];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> (8 * p)) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {            // one wave: suffix sums over 256 bins, 4 per lane
      uint32_t h4[4], s4 = 0;
#pragma unroll
      for (int u = 3; u >= 0; --u) { s4 += hist[tid * 4 + u]; h4[u] = s4; }
      // totals of all higher lanes: inclusive suffix scan over the wave
      uint32_t suf = s4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o, 64);
        if (tid + o < 64) suf += y;
      }
      const uint32_t above = suf - s4;
      const int need = sh_need;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t sufu = h4[u] + above;                      // keys with digit >= 4*tid+u
        const uint32_t sufn = (u < 3) ? h4[u + 1] + above : above; // digit > 4*tid+u
        if (sufu >= (uint32_t)need && sufn < (uint32_t)need) {
          sh_digit = tid * 4 + u;
          sh_need = need - (int)sufn;
        }
      }
    }
    __syncthreads();
    const uint32_t dg = (uint32_t)sh_digit;
    prefix |= dg << (8 * p);
    pmask |= 0xffu << (8 * p);
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int need_eq = sh_need;   // how many keys equal to thr to take (lowest chunk ids)

  // compaction in ascending chunk order: thread t owns chunks [8t, 8t + 8) of
  // each round of 8 * SEL_NT; one block scan of its (greater, equal) counts
  // gives where its selected chunks go.  Keys equal to thr are taken lowest
  // chunk id first, need_eq of them.
  constexpr int CPT = 8;
  int taken_all = 0, eq_all = 0;
  for (int base = 0; base < n; base += CPT * SEL_NT) {
    const int c0 = base + CPT * tid;
    uint32_t kv[CPT];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      kv[u] = (c0 + u < n) ? ky[c0 + u] : 0u;
      const bool in = c0 + u < n;
      ngt += (in && kv[u] > thr) ? 1 : 0;
      neq += (in && kv[u] == thr) ? 1 : 0;
    }
    // inclusive scan of the packed counts (greater in the low 16 bits)
    const uint32_t mine = (uint32_t)ngt | ((uint32_t)neq << 16);
    uint32_t inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wv] = (int)inc;
    __syncthreads();
    uint32_t before = inc - mine, total = 0;
    for (int u = 0; u < SEL_NW; ++u) {
      const uint32_t t = (uint32_t)wsum[u];
      if (u < wv) before += t;
      total += t;
    }
    __syncthreads();                       // wsum is rewritten next round
    const int gt_before = (int)(before & 0xffffu), eq_before = eq_all + (int)(before >> 16);
    // taken before this thread: earlier rounds, then this round's greater keys
    // and equal keys before it
    int pos = taken_all + gt_before + min(eq_before, need_eq) - min(eq_all, need_eq);
    int eqi = eq_before;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = c0 + u;
      if (c < n) {
        bool take = kv[u] > thr;
        if (kv[u] == thr) take = eqi++ < need_eq;
        if (take) {
          so[pos] = c;
          for (int r = 0; r < G; ++r) slog[hrow(r) * K + pos] = scores[hrow(r) * nmax + c];
          ++pos;
        }
      }
    }
    const int gt_tot = (int)(total & 0xffffu), eq_tot = (int)(total >> 16);
    taken_all += gt_tot + min(eq_all + eq_tot, need_eq) - min(eq_all, need_eq);
    eq_all += eq_tot;
  }
}

constexpr int AT_NT = 256;

// One workgroup per (sequence, KV group, split): a split is one selected chunk
// or one S-token window tile (S <= 64, G <= 8, checked on the host).  The K and
// V rows of the split are staged in LDS with 16-byte loads; thread (head, key)
// forms a logit, wave h takes head h's softmax over the split (lane = key),
// thread (head, element) forms the unnormalised output from the LDS V tile.
template <typename T, bool PAGED>
__global__ void __launch_bounds__(AT_NT)
k_dec_attn(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
           const int32_t* __restrict__ seqlen, const int32_t* __restrict__ sel, float* __restrict__ part,
           int Hq, int Hkv, int G, int N, int d, int S, int W, int K, int NS, float tau, int M,
           PageMap pm) {
  constexpr int V = Vec<T>::N;
  extern __shared__ __align__(16) unsigned char sm_raw[];
  const int kstr = d + V;                                     // padded row (elements), 16-byte multiple
  T* ks = reinterpret_cast<T*>(sm_raw);                       // [S][kstr]
  T* vs = ks + S * kstr;                                      // [S][kstr]
  float* qs = reinterpret_cast<float*>(vs + S * kstr);        // [G][d]
  const int SP = (S + 3) & ~3;                                // padded softmax row
  float* ps = qs + G * d;                                     // [G][SP], zero past the split
  __shared__ float hm[8], hl[8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bgm = blockIdx.x, s = blockIdx.y;      // (sequence, KV group, query), split
  const int m = bgm % M, bg = bgm / M;
  const int b = bg / Hkv, g = bg % Hkv;
  auto hrow = [&](int r) { return ((long long)b * Hq + (long long)g * G + r) * M + m; };
  // loads that do not need the sequence length go first: the query rows and,
  // for a chunk split, its chunk id (slots past the selection hold -1)
  for (int t = tid; t < G * d; t += AT_NT) {
    const int r = t / d;
    qs[t] = Elt<T>::ld(q + hrow(r) * d + (t - r * d));
  }
  const int csel = (s < K) ? sel[(long long)bgm * K + s] : -1;
  const long long i = dec_pos(seqlen[b], N, M, m);
  long long j0 = 0;
  int jn = 0;
  if (s < K) {
    if (csel >= 0) { j0 = (long long)csel * S; jn = S; }
  } else {
    j0 = window_start(i, W, S) + (long long)(s - K) * S;
    if (j0 <= i) jn = (int)min((long long)S, i - j0 + 1);
  }
  if (jn == 0) {               // empty split: weight 0 in the combine, zero partial
    for (int t = tid; t < G * (d + 2); t += AT_NT) {
      const int r = t / (d + 2), e = t - r * (d + 2);
      part[(hrow(r) * NS + s) * (long long)(d + 2) + e] = (e == 0) ? -INFINITY : 0.0f;
    }
    return;
  }
  // every split is one chunk-aligned S-token tile: one page of a paged cache
  const long long kvoff = PAGED ? (pm.page(b, j0 / S) * Hkv + g) * (long long)S * d
                                : ((b * (long long)Hkv + g) * N + j0) * d;
  const T* kg = k + kvoff;
  const T* vg = v + kvoff;
  const int vpr = d / V;                                      // 16-byte vectors per row
  const int nvec = jn * vpr;
  for (int base = 0; base < nvec; base += 4 * AT_NT) {        // 8 loads in flight per thread
    uint4 kx[4], vx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(base + u * AT_NT + tid, nvec - 1);
      const int j = t / vpr, e = (t - j * vpr) * V;
      kx[u] = *reinterpret_cast<const uint4*>(kg + (long long)j * d + e);
      vx[u] = *reinterpret_cast<const uint4*>(vg + (long long)j * d + e);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = base + u * AT_NT + tid;
      if (t < nvec) {
        const int j = t / vpr, e = (t - j * vpr) * V;
        *reinterpret_cast<uint4*>(ks + j * kstr + e) = kx[u];
        *reinterpret_cast<uint4*>(vs + j * kstr + e) = vx[u];
      }
    }
  }
  __syncthreads();
  for (int t = tid; t < G * SP; t += AT_NT) {
    const int r = t / SP, j = t - r * SP;
    float x = -INFINITY;
    if (j < jn) {
      const float* qq = qs + r * d;
      const T* kr = ks + j * kstr;
      float acc = 0.0f;
      for (int e = 0; e < d; e += V) {
        float kv[V];
        Vec<T>::load(kr + e, kv);
#pragma unroll
        for (int u = 0; u < V; u += 4) {
          const float4 qv = *reinterpret_cast<const float4*>(qq + e + u);
          acc = fmaf(qv.x, kv[u], acc);
          acc = fmaf(qv.y, kv[u + 1], acc);
          acc = fmaf(qv.z, kv[u + 2], acc);
          acc = fmaf(qv.w, kv[u + 3], acc);
        }
      }
      x = tau * acc;
    }
    ps[t] = x;
  }
  __syncthreads();
  for (int r = wv; r < G; r += AT_NT / 64) {
    const float x = (lane < SP) ? ps[r * SP + lane] : -INFINITY;
    const float m = wave_max_f(x);
    const float p = (lane < jn) ? __expf(x - m) : 0.0f;
    const float l = wave_sum_f(p);
    if (lane < SP) ps[r * SP + lane] = p;
    if (lane == 0) { hm[r] = m; hl[r] = l; }
  }
  __syncthreads();
  const int dh = d / 2;                                       // element pairs per row
  for (int t = tid; t < G * dh; t += AT_NT) {
    const int r = t / dh, e = 2 * (t - r * dh);
    const float* pr = ps + r * SP;
    float a0 = 0.0f, a1 = 0.0f;
    for (int j = 0; j < jn; j += 4) {                         // ps is zero past jn
      const float4 p4 = *reinterpret_cast<const float4*>(pr + j);
      const float pj[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j + u < jn) {
          a0 = fmaf(pj[u], Elt<T>::ld(vs + (j + u) * kstr + e), a0);
          a1 = fmaf(pj[u], Elt<T>::ld(vs + (j + u) * kstr + e + 1), a1);
        }
      }
    }
    float* pp = part + (hrow(r) * NS + s) * (long long)(d + 2);
    pp[2 + e] = a0;
    pp[3 + e] = a1;
    if (e == 0) { pp[0] = hm[r]; pp[1] = hl[r]; }
  }
}

// Specialised split attention for bf16, d = 128, S = 64, G <= 4 (same
// partials as k_dec_attn).  Every K and V load of the split is issued at the
// start, straight into registers:
//   logits: wave w takes elements [32w, 32w + 32) of key row j = lane and
//           forms its partial dot with each head's query (broadcast LDS
//           reads); the four partials meet in LDS and wave h takes head h's
//           softmax over the keys;
//   output: wave w takes keys [16w, 16w + 16), lane = (8-element slice e8 =
//           lane % 16, 4 keys 16w + 4 (lane / 16) + u); the four key groups of
//           a wave are summed with row swaps, the four waves in LDS.
// Rows past the split's last token are read at that token (their weight is
// 0), so every load stays inside the split's written rows.
constexpr int DA_D = 128, DA_S = 64;

template <bool PAGED, int G>
__global__ void __launch_bounds__(AT_NT)
k_dec_attn_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const int32_t* __restrict__ seqlen,
                const int32_t* __restrict__ sel, float* __restrict__ part, int Hq, int Hkv, int N,
                int W, int K, int NS, float tau, int M, PageMap pm) {
  constexpr int D = DA_D, S = DA_S;
  __shared__ __align__(16) float qs[G][D];
  __shared__ __align__(16) float dp[4][G][S];     // partial dots by element quarter
  __shared__ __align__(16) float ps[G][S];        // softmax weights
  __shared__ __align__(16) float red[4][G][D];    // output partials by key quarter
  __shared__ float hm[G], hl[G];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bgm = blockIdx.x, s = blockIdx.y;
  const int m = bgm % M, bg = bgm / M;
  const int b = bg / Hkv, g = bg % Hkv;
  auto hrow = [&](int r) { return ((long long)b * Hq + (long long)g * G + r) * M + m; };
  for (int t = tid; t < G * D; t += AT_NT) {
    const int r = t / D;
    qs[r][t - r * D] = bf16_to_f32(q[hrow(r) * D + (t - r * D)]);
  }
  const int csel = (s < K) ? sel[(long long)bgm * K + s] : -1;
  const long long i = dec_pos(seqlen[b], N, M, m);
  long long j0 = 0;
  int jn = 0;
  if (s < K) {
    if (csel >= 0) { j0 = (long long)csel * S; jn = S; }
  } else {
    j0 = window_start(i, W, S) + (long long)(s - K) * S;
    if (j0 <= i) jn = (int)min((long long)S, i - j0 + 1);
  }
  if (jn == 0) {
    for (int t = tid; t < G * (D + 2); t += AT_NT) {
      const int r = t / (D + 2), e = t - r * (D + 2);
      part[(hrow(r) * NS + s) * (long long)(D + 2) + e] = (e == 0) ? -INFINITY : 0.0f;
    }
    return;
  }
  const long long kvoff = PAGED ? (pm.page(b, j0 / S) * Hkv + g) * (long long)S * D
                                : ((b * (long long)Hkv + g) * N + j0) * D;
  const bf16_t* kg = k + kvoff;
  const bf16_t* vg = v + kvoff;
  // logit loads: key row min(lane, jn - 1), elements [32 wv, 32 wv + 32)
  uint4 kx[4];
  {
    const bf16_t* kr = kg + (long long)min(lane, jn - 1) * D + 32 * wv;
#pragma unroll
    for (int u = 0; u < 4; ++u) kx[u] = *reinterpret_cast<const uint4*>(kr + 8 * u);
  }
  // output loads: keys 16 wv + 4 kq + u, elements [8 e8, 8 e8 + 8)
  const int e8 = lane & 15, kq = lane >> 4;
  const int jb = 16 * wv + 4 * kq;
  uint4 vx[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    vx[u] = *reinterpret_cast<const uint4*>(vg + (long long)min(jb + u, jn - 1) * D + 8 * e8);
  __syncthreads();                                // qs
  {
    float kf[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w4[4] = {kx[u].x, kx[u].y, kx[u].z, kx[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kf[8 * u + 2 * t] = __uint_as_float(w4[t] << 16);
        kf[8 * u + 2 * t + 1] = __uint_as_float(w4[t] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float* qq = &qs[r][32 * wv];
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; e += 8) {
        const float4 qa = *reinterpret_cast<const float4*>(qq + e);
        const float4 qb = *reinterpret_cast<const float4*>(qq + e + 4);
        a0 = fmaf(qa.x, kf[e], a0);
        a1 = fmaf(qa.y, kf[e + 1], a1);
        a0 = fmaf(qa.z, kf[e + 2], a0);
        a1 = fmaf(qa.w, kf[e + 3], a1);
        a0 = fmaf(qb.x, kf[e + 4], a0);
        a1 = fmaf(qb.y, kf[e + 5], a1);
        a0 = fmaf(qb.z, kf[e + 6], a0);
        a1 = fmaf(qb.w, kf[e + 7], a1);
      }
      dp[wv][r][lane] = a0 + a1;
    }
  }
  __syncthreads();                                // dp
  if (wv < G) {
    const int r = wv;
    const float dot = (dp[0][r][lane] + dp[1][r][lane]) + (dp[2][r][lane] + dp[3][r][lane]);
    const float x = (lane < jn) ? tau * dot : -INFINITY;
    const float mx = wave_max_f(x);
    const float p = (lane < jn) ? __expf(x - mx) : 0.0f;
    const float l = wave_sum_f(p);
    ps[r][lane] = p;
    if (lane == 0) { hm[r] = mx; hl[r] = l; }
  }
  __syncthreads();                                // ps, hm, hl
  {
    float vf[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w4[4] = {vx[u].x, vx[u].y, vx[u].z, vx[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        vf[u][2 * t] = __uint_as_float(w4[t] << 16);
        vf[u][2 * t + 1] = __uint_as_float(w4[t] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float4 p4 = *reinterpret_cast<const float4*>(&ps[r][jb]);
      const float pu[4] = {p4.x, p4.y, p4.z, p4.w};
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = pu[0] * vf[0][e];
        a = fmaf(pu[1], vf[1][e], a);
        a = fmaf(pu[2], vf[2][e], a);
        a = fmaf(pu[3], vf[3][e], a);
        // the wave's four key groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
        o[e] = fastp::sum_x32(fastp::sum_x16(a));
      }
      if (kq == 0) {
        *reinterpret_cast<float4*>(&red[wv][r][8 * e8]) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(&red[wv][r][8 * e8 + 4]) = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
  __syncthreads();                                // red
  for (int t = tid; t < G * D; t += AT_NT) {
    const int r = t / D, e = t - r * D;
    float* pp = part + (hrow(r) * NS + s) * (long long)(D + 2);
    pp[2 + e] = (red[0][r][e] + red[1][r][e]) + (red[2][r][e] + red[3][r][e]);
    if (e == 0) { pp[0] = hm[r]; pp[1] = hl[r]; }
  }
}

// Per (sequence, query head): merge the window tiles in the log domain, take
// the chunk-level softmax over {s_hat_c} U {log Z_swa}, and form the output as
// one weighted sum of the split partials.  Wave 0 computes the split weights.
template <typename T>
__global__ void __launch_bounds__(256)
k_dec_combine(const float* __restrict__ part, const float* __restrict__ slog,
              const int32_t* __restrict__ seqlen, T* __restrict__ out, int Hq, int G, int N, int d,
              int S, int W, int K, int NS, int nwin, int M) {
  extern __shared__ float wsplit[];          // [NS] weight of each split's unnormalised o
  const int bh = blockIdx.x, tid = threadIdx.x;   // ((b * Hq + h) * M + m)
  const int b = bh / (Hq * M), m = bh % M;
  const long long i = dec_pos(seqlen[b], N, M, m);
  const int n = n_cand(i, W, S);
  const int kk = min(K, n);
  const float* pb = part + (long long)bh * NS * (d + 2);
  const float* sl = slog + (long long)bh * K;
  if (tid < 64) {
    float M = -INFINITY;
    for (int t = tid; t < nwin; t += 64) {
      const float* pp = pb + (long long)(K + t) * (d + 2);
      if (pp[1] > 0.0f) M = fmaxf(M, pp[0]);
    }
    M = wave_max_f(M);
    float L = 0.0f;
    for (int t = tid; t < nwin; t += 64) {
      const float* pp = pb + (long long)(K + t) * (d + 2);
      if (pp[1] > 0.0f) L += pp[1] * __expf(pp[0] - M);
    }
    L = wave_sum_f(L);
    const float logz = M + __logf(L);
    float Mx = logz;
    for (int kx = tid; kx < kk; kx += 64) Mx = fmaxf(Mx, sl[kx]);
    Mx = wave_max_f(Mx);
    float Z = 0.0f;
    for (int kx = tid; kx < kk; kx += 64) Z += __expf(sl[kx] - Mx);
    Z = wave_sum_f(Z) + __expf(logz - Mx);
    const float aw = __expf(logz - Mx) / Z / L;
    for (int kx = tid; kx < K; kx += 64)
      wsplit[kx] = (kx < kk) ? __expf(sl[kx] - Mx) / Z / pb[(long long)kx * (d + 2) + 1] : 0.0f;
    for (int t = tid; t < nwin; t += 64) {
      const float* pp = pb + (long long)(K + t) * (d + 2);
      wsplit[K + t] = (pp[1] > 0.0f) ? aw * __expf(pp[0] - M) : 0.0f;
    }
  }
  __syncthreads();
  for (int e = tid; e < d; e += 256) {      // every split holds a finite partial (zero if empty)
    float acc = 0.0f;
#pragma unroll 8
    for (int t = 0; t < NS; ++t) acc = fmaf(wsplit[t], pb[(long long)t * (d + 2) + 2 + e], acc);
    Elt<T>::st(out + (long long)bh * d + e, acc);
  }
}

template <typename T, bool PAGED, int MT>
void launch_score(const HilsShape& s, const void* qr, const int32_t* seqlen, const void* ksum,
                  const float* bsum, float* scores, float* lsep, unsigned nsb, PageMap pm,
                  hipStream_t st) {
  const unsigned nz = (unsigned)((s.M + MT - 1) / MT);
  { HilsProfScope ps_("k_dec_score", st);
    hipLaunchKernelGGL((k_dec_score<T, PAGED, MT>), dim3(nsb, s.B * s.Hq, nz), dim3(256), 0, st,
                       (const T*)qr, (const T*)ksum, bsum, seqlen, scores, lsep, s.Hq, s.nC, s.nmax,
                       (int)nsb, s.N, s.d, s.S, s.W, (float)s.tau, s.M, pm); }
}

template <typename T, bool PAGED>
void launch_decode_t(const HilsShape& s, const void* q, const void* qr, const void* k, const void* v,
                     const int32_t* seqlen, const void* ksum, const float* bsum, void* out,
                     int32_t* sel, float* scores, uint32_t* keys, float* slog, float* part,
                     float* lsep, PageMap pm, hipStream_t st) {
  const int NS = s.K + s.nwin;
  const float tau = (float)s.tau;
  const unsigned nsb = (unsigned)((s.nmax + SC_CPB - 1) / SC_CPB);
  const size_t esz = sizeof(T);
  const size_t ashm = 2 * (size_t)s.S * (s.d + 16 / esz) * esz + (size_t)s.G * s.d * 4 +
                      (size_t)s.G * ((s.S + 3) & ~3) * 4;
  const size_t cshm = (size_t)NS * 4;
  if (nsb > 0) {
    if (s.M == 1) launch_score<T, PAGED, 1>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
    else if (s.M == 2) launch_score<T, PAGED, 2>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
    else launch_score<T, PAGED, 4>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
  }
  const size_t sshm = (size_t)4 * (size_t)min(s.nmax > 0 ? s.nmax : 1, SEL_LDS_KEYS);
  hipFuncSetAttribute((const void*)k_dec_select, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sshm);
  { HilsProfScope ps_("k_dec_select", st); hipLaunchKernelGGL(k_dec_select, dim3(s.B * s.Hkv * s.M), dim3(SEL_NT), sshm, st, scores, lsep, seqlen,
                     keys, sel, slog, s.Hq, s.Hkv, s.G, s.nmax > 0 ? s.nmax : 1, (int)nsb, s.N, s.S,
                     s.W, s.K, s.M); }
  const dim3 agrid(s.B * s.Hkv * s.M, NS);
  if (std::is_same<T, bf16_t>::value && s.d == DA_D && s.S == DA_S && (s.G == 1 || s.G == 2 || s.G == 4)) {
    const bf16_t* qb = (const bf16_t*)q;
    const bf16_t* kb = (const bf16_t*)k;
    const bf16_t* vb = (const bf16_t*)v;
    HilsProfScope ps_("k_dec_attn", st);
    if (s.G == 1)
      hipLaunchKernelGGL((k_dec_attn_bf16<PAGED, 1>), agrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen, sel,
                         part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, tau, s.M, pm);
    else if (s.G == 2)
      hipLaunchKernelGGL((k_dec_attn_bf16<PAGED, 2>), agrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen, sel,
                         part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, tau, s.M, pm);
    else
      hipLaunchKernelGGL((k_dec_attn_bf16<PAGED, 4>), agrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen, sel,
                         part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, tau, s.M, pm);
  } else {
    hipFuncSetAttribute((const void*)k_dec_attn<T, PAGED>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ashm);
    HilsProfScope ps_("k_dec_attn", st);
    hipLaunchKernelGGL((k_dec_attn<T, PAGED>), agrid, dim3(AT_NT), ashm, st,
                       (const T*)q, (const T*)k, (const T*)v, seqlen, sel, part,
                       s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, NS, tau, s.M, pm);
  }
  { HilsProfScope ps_("k_dec_combine", st); hipLaunchKernelGGL(k_dec_combine<T>, dim3(s.B * s.Hq * s.M), dim3(256), cshm, st, part, slog,
                     seqlen, (T*)out, s.Hq, s.G, s.N, s.d, s.S, s.W, s.K, NS, s.nwin, s.M); }
}

}  // namespace

hipError_t hils_launch_decode(const HilsShape& s, const void* q, const void* qr, const void* k,
                              const void* v, const int32_t* seqlen, const void* ksum,
                              const float* bsum, void* out, int32_t* sel, float* scores,
                              uint32_t* keys, float* slog, float* part, float* lsep,
                              const int32_t* page_table, int max_pages, int num_pages,
                              hipStream_t st) {
  const PageMap pm{page_table, max_pages, num_pages};
  const bool paged = page_table != nullptr;
  if (s.dtype == 0) {
    if (paged) launch_decode_t<bf16_t, true>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, slog, part, lsep, pm, st);
    else launch_decode_t<bf16_t, false>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, slog, part, lsep, pm, st);
  } else {
    if (paged) launch_decode_t<float, true>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, slog, part, lsep, pm, st);
    else launch_decode_t<float, false>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, slog, part, lsep, pm, st);
  }
  return hipGetLastError();
}
