// Single-step HiLS decode: the prefill definition evaluated at i = T_b - 1
// ("Hierarchical Sparse Attention Done Right", sections 3 and 4.1; serving
// setup of section 7.1), split for bandwidth:
//   1. k_dec_score   — surrogate scores s_hat = scale*q_hat.k'_c + b'_c of every
//                      candidate chunk (a streaming read of the summary cache,
//                      the dominant HBM traffic);
//   2. k_dec_select  — per KV group: per-head log-sum-exp, max over heads, exact
//                      top-K by 32-bit radix select, ties to the lower chunk id;
//   3. k_dec_attn    — split-K attention: one workgroup per selected chunk or
//                      S-token window tile, partial (max, sum, unnormalised o);
//   4. k_dec_combine — window partials merged in the log domain, then the
//                      chunk-level softmax over {s_hat_c} U {log Z_swa}.
#include "hils_device.h"
#include "hils_internal.h"

namespace {

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

constexpr int SC_CPB = 256;   // chunks per scoring workgroup

// one 16-lane group per chunk row; d % Vec::N == 0 (checked on the host)
template <typename T>
__global__ void __launch_bounds__(256)
k_dec_score(const T* __restrict__ qr, const T* __restrict__ ksum, const float* __restrict__ bsum,
            const int32_t* __restrict__ seqlen, float* __restrict__ scores, int Hq, int nC, int nmax,
            int N, int d, int S, int W, float tau) {
  constexpr int V = Vec<T>::N;
  constexpr int MAXT = 256 / (16 * V) > 0 ? 256 / (16 * V) : 1;
  const long long bh = blockIdx.x;
  const int b = (int)(bh / Hq);
  const int n = n_cand(clamp_len(seqlen[b], N) - 1, W, S);
  const int c0 = blockIdx.y * SC_CPB;
  if (c0 >= n) return;
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
  float qv[MAXT][V];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const int e = (t * 16 + l16) * V;
    if (e < d) Vec<T>::load(qr + bh * d + e, qv[t]);
    else {
#pragma unroll
      for (int u = 0; u < V; ++u) qv[t][u] = 0.0f;
    }
  }
  const int c1 = min(n, c0 + SC_CPB);
  for (int c = c0 + grp; c < c1; c += 16) {
    const T* kp = ksum + (bh * nC + c) * (long long)d;
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      const int e = (t * 16 + l16) * V;
      if (e < d) {
        float kv[V];
        Vec<T>::load(kp + e, kv);
#pragma unroll
        for (int u = 0; u < V; ++u) acc = fmaf(qv[t][u], kv[u], acc);
      }
    }
    acc += __shfl_xor(acc, 8, 64);
    acc += __shfl_xor(acc, 4, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 1, 64);
    if (l16 == 0) scores[bh * nmax + c] = fmaf(tau, acc, bsum[bh * nC + c]);
  }
}

constexpr int SEL_NT = 1024;
constexpr int SEL_NW = SEL_NT / 64;

__device__ __forceinline__ int sel_excl_scan(int flag, int* wsum, int& pos) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int inwave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(bal);
  __syncthreads();
  int before = 0, total = 0;
  for (int u = 0; u < SEL_NW; ++u) {
    if (u < w) before += wsum[u];
    total += wsum[u];
  }
  pos = before + inwave;
  __syncthreads();
  return total;
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) { m = M; s = 0.0f; return; }
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

__global__ void __launch_bounds__(SEL_NT)
k_dec_select(const float* __restrict__ scores, const int32_t* __restrict__ seqlen,
             uint32_t* __restrict__ keys, int32_t* __restrict__ sel, float* __restrict__ slog,
             int Hq, int Hkv, int G, int nmax, int N, int S, int W, int K) {
  __shared__ uint32_t hist[256];
  __shared__ float red_m[SEL_NW][8], red_s[SEL_NW][8];
  __shared__ float Lh[8];
  __shared__ int wsum[SEL_NW];
  __shared__ int sh_digit, sh_need;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int n = n_cand(clamp_len(seqlen[b], N) - 1, W, S);
  const int kk = min(K, n);
  const long long hbase = (long long)b * Hq + (long long)g * G;
  int32_t* so = sel + (long long)bg * K;
  for (int t = tid; t < K; t += SEL_NT) if (t >= kk) so[t] = -1;
  for (int t = tid; t < G * K; t += SEL_NT) {
    const int r = t / K, kx = t % K;
    if (kx >= kk) slog[(hbase + r) * K + kx] = 0.0f;
  }
  if (n == 0) return;
  uint32_t* ky = keys + (long long)bg * nmax;

  if (G > 1) {
    for (int r = 0; r < G; ++r) {
      const float* sr = scores + (hbase + r) * nmax;
      float m = -INFINITY, s = 0.0f;
      for (int c = tid; c < n; c += SEL_NT) {
        const float x = sr[c];
        if (x > m) { s = s * __expf(m - x) + 1.0f; m = x; } else { s += __expf(x - m); }
      }
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float m2 = __shfl_xor(m, msk, 64), s2 = __shfl_xor(s, msk, 64);
        lse_merge(m, s, m2, s2);
      }
      if (lane == 0) { red_m[wv][r] = m; red_s[wv][r] = s; }
    }
    __syncthreads();
    if (tid < G) {
      float m = red_m[0][tid], s = red_s[0][tid];
      for (int u = 1; u < SEL_NW; ++u) lse_merge(m, s, red_m[u][tid], red_s[u][tid]);
      Lh[tid] = m + __logf(s);
    }
    __syncthreads();
  }
  for (int c = tid; c < n; c += SEL_NT) {
    float gs;
    if (G == 1) {
      gs = scores[hbase * nmax + c];
    } else {
      gs = -INFINITY;
      for (int r = 0; r < G; ++r) gs = fmaxf(gs, scores[(hbase + r) * nmax + c] - Lh[r]);
    }
    ky[c] = f32_order_key(gs);
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
      // totals of all higher lanes (uniform loop: every lane takes part in every shuffle)
      uint32_t above = 0;
      for (int l2 = 0; l2 < 64; ++l2) {
        const uint32_t y = __shfl(s4, l2, 64);
        if (l2 > tid) above += y;
      }
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

  int running = 0, eq_seen = 0;
  for (int base = 0; base < n; base += SEL_NT) {
    const int c = base + tid;
    const uint32_t key = (c < n) ? ky[c] : 0u;
    const int eq = (c < n) && (key == thr);
    int eqpos;
    const int eqtot = sel_excl_scan(eq, wsum, eqpos);
    const int f = (c < n) && (key > thr || (eq && eq_seen + eqpos < need_eq));
    int pos;
    const int tot = sel_excl_scan(f, wsum, pos);
    if (f) {
      so[running + pos] = c;
      for (int r = 0; r < G; ++r) slog[(hbase + r) * K + running + pos] = scores[(hbase + r) * nmax + c];
    }
    running += tot;
    eq_seen += eqtot;
  }
}

constexpr int AT_NT = 256;

template <typename T>
__global__ void __launch_bounds__(AT_NT)
k_dec_attn(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
           const int32_t* __restrict__ seqlen, const int32_t* __restrict__ sel, float* __restrict__ part,
           int Hq, int Hkv, int G, int N, int d, int S, int W, int K, int NS, float tau) {
  extern __shared__ __align__(16) unsigned char sm_raw[];
  float* qs = reinterpret_cast<float*>(sm_raw);   // [G][d]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x, s = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const long long i = clamp_len(seqlen[b], N) - 1;
  const int n = n_cand(i, W, S);
  const int kk = min(K, n);
  const long long w0 = window_start(i, W, S);
  const long long hbase = (long long)b * Hq + (long long)g * G;
  long long j0 = 0;
  int jn = 0;
  if (s < K) {
    if (s < kk) { j0 = (long long)sel[(long long)bg * K + s] * S; jn = S; }
  } else {
    j0 = w0 + (long long)(s - K) * S;
    if (j0 <= i) jn = (int)min((long long)S, i - j0 + 1);
  }
  if (jn == 0) {
    for (int t = tid; t < G; t += AT_NT) {
      float* pp = part + ((hbase + t) * NS + s) * (long long)(d + 2);
      pp[0] = -INFINITY;
      pp[1] = 0.0f;
    }
    return;
  }
  for (int t = tid; t < G * d; t += AT_NT) qs[t] = Elt<T>::ld(q + (hbase + t / d) * d + t % d);
  __syncthreads();
  const T* kg = k + (b * (long long)Hkv + g) * N * d;
  const T* vg = v + (b * (long long)Hkv + g) * N * d;
  for (int r = wv; r < G; r += AT_NT / 64) {
    float x = -INFINITY;
    if (lane < jn) {
      const T* kr = kg + (j0 + lane) * d;
      const float* qq = qs + r * d;
      float acc = 0.0f;
      for (int e = 0; e < d; ++e) acc = fmaf(qq[e], Elt<T>::ld(kr + e), acc);
      x = tau * acc;
    }
    const float m = wave_max_f(x);
    const float p = (lane < jn) ? __expf(x - m) : 0.0f;
    const float l = wave_sum_f(p);
    float* pp = part + ((hbase + r) * NS + s) * (long long)(d + 2);
    for (int e0 = 0; e0 < d; e0 += 64) {      // uniform trip count across lanes
      const int e = e0 + lane;
      float acc = 0.0f;
      for (int j = 0; j < jn; ++j) {
        const float pj = __shfl(p, j, 64);   // every lane runs the same j loop
        if (e < d) acc = fmaf(pj, Elt<T>::ld(vg + (j0 + j) * d + e), acc);
      }
      if (e < d) pp[2 + e] = acc;
    }
    if (lane == 0) { pp[0] = m; pp[1] = l; }
  }
}

template <typename T>
__global__ void __launch_bounds__(64)
k_dec_combine(const float* __restrict__ part, const float* __restrict__ slog,
              const int32_t* __restrict__ seqlen, T* __restrict__ out, int Hq, int G, int N, int d,
              int S, int W, int K, int NS, int nwin) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int b = bh / Hq;
  const long long i = clamp_len(seqlen[b], N) - 1;
  const int n = n_cand(i, W, S);
  const int kk = min(K, n);
  const float* pb = part + (long long)bh * NS * (d + 2);
  // window: log-domain merge of the tile partials
  float M = -INFINITY;
  for (int t = 0; t < nwin; ++t) {
    const float* pp = pb + (long long)(K + t) * (d + 2);
    if (pp[1] > 0.0f) M = fmaxf(M, pp[0]);
  }
  float L = 0.0f;
  constexpr int MAXE = 4;   // d <= 256
  float ow[MAXE], acc[MAXE];
#pragma unroll
  for (int u = 0; u < MAXE; ++u) { ow[u] = 0.0f; acc[u] = 0.0f; }
  for (int t = 0; t < nwin; ++t) {
    const float* pp = pb + (long long)(K + t) * (d + 2);
    if (!(pp[1] > 0.0f)) continue;
    const float sc = __expf(pp[0] - M);
    L += pp[1] * sc;
#pragma unroll
    for (int u = 0; u < MAXE; ++u) {
      const int e = lane + 64 * u;
      if (e < d) ow[u] = fmaf(pp[2 + e], sc, ow[u]);
    }
  }
  const float logz = M + __logf(L);
  const float* sl = slog + (long long)bh * K;
  float Mx = logz;
  for (int kx = 0; kx < kk; ++kx) Mx = fmaxf(Mx, sl[kx]);
  float Z = __expf(logz - Mx);
  for (int kx = 0; kx < kk; ++kx) Z += __expf(sl[kx] - Mx);
  const float aw = __expf(logz - Mx) / Z / L;
#pragma unroll
  for (int u = 0; u < MAXE; ++u) acc[u] = ow[u] * aw;
  for (int kx = 0; kx < kk; ++kx) {
    const float* pp = pb + (long long)kx * (d + 2);
    const float a = __expf(sl[kx] - Mx) / Z / pp[1];
#pragma unroll
    for (int u = 0; u < MAXE; ++u) {
      const int e = lane + 64 * u;
      if (e < d) acc[u] = fmaf(a, pp[2 + e], acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < MAXE; ++u) {
    const int e = lane + 64 * u;
    if (e < d) Elt<T>::st(out + (long long)bh * d + e, acc[u]);
  }
}

}  // namespace

hipError_t hils_launch_decode(const HilsShape& s, const void* q, const void* qr, const void* k,
                              const void* v, const int32_t* seqlen, const void* ksum,
                              const float* bsum, void* out, int32_t* sel, float* scores,
                              uint32_t* keys, float* slog, float* part, hipStream_t st) {
  const int NS = s.K + s.nwin;
  const float tau = (float)s.tau;
  const unsigned nsb = (unsigned)((s.nmax + SC_CPB - 1) / SC_CPB);
  const size_t ashm = (size_t)s.G * s.d * 4;
  if (s.dtype == 0) {
    if (nsb > 0)
      { HilsProfScope ps_("k_dec_score", st); hipLaunchKernelGGL(k_dec_score<bf16_t>, dim3(s.B * s.Hq, nsb), dim3(256), 0, st,
                         (const bf16_t*)qr, (const bf16_t*)ksum, bsum, seqlen, scores, s.Hq, s.nC,
                         s.nmax, s.N, s.d, s.S, s.W, tau); }
  } else {
    if (nsb > 0)
      { HilsProfScope ps_("k_dec_score", st); hipLaunchKernelGGL(k_dec_score<float>, dim3(s.B * s.Hq, nsb), dim3(256), 0, st,
                         (const float*)qr, (const float*)ksum, bsum, seqlen, scores, s.Hq, s.nC,
                         s.nmax, s.N, s.d, s.S, s.W, tau); }
  }
  { HilsProfScope ps_("k_dec_select", st); hipLaunchKernelGGL(k_dec_select, dim3(s.B * s.Hkv), dim3(SEL_NT), 0, st, scores, seqlen, keys,
                     sel, slog, s.Hq, s.Hkv, s.G, s.nmax > 0 ? s.nmax : 1, s.N, s.S, s.W, s.K); }
  if (s.dtype == 0) {
    { HilsProfScope ps_("k_dec_attn", st); hipLaunchKernelGGL(k_dec_attn<bf16_t>, dim3(s.B * s.Hkv, NS), dim3(AT_NT), ashm, st,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, seqlen, sel, part,
                       s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, NS, tau); }
    { HilsProfScope ps_("k_dec_combine", st); hipLaunchKernelGGL(k_dec_combine<bf16_t>, dim3(s.B * s.Hq), dim3(64), 0, st, part, slog,
                       seqlen, (bf16_t*)out, s.Hq, s.G, s.N, s.d, s.S, s.W, s.K, NS, s.nwin); }
  } else {
    { HilsProfScope ps_("k_dec_attn", st); hipLaunchKernelGGL(k_dec_attn<float>, dim3(s.B * s.Hkv, NS), dim3(AT_NT), ashm, st,
                       (const float*)q, (const float*)k, (const float*)v, seqlen, sel, part,
                       s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, NS, tau); }
    { HilsProfScope ps_("k_dec_combine", st); hipLaunchKernelGGL(k_dec_combine<float>, dim3(s.B * s.Hq), dim3(64), 0, st, part, slog,
                       seqlen, (float*)out, s.Hq, s.G, s.N, s.d, s.S, s.W, s.K, NS, s.nwin); }
  }
  return hipGetLastError();
}
