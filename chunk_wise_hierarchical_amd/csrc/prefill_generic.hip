// Generic vector-ALU prefill kernels: chunk scoring + exact top-K selection,
// and window + selected-chunk attention with chunk-level fusion.
//
// These handle every supported shape and both element types (bf16, fp32);
// the MFMA kernels cover the bf16 d=128, S=64 fast path.  One workgroup per
// (batch, KV head, query position).
//
// "Hierarchical Sparse Attention Done Right":
//   section 3, routing equation — s_hat = scale * q_hat . k'_c + b'_c over the
//     candidate chunks C_i, top-K by s_hat (ties: lower chunk id first);
//   section 4.1, GQA — per-head log-softmax of s_hat over C_i, maximum over the
//     heads of the group, one shared top-K;
//   section 3, hierarchical softmax — independent softmax inside the window
//     and inside each selected chunk; chunk-level softmax over
//     {s_hat_c : c selected} U {log Z_swa} mixes the parts.
#include "hils_device.h"
#include "hils_internal.h"

namespace {

constexpr int NT = 256;  // threads per workgroup (4 wavefronts)

// exclusive prefix count of `flag` across the workgroup; returns the total.
__device__ __forceinline__ int block_excl_scan(int flag, int* wsum, int& pos) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int inwave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(bal);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int u = 0; u < NT / 64; ++u) {
    if (u < w) before += wsum[u];
    total += wsum[u];
  }
  pos = before + inwave;
  __syncthreads();
  return total;
}

// combine two (max, sum-of-exp) pairs
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) { m = M; s = 0.0f; return; }
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_select_generic(const T* __restrict__ qr, const T* __restrict__ kk_, const T* __restrict__ ksum,
                 const float* __restrict__ bsum, int32_t* __restrict__ sel,
                 float* __restrict__ slog, int Hq, int Hkv, int G, int N, int d, int S, int W,
                 int K, int nC, float tau, int exact) {
  extern __shared__ __align__(16) unsigned char sm_raw[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t suf[256];
  __shared__ float red_m[NT / 64][8], red_s[NT / 64][8];
  __shared__ float Lh[8];
  __shared__ int wsum[NT / 64];
  __shared__ int sh_digit, sh_need;
  __shared__ int wl[128];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long blk = blockIdx.x;
  const int i = (int)(blk % N);
  const long long bg = blk / N;
  const int g = (int)(bg % Hkv);
  const long long b = bg / Hkv;
  const int n = n_cand(i, W, S);
  const int kk = min(K, n);
  int32_t* so = sel + ((b * Hkv + g) * (long long)N + i) * K;
  const long long hbase = b * Hq + (long long)g * G;   // first query head of the group

  for (int t = tid; t < K; t += NT)
    if (t >= kk) so[t] = -1;
  for (int t = tid; t < G * K; t += NT) {
    const int r = t / K, kx = t % K;
    if (kx >= kk) slog[((hbase + r) * N + i) * (long long)K + kx] = 0.0f;
  }
  if (n == 0) return;

  float* qs = reinterpret_cast<float*>(sm_raw);
  uint64_t* keys = reinterpret_cast<uint64_t*>(sm_raw + (((size_t)G * d * 4 + 15) & ~(size_t)15));
  for (int t = tid; t < G * d; t += NT) {
    const int r = t / d, e = t % d;
    qs[t] = Elt<T>::ld(qr + ((hbase + r) * N + i) * (long long)d + e);
  }
  __syncthreads();

  // s_hat for head r of the group and chunk c (fixed fma order => reproducible).
  // Exact mode (section 2.1): log sum_{j in chunk c} exp(scale q.k_j), max-shifted.
  auto score = [&](int r, int c) -> float {
    const float* qq = qs + r * d;
    if (exact) {
      const T* kc = kk_ + ((b * Hkv + g) * (long long)N + (long long)c * S) * d;
      float m = -INFINITY, s = 0.0f;
      for (int j = 0; j < S; ++j) {
        float acc = 0.0f;
        for (int e = 0; e < d; ++e) acc = fmaf(qq[e], Elt<T>::ld(kc + (long long)j * d + e), acc);
        const float x = tau * acc;
        if (x > m) { s = s * expf(m - x) + 1.0f; m = x; } else { s += expf(x - m); }
      }
      return m + logf(s);
    }
    const T* kp = ksum + ((hbase + r) * nC + c) * (long long)d;
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc = fmaf(qq[e], Elt<T>::ld(kp + e), acc);
    return fmaf(tau, acc, bsum[(hbase + r) * nC + c]);
  };

  // per-head log-sum-exp over the candidates (GQA normalisation)
  if (G > 1) {
    for (int r = 0; r < G; ++r) {
      float m = -INFINITY, s = 0.0f;
      for (int c = tid; c < n; c += NT) {
        const float x = score(r, c);
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
      for (int u = 1; u < NT / 64; ++u) lse_merge(m, s, red_m[u][tid], red_s[u][tid]);
      Lh[tid] = m + __logf(s);
    }
    __syncthreads();
  }

  // unique 64-bit keys: high word = ordered group score, low word = ~chunk id
  for (int c = tid; c < n; c += NT) {
    float gs;
    if (G == 1) {
      gs = score(0, c);
    } else {
      gs = -INFINITY;
      for (int r = 0; r < G; ++r) gs = fmaxf(gs, score(r, c) - Lh[r]);
    }
    keys[c] = ((uint64_t)f32_order_key(gs) << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
  }
  if (tid == 0) sh_need = kk;
  __syncthreads();

  // MSD radix select of the kk-th largest key, 8 bits per pass
  uint64_t prefix = 0, pmask = 0;
  for (int p = 7; p >= 0; --p) {
    hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < n; c += NT) {
      const uint64_t key = keys[c];
      if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> (8 * p)) & 255u], 1u);
    }
    __syncthreads();
    suf[tid] = hist[tid];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {            // inclusive suffix sums
      const uint32_t add = (tid + off < 256) ? suf[tid + off] : 0u;
      __syncthreads();
      suf[tid] += add;
      __syncthreads();
    }
    const int need = sh_need;
    const uint32_t above = (tid < 255) ? suf[tid + 1] : 0u;
    if (suf[tid] >= (uint32_t)need && above < (uint32_t)need) { sh_digit = tid; }
    __syncthreads();
    const int dg = sh_digit;
    if (tid == dg) sh_need = need - (int)((dg < 255) ? suf[dg + 1] : 0u);
    prefix |= (uint64_t)dg << (8 * p);
    pmask |= (uint64_t)0xff << (8 * p);
    __syncthreads();
  }
  const uint64_t thr = prefix;  // the kk-th largest key; exactly kk keys are >= thr

  // compaction in ascending chunk order
  int running = 0;
  for (int base = 0; base < n; base += NT) {
    const int c = base + tid;
    const int f = (c < n) && (keys[c] >= thr);
    int pos;
    const int tot = block_excl_scan(f, wsum, pos);
    if (f) { so[running + pos] = c; wl[running + pos] = c; }
    running += tot;
  }
  __syncthreads();
  for (int t = tid; t < G * kk; t += NT) {
    const int r = t / kk, kx = t % kk;
    slog[((hbase + r) * N + i) * (long long)K + kx] = score(r, wl[kx]);
  }
}

template <typename T>
__global__ void __launch_bounds__(NT)
k_attn_generic(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
               const int32_t* __restrict__ sel, const float* __restrict__ slog, T* __restrict__ out,
               int Hq, int Hkv, int G, int N, int d, int S, int W, int K, float tau) {
  extern __shared__ __align__(16) unsigned char sm_raw[];
  __shared__ float m_run[8], l_run[8], scl[8], lz[8], a_swa[8];
  __shared__ float alpha[8][128];
  __shared__ int csel[128];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long blk = blockIdx.x;
  const int i = (int)(blk % N);
  const long long bg = blk / N;
  const int g = (int)(bg % Hkv);
  const long long b = bg / Hkv;
  const int n = n_cand(i, W, S);
  const int kk = min(K, n);
  const long long w0 = window_start(i, W, S);
  const long long hbase = b * Hq + (long long)g * G;
  const T* kg = k + (b * Hkv + g) * (long long)N * d;
  const T* vg = v + (b * Hkv + g) * (long long)N * d;

  float* qs = reinterpret_cast<float*>(sm_raw);            // [G][d]
  float* ps = qs + G * d;                                  // [G][NT] logits / probabilities
  const int GD = G * d;
  constexpr int MAXO = 8;                                  // G*d <= 2048 = 8 * NT
  float o[MAXO];
#pragma unroll
  for (int u = 0; u < MAXO; ++u) o[u] = 0.0f;

  for (int t = tid; t < GD; t += NT) {
    const int r = t / d, e = t % d;
    qs[t] = Elt<T>::ld(q + ((hbase + r) * N + i) * (long long)d + e);
  }
  if (tid < G) { m_run[tid] = -INFINITY; l_run[tid] = 0.0f; }
  if (tid < kk) csel[tid] = sel[((b * Hkv + g) * (long long)N + i) * K + tid];
  __syncthreads();

  // logits of tokens [j0, j0+jn) for every head of the group into ps
  auto logits = [&](long long j0, int jn) {
    if (tid < jn) {
      const T* kr = kg + (j0 + tid) * d;
      for (int r = 0; r < G; ++r) {
        const float* qq = qs + r * d;
        float acc = 0.0f;
        for (int e = 0; e < d; ++e) acc = fmaf(qq[e], Elt<T>::ld(kr + e), acc);
        ps[r * NT + tid] = tau * acc;
      }
    }
  };

  // ---- window [w0, i]: online softmax over tiles of NT tokens ----------------
  for (long long j0 = w0; j0 <= i; j0 += NT) {
    const int jn = (int)min((long long)NT, (long long)i - j0 + 1);
    logits(j0, jn);
    __syncthreads();
    for (int r = wv; r < G; r += NT / 64) {
      float mx = -INFINITY;
      for (int t = lane; t < jn; t += 64) mx = fmaxf(mx, ps[r * NT + t]);
      mx = wave_max_f(mx);
      const float mnew = fmaxf(m_run[r], mx);
      float sum = 0.0f;
      for (int t = lane; t < jn; t += 64) {
        const float p = __expf(ps[r * NT + t] - mnew);
        ps[r * NT + t] = p;
        sum += p;
      }
      sum = wave_sum_f(sum);
      if (lane == 0) {
        const float sc = __expf(m_run[r] - mnew);     // 0 on the first tile
        scl[r] = sc;
        l_run[r] = l_run[r] * sc + sum;
        m_run[r] = mnew;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MAXO; ++u) {
      const int idx = tid + u * NT;
      if (idx < GD) {
        const int r = idx / d, e = idx % d;
        float acc = o[u] * scl[r];
        const float* pr = ps + r * NT;
        for (int t = 0; t < jn; ++t) acc = fmaf(pr[t], Elt<T>::ld(vg + (j0 + t) * d + e), acc);
        o[u] = acc;
      }
    }
    __syncthreads();
  }

  // ---- chunk-level fusion weights: softmax over {s_hat_c} U {log Z_swa} -------
  if (tid < G) {
    const int r = tid;
    const float logz = m_run[r] + __logf(l_run[r]);
    lz[r] = logz;
    const float* sl = slog + ((hbase + r) * N + i) * (long long)K;
    float M = logz;
    for (int kx = 0; kx < kk; ++kx) M = fmaxf(M, sl[kx]);
    float Z = __expf(logz - M);
    for (int kx = 0; kx < kk; ++kx) Z += __expf(sl[kx] - M);
    for (int kx = 0; kx < kk; ++kx) alpha[r][kx] = __expf(sl[kx] - M) / Z;
    a_swa[r] = __expf(logz - M) / Z;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < MAXO; ++u) {
    const int idx = tid + u * NT;
    if (idx < GD) { const int r = idx / d; o[u] = o[u] * (a_swa[r] / l_run[r]); }
  }

  // ---- selected chunks: one independent softmax per chunk ---------------------
  for (int kx = 0; kx < kk; ++kx) {
    const long long j0 = (long long)csel[kx] * S;
    logits(j0, S);
    __syncthreads();
    for (int r = wv; r < G; r += NT / 64) {
      float mx = -INFINITY;
      for (int t = lane; t < S; t += 64) mx = fmaxf(mx, ps[r * NT + t]);
      mx = wave_max_f(mx);
      float sum = 0.0f;
      for (int t = lane; t < S; t += 64) {
        const float p = __expf(ps[r * NT + t] - mx);
        ps[r * NT + t] = p;
        sum += p;
      }
      sum = wave_sum_f(sum);
      if (lane == 0) scl[r] = alpha[r][kx] / sum;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MAXO; ++u) {
      const int idx = tid + u * NT;
      if (idx < GD) {
        const int r = idx / d, e = idx % d;
        const float* pr = ps + r * NT;
        float acc = 0.0f;
        for (int t = 0; t < S; ++t) acc = fmaf(pr[t], Elt<T>::ld(vg + (j0 + t) * d + e), acc);
        o[u] = fmaf(scl[r], acc, o[u]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < MAXO; ++u) {
    const int idx = tid + u * NT;
    if (idx < GD) {
      const int r = idx / d, e = idx % d;
      Elt<T>::st(out + ((hbase + r) * N + i) * (long long)d + e, o[u]);
    }
  }
}

}  // namespace

hipError_t hils_launch_select_generic(const HilsShape& s, const void* qr, const void* k,
                                      const void* ksum, const float* bsum, int32_t* sel,
                                      float* slog, hipStream_t st) {
  const int exact = (s.mode == 2);
  const long long nblk = (long long)s.B * s.Hkv * s.N;
  const size_t shm = (((size_t)s.G * s.d * 4 + 15) & ~(size_t)15) + (size_t)8 * (s.nmax > 0 ? s.nmax : 1);
  if (s.dtype == 0) {
    auto f = k_select_generic<bf16_t>;
    hils_allow_lds((const void*)f, shm);
    { HilsProfScope ps_("k_select_generic", st); hipLaunchKernelGGL(f, dim3((unsigned)nblk), dim3(NT), shm, st, (const bf16_t*)qr,
                       (const bf16_t*)k, (const bf16_t*)ksum, bsum, sel, slog, s.Hq, s.Hkv, s.G, s.N,
                       s.d, s.S, s.W, s.K, s.nC, (float)s.tau, exact); }
  } else {
    auto f = k_select_generic<float>;
    hils_allow_lds((const void*)f, shm);
    { HilsProfScope ps_("k_select_generic", st); hipLaunchKernelGGL(f, dim3((unsigned)nblk), dim3(NT), shm, st, (const float*)qr,
                       (const float*)k, (const float*)ksum, bsum, sel, slog, s.Hq, s.Hkv, s.G, s.N,
                       s.d, s.S, s.W, s.K, s.nC, (float)s.tau, exact); }
  }
  return hipGetLastError();
}

hipError_t hils_launch_attn_generic(const HilsShape& s, const void* q, const void* k, const void* v,
                                    const int32_t* sel, const float* slog, void* out, hipStream_t st) {
  const long long nblk = (long long)s.B * s.Hkv * s.N;
  const size_t shm = (size_t)s.G * s.d * 4 + (size_t)s.G * NT * 4;
  if (s.dtype == 0) {
    auto f = k_attn_generic<bf16_t>;
    hils_allow_lds((const void*)f, shm);
    { HilsProfScope ps_("k_attn_generic", st); hipLaunchKernelGGL(f, dim3((unsigned)nblk), dim3(NT), shm, st, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, sel, slog, (bf16_t*)out, s.Hq, s.Hkv,
                       s.G, s.N, s.d, s.S, s.W, s.K, (float)s.tau); }
  } else {
    auto f = k_attn_generic<float>;
    hils_allow_lds((const void*)f, shm);
    { HilsProfScope ps_("k_attn_generic", st); hipLaunchKernelGGL(f, dim3((unsigned)nblk), dim3(NT), shm, st, (const float*)q,
                       (const float*)k, (const float*)v, sel, slog, (float*)out, s.Hq, s.Hkv,
                       s.G, s.N, s.d, s.S, s.W, s.K, (float)s.tau); }
  }
  return hipGetLastError();
}
