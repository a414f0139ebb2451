// Landmark chunk summaries (k'_c, b'_c).
//
// "Hierarchical Sparse Attention Done Right", section 3 (Proposition 3.1 and
// the landmark-token text): the landmark query q'_c attends over the S keys of
// chunk c; k'_c is the attention-weighted key sum and b'_c the entropy of the
// attention weights, i.e. Attn(q'_c, K_c, K_c).  One wavefront per
// (batch, query head, chunk); lane j owns token j of the chunk.  The math is
// done in double precision and rounded once to the storage type, so the
// bf16/fp32 summary is the correctly rounded value of the exact summary.
#include "hils_device.h"
#include "hils_internal.h"

namespace {

// Paged cache (pages != nullptr): item = listed page x query head; the page's
// S keys are k[p][g][0..S), its landmark query lm[p][h], and the summary goes
// to ksum[p][h], bsum[p][h].  Page ids are clamped into [0, npages).
template <typename T>
__global__ void __launch_bounds__(64)
k_summarize(const T* __restrict__ k, const T* __restrict__ lm, T* __restrict__ ksum,
            float* __restrict__ bsum, int Hq, int Hkv, int N, int d, int S, int nC,
            int c0, int ncs, double tau, int landmark_key, const int32_t* __restrict__ pages,
            int npages) {
  extern __shared__ double sm_sum[];
  double* qd = sm_sum;        // [d]
  double* pj = sm_sum + d;    // [S]
  const int lane = threadIdx.x;
  const long long item = blockIdx.x;
  const T* kc;
  const T* qc;
  T* ko;
  float* bo;
  int h;
  if (pages) {
    h = (int)(item % Hq);
    const long long p = min(max(pages[item / Hq], 0), npages - 1);
    const int g = h / (Hq / Hkv);
    kc = k + ((p * Hkv + g) * (long long)S) * d;
    qc = lm + (p * Hq + h) * (long long)d;
    ko = ksum + (p * Hq + h) * (long long)d;
    bo = bsum + p * Hq + h;
  } else {
    const int c = c0 + (int)(item % ncs);
    const long long bh = item / ncs;
    h = (int)(bh % Hq);
    const long long b = bh / Hq;
    const int g = h / (Hq / Hkv);
    kc = k + (((b * Hkv + g) * (long long)N) + (long long)c * S) * d;
    qc = lm + ((b * Hq + h) * (long long)nC + c) * d;
    ko = ksum + ((b * Hq + h) * (long long)nC + c) * d;
    bo = bsum + (b * Hq + h) * (long long)nC + c;
  }

  if (landmark_key == 1) {       // ablation: the landmark row is the routing key
    for (int e = lane; e < d; e += 64) ko[e] = qc[e];
    if (lane == 0) *bo = 0.0f;
    return;
  }
  if (landmark_key == 3) {       // mean-pooled key, b' = ln S (uniform weights)
    for (int e = lane; e < d; e += 64) {
      double acc = 0.0;
      for (int j = 0; j < S; ++j) acc += (double)Elt<T>::ld(kc + (long long)j * d + e);
      Elt<T>::st64(ko + e, acc / (double)S);
    }
    if (lane == 0) *bo = (float)log((double)S);
    return;
  }
  for (int e = lane; e < d; e += 64) qd[e] = (double)Elt<T>::ld(qc + e);
  __syncthreads();
  double t = -INFINITY;
  if (lane < S) {
    const T* kr = kc + (long long)lane * d;
    double acc = 0.0;
    for (int e = 0; e < d; ++e) acc = fma(qd[e], (double)Elt<T>::ld(kr + e), acc);
    t = tau * acc;
  }
  const double m = wave_max_d(t);
  const double ex = (lane < S) ? exp(t - m) : 0.0;
  const double z = wave_sum_d(ex);
  const double p = ex / z;
  const double logp = (t - m) - log(z);
  const double ent = wave_sum_d((lane < S) ? -p * logp : 0.0);
  if (lane < S) pj[lane] = p;
  __syncthreads();
  for (int e = lane; e < d; e += 64) {
    double acc = 0.0;
    for (int j = 0; j < S; ++j) acc = fma(pj[j], (double)Elt<T>::ld(kc + (long long)j * d + e), acc);
    Elt<T>::st64(ko + e, acc);
  }
  if (lane == 0) *bo = (float)ent;
}

}  // namespace

hipError_t hils_launch_summarize(const HilsShape& s, const void* k, const void* lm, int c0, int c1,
                                 void* ksum, float* bsum, hipStream_t st) {
  const int ncs = c1 - c0;
  if (ncs <= 0) return hipSuccess;
  const long long nblk = (long long)s.B * s.Hq * ncs;
  const size_t shm = sizeof(double) * (s.d + 64);
  const int lk = s.mode;          // 0 surrogate, 1 landmark key, 3 mean pool
  if (s.dtype == 0)
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<bf16_t>, dim3((unsigned)nblk), dim3(64), shm, st,
                       (const bf16_t*)k, (const bf16_t*)lm, (bf16_t*)ksum, bsum, s.Hq, s.Hkv, s.N,
                       s.d, s.S, s.nC, c0, ncs, (double)s.tau, lk, nullptr, 0); }
  else
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<float>, dim3((unsigned)nblk), dim3(64), shm, st,
                       (const float*)k, (const float*)lm, (float*)ksum, bsum, s.Hq, s.Hkv, s.N,
                       s.d, s.S, s.nC, c0, ncs, (double)s.tau, lk, nullptr, 0); }
  return hipGetLastError();
}

hipError_t hils_launch_summarize_paged(const HilsShape& s, const void* k_pages, const void* lm_pages,
                                       const int32_t* pages, int npages_listed, int num_pages,
                                       void* ksum_pages, float* bsum_pages, hipStream_t st) {
  if (npages_listed <= 0) return hipSuccess;
  const long long nblk = (long long)npages_listed * s.Hq;
  const size_t shm = sizeof(double) * (s.d + 64);
  const int lk = s.mode;
  if (s.dtype == 0)
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<bf16_t>, dim3((unsigned)nblk), dim3(64), shm, st,
                       (const bf16_t*)k_pages, (const bf16_t*)lm_pages, (bf16_t*)ksum_pages, bsum_pages,
                       s.Hq, s.Hkv, s.N, s.d, s.S, s.nC, 0, 1, (double)s.tau, lk, pages, num_pages); }
  else
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<float>, dim3((unsigned)nblk), dim3(64), shm, st,
                       (const float*)k_pages, (const float*)lm_pages, (float*)ksum_pages, bsum_pages,
                       s.Hq, s.Hkv, s.N, s.d, s.S, s.nC, 0, 1, (double)s.tau, lk, pages, num_pages); }
  return hipGetLastError();
}
