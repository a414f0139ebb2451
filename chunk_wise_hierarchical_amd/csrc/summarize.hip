// Landmark chunk summaries (k'_c, b'_c).
//
// "Hierarchical Sparse Attention Done Right", section 3 (Proposition 3.1 and
// the landmark-token text): the landmark query q'_c attends over the S keys of
// chunk c; k'_c is the attention-weighted key sum and b'_c the entropy of the
// attention weights, i.e. Attn(q'_c, K_c, K_c).  One workgroup (4 wavefronts)
// per (batch, KV group, chunk): the chunk's key rows are staged in LDS once,
// with 16-byte loads, and serve every query head of the group; wavefront w
// takes the group's heads w, w + 4, ...  For the logits lane j owns key j and
// reads its row from LDS in element order; the weighted key sum takes one
// element per lane.  The math is done in double precision and rounded once to
// the storage type, so the bf16/fp32 summary is the correctly rounded value
// of the exact summary.
#include "hils_device.h"
#include "hils_internal.h"

namespace {

constexpr int SM_NT = 256;

// Paged cache (pages != nullptr): item = listed page x KV group; the page's S
// keys are k[p][g][0..S), the landmark query of head h lm[p][h], and the
// summary goes to ksum[p][h], bsum[p][h].  Page ids are clamped into
// [0, npages).
template <typename T>
__global__ void __launch_bounds__(SM_NT)
k_summarize(const T* __restrict__ k, const T* __restrict__ lm, T* __restrict__ ksum,
            float* __restrict__ bsum, int Hq, int Hkv, int N, int d, int S, int nC,
            int c0, int ncs, double tau, int landmark_key, const int32_t* __restrict__ pages,
            int npages) {
  constexpr int V = 16 / (int)sizeof(T);       // elements per 16-byte piece
  extern __shared__ double sm_sum[];
  const int kst = d + V;                       // key row stride in LDS (elements)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double* qd = sm_sum + (size_t)w * (d + 64);  // this wavefront's [d] landmark query
  double* pj = qd + d;                         // and [S] attention weights
  T* tile = reinterpret_cast<T*>(sm_sum + (size_t)4 * (d + 64));   // [S][kst]
  const int G = Hq / Hkv;
  const long long item = blockIdx.x;
  const T* kc;
  long long p = 0, b = 0;
  int g, c = 0;
  if (pages) {
    g = (int)(item % Hkv);
    p = min(max(pages[item / Hkv], 0), npages - 1);
    kc = k + ((p * Hkv + g) * (long long)S) * d;
  } else {
    c = c0 + (int)(item % ncs);
    const long long bg = item / ncs;
    g = (int)(bg % Hkv);
    b = bg / Hkv;
    kc = k + (((b * Hkv + g) * (long long)N) + (long long)c * S) * d;
  }
  // 16-byte pieces when a row is a whole number of them (rows then stay
  // 16-byte aligned in memory and in LDS), single elements otherwise
  const bool vec = d % V == 0;
  if (landmark_key != 1) {
    if (vec) {
      const int ppr = d / V;                   // pieces per row
      for (int t = threadIdx.x; t < S * ppr; t += SM_NT) {
        const int row = t / ppr, pc = t - row * ppr;
        *reinterpret_cast<uint4*>(tile + row * kst + pc * V) =
            *reinterpret_cast<const uint4*>(kc + (long long)row * d + pc * V);
      }
    } else {
      for (int t = threadIdx.x; t < S * d; t += SM_NT) {
        const int row = t / d, e = t - row * d;
        tile[row * kst + e] = kc[(long long)row * d + e];
      }
    }
    __syncthreads();
  }
  for (int r = w; r < G; r += 4) {
    const int h = g * G + r;
    const T* qc;
    T* ko;
    float* bo;
    if (pages) {
      qc = lm + (p * Hq + h) * (long long)d;
      ko = ksum + (p * Hq + h) * (long long)d;
      bo = bsum + p * Hq + h;
    } else {
      qc = lm + ((b * Hq + h) * (long long)nC + c) * d;
      ko = ksum + ((b * Hq + h) * (long long)nC + c) * d;
      bo = bsum + (b * Hq + h) * (long long)nC + c;
    }
    if (landmark_key == 1) {       // ablation: the landmark row is the routing key
      for (int e = lane; e < d; e += 64) ko[e] = qc[e];
      if (lane == 0) *bo = 0.0f;
      continue;
    }
    if (landmark_key == 3) {       // mean-pooled key, b' = ln S (uniform weights)
      for (int e = lane; e < d; e += 64) {
        double acc = 0.0;
        for (int j = 0; j < S; ++j) acc += (double)Elt<T>::ld(tile + j * kst + e);
        Elt<T>::st64(ko + e, acc / (double)S);
      }
      if (lane == 0) *bo = (float)log((double)S);
      continue;
    }
    for (int e = lane; e < d; e += 64) qd[e] = (double)Elt<T>::ld(qc + e);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // qd, from every lane
    double t = -INFINITY;
    if (lane < S) {
      const T* kr = tile + lane * kst;
      double acc = 0.0;
      if (vec) {
        for (int e0 = 0; e0 < d; e0 += V) {
          const uint4 u = *reinterpret_cast<const uint4*>(kr + e0);
          const T* x = reinterpret_cast<const T*>(&u);
#pragma unroll
          for (int u2 = 0; u2 < V; ++u2) acc = fma(qd[e0 + u2], (double)Elt<T>::ld(x + u2), acc);
        }
      } else {
        for (int e = 0; e < d; ++e) acc = fma(qd[e], (double)Elt<T>::ld(kr + e), acc);
      }
      t = tau * acc;
    }
    const double m = wave_max_d(t);
    const double ex = (lane < S) ? exp(t - m) : 0.0;
    const double z = wave_sum_d(ex);
    const double pr = ex / z;
    const double logp = (t - m) - log(z);
    const double ent = wave_sum_d((lane < S) ? -pr * logp : 0.0);
    if (lane < S) pj[lane] = pr;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // pj, from every lane
    for (int e = lane; e < d; e += 64) {
      double acc = 0.0;
      for (int j = 0; j < S; ++j) acc = fma(pj[j], (double)Elt<T>::ld(tile + j * kst + e), acc);
      Elt<T>::st64(ko + e, acc);
    }
    if (lane == 0) *bo = (float)ent;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // qd and pj read before the next head
  }
}

size_t summarize_lds(const HilsShape& s) {
  const size_t esz = s.dtype == 0 ? 2 : 4;
  return sizeof(double) * 4 * (s.d + 64) + (size_t)s.S * (s.d + 16 / esz) * esz;
}

}  // namespace

hipError_t hils_launch_summarize(const HilsShape& s, const void* k, const void* lm, int c0, int c1,
                                 void* ksum, float* bsum, hipStream_t st) {
  const int ncs = c1 - c0;
  if (ncs <= 0) return hipSuccess;
  const long long nblk = (long long)s.B * s.Hkv * ncs;
  const size_t shm = summarize_lds(s);
  const int lk = s.mode;          // 0 surrogate, 1 landmark key, 3 mean pool
  hils_allow_lds(s.dtype == 0 ? (const void*)k_summarize<bf16_t> : (const void*)k_summarize<float>, shm);
  if (s.dtype == 0)
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<bf16_t>, dim3((unsigned)nblk), dim3(SM_NT), shm, st,
                       (const bf16_t*)k, (const bf16_t*)lm, (bf16_t*)ksum, bsum, s.Hq, s.Hkv, s.N,
                       s.d, s.S, s.nC, c0, ncs, (double)s.tau, lk, nullptr, 0); }
  else
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<float>, dim3((unsigned)nblk), dim3(SM_NT), shm, st,
                       (const float*)k, (const float*)lm, (float*)ksum, bsum, s.Hq, s.Hkv, s.N,
                       s.d, s.S, s.nC, c0, ncs, (double)s.tau, lk, nullptr, 0); }
  return hipGetLastError();
}

hipError_t hils_launch_summarize_paged(const HilsShape& s, const void* k_pages, const void* lm_pages,
                                       const int32_t* pages, int npages_listed, int num_pages,
                                       void* ksum_pages, float* bsum_pages, hipStream_t st) {
  if (npages_listed <= 0) return hipSuccess;
  const long long nblk = (long long)npages_listed * s.Hkv;
  const size_t shm = summarize_lds(s);
  const int lk = s.mode;
  hils_allow_lds(s.dtype == 0 ? (const void*)k_summarize<bf16_t> : (const void*)k_summarize<float>, shm);
  if (s.dtype == 0)
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<bf16_t>, dim3((unsigned)nblk), dim3(SM_NT), shm, st,
                       (const bf16_t*)k_pages, (const bf16_t*)lm_pages, (bf16_t*)ksum_pages, bsum_pages,
                       s.Hq, s.Hkv, s.N, s.d, s.S, s.nC, 0, 1, (double)s.tau, lk, pages, num_pages); }
  else
    { HilsProfScope ps_("k_summarize", st); hipLaunchKernelGGL(k_summarize<float>, dim3((unsigned)nblk), dim3(SM_NT), shm, st,
                       (const float*)k_pages, (const float*)lm_pages, (float*)ksum_pages, bsum_pages,
                       s.Hq, s.Hkv, s.N, s.d, s.S, s.nC, 0, 1, (double)s.tau, lk, pages, num_pages); }
  return hipGetLastError();
}
