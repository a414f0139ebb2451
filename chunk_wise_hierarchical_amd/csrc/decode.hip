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

using fastp::fast_exp2;
using fastp::ld_bf16x8;
using fastp::LN2;
using fastp::LOG2E;
using fastp::max_x16;
using fastp::max_x32;
using fastp::mfma16;
using fastp::pack_bf16x2;
using fastp::sum_x16;
using fastp::sum_x32;

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
constexpr int AT_NT = 256;                    // threads of a split-attention workgroup
constexpr int DA_D = 128, DA_S = 64;          // shape of the specialised bf16 split attention

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

template <bool PAGED, int G>
__device__ __forceinline__ void dec_split_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                               const bf16_t* __restrict__ v, const int32_t* __restrict__ seqlen,
                                               const int32_t* __restrict__ sel, float* __restrict__ part,
                                               int Hq, int Hkv, int N, int W, int K, int NS, float tau,
                                               int M, PageMap pm, int bgm, int s);

// The window tiles of a single-token step do not depend on the selection, so
// with WG > 0 (bf16, d = 128, S = 64, G = WG heads per KV group) the scoring
// grid carries them: workgroups x >= nsb of row y = (sequence, head h) run
// window splits h % WG + WG j of that head's KV group, interleaved with the
// scoring workgroups so that their loads share the scoring pass's time.
struct WinArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  float* part;
  int Hkv, K, NS, nwin;
};

template <typename T, bool PAGED, int MT, int WG>
__global__ void __launch_bounds__(256)
k_dec_score(const T* __restrict__ qr, const T* __restrict__ ksum, const float* __restrict__ bsum,
            const int32_t* __restrict__ seqlen, float* __restrict__ scores, float* __restrict__ lsep,
            int Hq, int nC, int nmax, int nsb, int N, int d, int S, int W, float tau, int M,
            PageMap pm, WinArgs wa) {
  constexpr int V = Vec<T>::N;
  constexpr int MAXT = 256 / (16 * V) > 0 ? 256 / (16 * V) : 1;
  constexpr int R = 16;
  __shared__ float red_m[4][MT], red_s[4][MT];
  if constexpr (WG > 0) {
    if ((int)blockIdx.x >= nsb) {
      const int bq = (int)(blockIdx.y / Hq), hq = (int)(blockIdx.y % Hq);
      const int w = hq % WG + WG * ((int)blockIdx.x - nsb);
      if (w < wa.nwin)
        dec_split_bf16<PAGED, WG>(wa.q, wa.k, wa.v, seqlen, nullptr, wa.part, Hq, wa.Hkv, N, W, wa.K,
                                  wa.NS, tau, 1, pm, bq * wa.Hkv + hq / WG, wa.K + w);
      return;
    }
  }
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

constexpr int SEL_LDS_KEYS = HILS_DEC_SEL_LDS_KEYS;   // keys kept in LDS (96 KB) when they fit

// Exact top-K of the group scores, ties to the lower chunk id.  A query with
// at most `span` candidates takes one workgroup (SEL_WHOLE).  A longer
// candidate list is cut into P partitions of `span` chunks: SEL_PART finds
// each partition's own top-K (the global top-K is contained in the union of
// the partitions' top-K lists under the same order) and writes it as
// (key, chunk id) in ascending chunk order, and SEL_MERGE selects the top-K
// of those P * K candidates; the merged list is in ascending chunk order too,
// so both paths take tied keys lowest chunk id first.
enum { SEL_WHOLE = 0, SEL_PART = 1, SEL_MERGE = 2 };

// The radix histogram is kept in SEL_REP copies, lane l counting into copy
// l % SEL_REP: the keys of one query sit within a few octaves, so most of a
// pass's keys share a digit and one shared copy would serialise their atomics.
constexpr int SEL_REP = 32;

// GT > 0: G is GT, and every head's scores of a round of 8 x SEL_NT candidates
// are loaded together (before the log-sum-exp, whose latency they overlap).
template <int PH, int GT>
__global__ void __launch_bounds__(SEL_NT)
k_dec_select(const float* __restrict__ scores, const float* __restrict__ lsep,
             const int32_t* __restrict__ seqlen, uint32_t* __restrict__ keys, uint2* __restrict__ cand,
             int32_t* __restrict__ sel, float* __restrict__ slog, int Hq, int Hkv, int Gr, int nmax,
             int nsb, int N, int S, int W, int K, int M, int span, int P) {
  extern __shared__ uint32_t sel_keys_lds[];
  __shared__ __align__(16) uint32_t hist[256 * SEL_REP];
  __shared__ uint32_t htot[256];
  __shared__ float Lh[8];
  const int G = GT > 0 ? GT : Gr;
  __shared__ int wsum[SEL_NW];
  __shared__ int sh_digit, sh_need;
  __shared__ uint32_t sh_tkey;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bgm = blockIdx.x;                 // (sequence, KV group, query)
  const int part = (PH == SEL_PART) ? (int)blockIdx.y : 0;
  const int m = bgm % M, bg = bgm / M;
  const int b = bg / Hkv, g = bg % Hkv;
  const int n = n_cand(dec_pos(seqlen[b], N, M, m), W, S);
  const int kk = min(K, n);
  // per-head rows of this query: ((b * Hq + g * G + r) * M + m)
  auto hrow = [&](int r) { return ((long long)b * Hq + (long long)g * G + r) * M + m; };
  int32_t* so = sel + (long long)bgm * K;
  uint2* co = cand + ((long long)bgm * P + part) * K;   // this partition's candidate slots
  // the candidate range of this workgroup: chunks [c0, c0 + cnt) (SEL_MERGE:
  // the P * K candidate slots)
  const int c0 = (PH == SEL_PART) ? part * span : 0;
  const int cnt = (PH == SEL_WHOLE) ? n : (PH == SEL_PART) ? max(0, min(n - c0, span)) : P * K;
  const int kl = (PH == SEL_PART) ? min(K, cnt) : kk;   // keys this workgroup selects
  if (PH != SEL_PART) {
    for (int t = tid; t < K; t += SEL_NT) if (t >= kk) so[t] = -1;
    for (int t = tid; t < G * K; t += SEL_NT) {
      const int r = t / K, kx = t % K;
      if (kx >= kk) slog[hrow(r) * K + kx] = 0.0f;
    }
  } else {
    for (int t = tid; t < K; t += SEL_NT) if (t >= kl) co[t] = make_uint2(0u, 0xffffffffu);
  }
  if (kk == 0 || kl == 0) return;
  uint32_t* ky = (cnt <= SEL_LDS_KEYS) ? sel_keys_lds : keys + (long long)bgm * nmax + c0;
  // SEL_MERGE: candidate chunk ids next to their keys in LDS (cnt <= 8192)
  int32_t* cid = reinterpret_cast<int32_t*>(sel_keys_lds) + cnt;

  if (PH == SEL_MERGE) {
    const uint2* ci = cand + (long long)bgm * P * K;
    for (int t = tid; t < cnt; t += SEL_NT) {
      const uint2 e = ci[t];
      ky[t] = e.x;                           // empty slots hold key 0, below every score
      cid[t] = (int32_t)e.y;
    }
  } else {
    constexpr int KB = 8;                       // candidates per thread and round (GT > 0)
    constexpr int GB = GT > 0 ? GT : 1;
    float xb[GB][KB];
    auto load_round = [&](int base) {
#pragma unroll
      for (int r = 0; r < GB; ++r) {
        const float* sr = scores + hrow(r) * nmax + c0;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int c = base + u * SEL_NT + tid;
          xb[r][u] = (c < cnt) ? sr[c] : -INFINITY;
        }
      }
    };
    if (GT > 0) load_round(0);
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
    if constexpr (GT > 0) {
      for (int base = 0; base < cnt; base += KB * SEL_NT) {
        if (base > 0) load_round(base);
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          float gs = -INFINITY;
#pragma unroll
          for (int r = 0; r < GB; ++r) gs = fmaxf(gs, xb[r][u] - ((GT == 1) ? 0.0f : Lh[r]));
          const int c = base + u * SEL_NT + tid;
          if (c < cnt) ky[c] = f32_order_key(gs);
        }
      }
    } else {
    constexpr int KU = 4;
    for (int base = 0; base < cnt; base += KU * SEL_NT) {
      float gs[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) gs[u] = -INFINITY;
      for (int r = 0; r < G; ++r) {
        const float* sr = scores + hrow(r) * nmax + c0;
        const float lr = (G == 1) ? 0.0f : Lh[r];
        float x[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const int c = base + u * SEL_NT + tid;
          x[u] = (c < cnt) ? sr[c] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) gs[u] = fmaxf(gs[u], x[u] - lr);
      }
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int c = base + u * SEL_NT + tid;
        if (c < cnt) ky[c] = f32_order_key(gs[u]);
      }
    }
    }
  }
  if (tid == 0) sh_need = kl;

  // Bound and short path (partitioned selections: a whole-row selection
  // measured faster with the radix passes, its bound over few blocks admitting
  // too many keys).  Each scoring workgroup's partial holds, per head,
  // the largest score m of its block of SC_CPB chunks (a stored score), so the
  // chunk attaining it has group score >= m - L_h, by the same fp32
  // subtraction as the keys.  The blocks are disjoint: when at least kk of
  // them have a finite bound B_t = max_h (m_h,t - L_h), at least kk distinct
  // chunks reach the kk-th largest bound T, so every chunk of the row's top kk
  // (and of any partition's share of it) has a key >= key(T).  When at most
  // FCAP keys reach the bound they are ranked directly (rank = keys above, or
  // equal at a lower position), which takes the place of the radix passes and
  // the compaction.  Merge slots with key 0 are empty.
  constexpr int FCAP = SEL_NT;
  float* bnd = reinterpret_cast<float*>(hist);               // [nsb] block bounds
  uint32_t* fk = hist + SEL_NT;                              // [FCAP] candidate keys
  int* fp = reinterpret_cast<int*>(hist + SEL_NT + FCAP);    // [FCAP] their positions
  if (tid == 0) sh_tkey = (PH == SEL_MERGE) ? 1u : 0u;
  if (PH == SEL_PART && nsb <= SEL_NT) {
    if (tid < nsb) {
      float bt = -INFINITY;
      for (int r = 0; r < G; ++r)
        bt = fmaxf(bt, lsep[(hrow(r) * nsb + tid) * 2] - ((G == 1) ? 0.0f : Lh[r]));
      bnd[tid] = bt;
    }
    __syncthreads();
    if (tid < nsb) {
      const float v = bnd[tid];
      int rank = 0;
      for (int u = 0; u < nsb; ++u) {
        const float x = bnd[u];
        rank += (x > v || (x == v && u < tid)) ? 1 : 0;
      }
      if (v != -INFINITY && rank == kk - 1) sh_tkey = f32_order_key(v);
    }
  }
  __syncthreads();
  if (PH != SEL_WHOLE) {
    const uint32_t tkey = sh_tkey;
    constexpr int CPT = 8;
    int total = 0;
    bool fast = true;
    for (int base = 0; base < cnt; base += CPT * SEL_NT) {
      const int q0 = base + CPT * tid;
      uint32_t kv[CPT];
      int nin = 0;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        kv[u] = (q0 + u < cnt) ? ky[q0 + u] : 0u;
        nin += (q0 + u < cnt && kv[u] >= tkey && kv[u] != 0u) ? 1 : 0;
      }
      int inc = nin;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      if (lane == 63) wsum[wv] = inc;
      __syncthreads();
      int before = inc - nin, rt = 0;
      for (int u = 0; u < SEL_NW; ++u) {
        const int t = wsum[u];
        if (u < wv) before += t;
        rt += t;
      }
      __syncthreads();                     // wsum is rewritten next round
      if (total + rt > FCAP) { fast = false; break; }   // uniform
      int pos = total + before;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        if (q0 + u < cnt && kv[u] >= tkey && kv[u] != 0u) {
          fk[pos] = kv[u];
          fp[pos] = q0 + u;
          ++pos;
        }
      }
      total += rt;
    }
    if (fast) {
      if (tid < 3 && total + tid < FCAP) fk[total + tid] = 0u;   // pad to a multiple of 4
      __syncthreads();                     // candidates written
      const int C = total, want = min(kl, C);
      bool take = false;
      uint32_t kj = 0u;
      int pj = 0;
      if (tid < C) {
        kj = fk[tid];
        pj = fp[tid];
        // candidates are in position order; keys past C read as 0 (below every
        // candidate), four per LDS read
        int rank = 0;
        for (int u = 0; u < C; u += 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(fk + u);
          rank += (x.x > kj || (x.x == kj && u < tid)) ? 1 : 0;
          rank += (x.y > kj || (x.y == kj && u + 1 < tid)) ? 1 : 0;
          rank += (x.z > kj || (x.z == kj && u + 2 < tid)) ? 1 : 0;
          rank += (x.w > kj || (x.w == kj && u + 3 < tid)) ? 1 : 0;
        }
        take = rank < want;
      }
      // output slot: selected candidates before this one, i.e. ascending position
      const uint64_t bal = __ballot(take);
      if (lane == 0) wsum[wv] = __popcll(bal);
      __syncthreads();
      int pos = __popcll(bal & ((1ull << lane) - 1ull));
      for (int u = 0; u < wv; ++u) pos += wsum[u];
      if (take) {
        if (PH == SEL_PART) {
          co[pos] = make_uint2(kj, (uint32_t)(c0 + pj));
        } else {
          const int c = (PH == SEL_MERGE) ? cid[pj] : pj;
          so[pos] = c;
          for (int r = 0; r < G; ++r) slog[hrow(r) * K + pos] = scores[hrow(r) * nmax + c];
        }
      }
      if (PH == SEL_PART)
        for (int t = want + tid; t < kl; t += SEL_NT) co[t] = make_uint2(0u, 0xffffffffu);
      return;
    }
  }
  __syncthreads();

  // MSD radix select of the kl-th largest 32-bit key
  uint32_t prefix = 0, pmask = 0;
  const uint32_t rep = (uint32_t)lane & (SEL_REP - 1);
  for (int p = 3; p >= 0; --p) {
    for (int t = tid; t < 64 * SEL_REP; t += SEL_NT)
      reinterpret_cast<uint4*>(hist)[t] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    for (int c = tid; c < cnt; c += SEL_NT) {
      const uint32_t key = ky[c];
      if ((key & pmask) == prefix) atomicAdd(&hist[((key >> (8 * p)) & 255u) * SEL_REP + rep], 1u);
    }
    __syncthreads();
    if (tid < 256) {           // bin tid's total over the copies, starting at a
      uint32_t tot = 0;        // rotated copy so that a wave's reads spread over the banks
#pragma unroll
      for (int j = 0; j < SEL_REP; ++j) tot += hist[tid * SEL_REP + ((j + tid) & (SEL_REP - 1))];
      htot[tid] = tot;
    }
    __syncthreads();
    if (tid < 64) {            // one wave: suffix sums over 256 bins, 4 per lane
      uint32_t h4[4], s4 = 0;
#pragma unroll
      for (int u = 3; u >= 0; --u) { s4 += htot[tid * 4 + u]; h4[u] = s4; }
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
  const int need_eq = sh_need;   // how many keys equal to thr to take (lowest positions)

  // compaction in ascending position order: thread t owns positions [8t, 8t + 8)
  // of each round of 8 * SEL_NT; one block scan of its (greater, equal) counts
  // gives where its selected entries go.  Keys equal to thr are taken lowest
  // position (= lowest chunk id) first, need_eq of them.
  constexpr int CPT = 8;
  int taken_all = 0, eq_all = 0;
  for (int base = 0; base < cnt; base += CPT * SEL_NT) {
    const int q0 = base + CPT * tid;
    uint32_t kv[CPT];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      kv[u] = (q0 + u < cnt) ? ky[q0 + u] : 0u;
      const bool in = q0 + u < cnt;
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
      const int t = q0 + u;
      if (t < cnt) {
        bool take = kv[u] > thr;
        if (kv[u] == thr) take = eqi++ < need_eq;
        if (take) {
          if (PH == SEL_PART) {
            co[pos] = make_uint2(kv[u], (uint32_t)(c0 + t));
          } else {
            const int c = (PH == SEL_MERGE) ? cid[t] : t;
            so[pos] = c;
            for (int r = 0; r < G; ++r) slog[hrow(r) * K + pos] = scores[hrow(r) * nmax + c];
          }
          ++pos;
        }
      }
    }
    const int gt_tot = (int)(total & 0xffffu), eq_tot = (int)(total >> 16);
    taken_all += gt_tot + min(eq_all + eq_tot, need_eq) - min(eq_all, need_eq);
    eq_all += eq_tot;
  }
}

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

// Split attention on the matrix cores for bf16, d = 128, S = 64 (same
// partials as k_dec_attn): up to 16 query rows (the G heads of a query, or the
// heads of several tokens of a block) against one S-token tile, as
// S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_16x16x32_bf16 (lane l, i =
// l % 16, g = l / 16: A operand A[i][8g..8g+7], B operand B[8g..8g+7][i],
// result D[4g + r][i]).  Wave w scores 16 keys: A-operand row i stands for key
// kperm(w, i) = 32 (w / 2) + 8 (i / 4) + 4 (w % 2) + i % 4, so that the four
// waves' results put keys 32 kb + 8g .. 32 kb + 8g + 7 of every row in lane
// group g, which is the B operand of O^T's k-block kb as stored.  V^T is
// staged in LDS (the cache holds V row-major); wave w forms output elements
// 32w .. 32w + 31.  Softmax statistics meet in LDS (two barriers).
constexpr int VTS = DA_S + 4;   // V^T row stride (bf16): 8-byte aligned rows, banks spread
constexpr int PTS = DA_S + 8;   // P row stride (bf16): 16-byte aligned rows

struct MfLds {
  uint16_t vt[DA_D][VTS];       // V^T of the tile, zero past its valid keys
  uint16_t pt[16][PTS];         // P (row = query row), bf16
  float mx[4][16], sm[4][16];   // per-wave row maxima and exp sums
};

__device__ __forceinline__ int kperm(int w, int i) {
  return 32 * (w >> 1) + 8 * (i >> 2) + 4 * (w & 1) + (i & 3);
}

// this wave's K A operand (keys kperm(w, i), rows past jmax - 1 read row jmax - 1)
__device__ __forceinline__ void mf_load_k(const bf16_t* __restrict__ kg, int jmax, uint4 (&ka)[4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int key = min(kperm(w, lane & 15), jmax - 1);
  const bf16_t* kr = kg + (long long)key * DA_D + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka[ks] = *reinterpret_cast<const uint4*>(kr + 32 * ks);
}

// V tile (jmax valid rows) into L.vt, transposed; rows past jmax are zero and
// are not read.  Lane (e8 = l % 16, kq = l / 16) of wave w loads keys
// 16 w + 4 kq + u, elements 8 e8 .. 8 e8 + 7 (whole rows per instruction).
__device__ __forceinline__ void mf_stage_v(MfLds& L, const bf16_t* __restrict__ vg, int jmax) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e8 = lane & 15, kq = lane >> 4;
  uint4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int key = 16 * w + 4 * kq + u;
    x[u] = (key < jmax) ? *reinterpret_cast<const uint4*>(vg + (long long)key * DA_D + 8 * e8)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int key = 16 * w + 4 * kq + u;
    const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      L.vt[8 * e8 + 2 * t][key] = (uint16_t)(wd[t] & 0xffffu);
      L.vt[8 * e8 + 2 * t + 1][key] = (uint16_t)(wd[t] >> 16);
    }
  }
}

// the empty partial (weight 0) of split s for rows hrow0 + r * hstep
template <int G>
__device__ __forceinline__ void split_empty(float* __restrict__ part, long long hrow0, int hstep, int NS, int s) {
  for (int t = threadIdx.x; t < G * (DA_D + 2); t += AT_NT) {
    const int r = t / (DA_D + 2), e = t - r * (DA_D + 2);
    part[((hrow0 + (long long)r * hstep) * NS + s) * (long long)(DA_D + 2) + e] = (e == 0) ? -INFINITY : 0.0f;
  }
}

// One pass over up to 16 rows; every thread calls it with the data of row
// j = lane % 16: its query's B operand (mf_load_q), ok (row exists), hrow (its
// partial row), slot (its split) and jn (its valid keys, >= 1).  L.vt must hold the tile (a
// barrier after staging); a pass after the first (first = false) waits for
// the previous pass's LDS readers.
__device__ __forceinline__ void mf_load_q(const bf16_t* __restrict__ q, bool ok, long long hrow, bf16x8_t (&qb)[4]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qb[ks] = ok ? ld_bf16x8(q + hrow * DA_D + 32 * ks + 8 * g)
                : __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
}

__device__ __forceinline__ void mf_rows(MfLds& L, const bf16x8_t (&qb)[4], float* __restrict__ part,
                                        int NS, float tau2, const uint4 (&ka)[4], bool ok,
                                        long long hrow, int slot, int jn, bool first) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) sc = mfma16(__builtin_bit_cast(bf16x8_t, ka[ks]), qb[ks], sc);
  // sc[r]: row j, key kb0 + r (base-2 logits after scaling)
  const int kb0 = 32 * (w >> 1) + 8 * g + 4 * (w & 1);
  float x[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = (kb0 + r < jn) ? sc[r] * tau2 : -INFINITY;
    mloc = fmaxf(mloc, x[r]);
  }
  mloc = max_x32(max_x16(mloc));
  if (!first) __syncthreads();                   // the previous pass's readers
  if (g == 0) L.mx[w][j] = mloc;
  __syncthreads();                                // mx
  const float Mj = fmaxf(fmaxf(L.mx[0][j], L.mx[1][j]), fmaxf(L.mx[2][j], L.mx[3][j]));
  float p[4];
  float ps = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = (x[r] == -INFINITY) ? 0.0f : fast_exp2(x[r] - Mj);
    ps += p[r];
  }
  ps = sum_x32(sum_x16(ps));
  if (g == 0) L.sm[w][j] = ps;
  *reinterpret_cast<uint2*>(&L.pt[j][kb0]) = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  __syncthreads();                                // pt, sm
  bf16x8_t pb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) pb[kb] = ld_bf16x8(reinterpret_cast<const bf16_t*>(&L.pt[j][32 * kb + 8 * g]));
  float* pp = part + (hrow * NS + slot) * (long long)(DA_D + 2);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int dt = 2 * w + h2;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t* vr = &L.vt[16 * dt + j][32 * kb + 8 * g];
      const uint2 lo = *reinterpret_cast<const uint2*>(vr);
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 4);
      o = mfma16(__builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[kb], o);
    }
    // o[r] = O^T[16 dt + 4g + r][row j], unnormalised
    if (ok) {
      *reinterpret_cast<float2*>(pp + 2 + 16 * dt + 4 * g) = make_float2(o[0], o[1]);
      *reinterpret_cast<float2*>(pp + 2 + 16 * dt + 4 * g + 2) = make_float2(o[2], o[3]);
    }
  }
  if (ok && w == 0 && g == 0) {
    pp[0] = Mj * LN2;                             // natural-log units, as the combine takes them
    pp[1] = (L.sm[0][j] + L.sm[1][j]) + (L.sm[2][j] + L.sm[3][j]);
  }
}

// split s of query row bgm = (sequence, KV group, query), by a workgroup of
// AT_NT threads
template <bool PAGED, int G>
__device__ __forceinline__ void dec_split_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                               const bf16_t* __restrict__ v, const int32_t* __restrict__ seqlen,
                                               const int32_t* __restrict__ sel, float* __restrict__ part,
                                               int Hq, int Hkv, int N, int W, int K, int NS, float tau,
                                               int M, PageMap pm, int bgm, int s) {
  constexpr int D = DA_D, S = DA_S;
  __shared__ __align__(16) MfLds L;
  const int m = bgm % M, bg = bgm / M;
  const int b = bg / Hkv, g = bg % Hkv;
  const long long hrow0 = ((long long)b * Hq + (long long)g * G) * M + m;   // row r: hrow0 + r M
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
    split_empty<G>(part, hrow0, M, NS, s);
    return;
  }
  const long long kvoff = PAGED ? (pm.page(b, j0 / S) * Hkv + g) * (long long)S * D
                                : ((b * (long long)Hkv + g) * N + j0) * D;
  const int r = threadIdx.x & 15;
  const long long hrow = hrow0 + (long long)min(r, G - 1) * M;
  bf16x8_t qb[4];
  mf_load_q(q, r < G, hrow, qb);
  uint4 ka[4];
  mf_load_k(k + kvoff, jn, ka);
  mf_stage_v(L, v + kvoff, jn);
  __syncthreads();                                // vt
  mf_rows(L, qb, part, NS, tau * LOG2E, ka, r < G, hrow, s, jn, true);
}

// grid (sequence x KV group x query, split)
template <bool PAGED, int G>
__global__ void __launch_bounds__(AT_NT)
k_dec_attn_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const int32_t* __restrict__ seqlen,
                const int32_t* __restrict__ sel, float* __restrict__ part, int Hq, int Hkv, int N,
                int W, int K, int NS, float tau, int M, PageMap pm) {
  dec_split_bf16<PAGED, G>(q, k, v, seqlen, sel, part, Hq, Hkv, N, W, K, NS, tau, M, pm,
                           (int)blockIdx.x, (int)blockIdx.y);
}

// Multi-token blocks (M > 1), bf16, d = 128, S = 64: the block's tokens share
// most of their window tiles and, when their queries are alike, many selected
// chunks (section 4.2: a query block loads the union of its chunks once;
// section 7.2: chunk overlap of adjacent queries).  One workgroup per
// (sequence, KV group, union element) loads a tile once and attends it for
// every token of the block that uses it, writing the same split partials as
// the per-token kernel (the combine is unchanged):
//   y < M K:  the y-th smallest distinct chunk id of the block's M selections
//             (k_dec_union lists them; workgroups past the union's size have
//             none), for each token that selected it at its own slot; the
//             workgroup also writes the empty partial of slot (y / K, y % K)
//             when that token selected fewer chunks;
//   y >= M K: window tile ws_0 / S + (y - M K), ws_0 = the first token's window
//             start, for each token whose window holds it (tokens differ only
//             in where their windows start and end); the workgroup also writes
//             the empty partial of window slot y - M K of tokens whose
//             windows span fewer tiles.
constexpr int UN_IDS = HILS_DEC_UNION_IDS;       // M K ids held in LDS
constexpr int UN_WORDS = HILS_DEC_UNION_CHUNKS / 32;   // bitmap words over chunk ids

__device__ __forceinline__ int lower_bound_i32(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Per (sequence, KV group) of a multi-token block: the union of the tokens'
// selections in ascending chunk order (a bitmap over chunk ids, then one block
// scan of its set-bit counts) and each token's slot of every union element.
// Layout of `uni`: per (sequence, KV group) the union's size and its M K ids;
// then per (sequence, KV group, union element, token) one signed byte.
__global__ void __launch_bounds__(AT_NT)
k_dec_union(const int32_t* __restrict__ sel, const int32_t* __restrict__ seqlen, int32_t* __restrict__ uni,
            int Hkv, int N, int W, int S, int K, int M, int nC) {
  __shared__ uint32_t bits[UN_WORDS];
  __shared__ int ids[UN_IDS], uu[UN_IDS];
  __shared__ int wtot[AT_NT / 64];
  __shared__ int kkm[HILS_MAX_DECODE_QUERIES];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x, nbg = gridDim.x, b = bg / Hkv;
  const int mk = M * K;
  int32_t* ub = uni + (long long)bg * (mk + 1);
  int8_t* us = reinterpret_cast<int8_t*>(uni + (long long)nbg * (mk + 1)) + (long long)bg * mk * M;
  const int nw = (nC + 31) >> 5;
  for (int t = tid; t < nw; t += AT_NT) bits[t] = 0u;
  if (tid < M) kkm[tid] = min(K, n_cand(dec_pos(seqlen[b], N, M, tid), W, S));
  __syncthreads();
  for (int e = tid; e < mk; e += AT_NT) {
    const int m = e / K, kx = e - m * K;
    const int c = (kx < kkm[m]) ? sel[((long long)bg * M + m) * K + kx] : -1;
    ids[e] = c;
    if (c >= 0 && c < nC) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // each thread takes a contiguous run of words; its set bits go to the union
  // after those of the runs before it
  const int per = (nw + AT_NT - 1) / AT_NT;
  const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  for (int t = w0; t < w1; ++t) cnt += __popc(bits[t]);
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(inc, o, 64);
    if (lane >= o) inc += up;
  }
  if (lane == 63) wtot[wv] = inc;
  __syncthreads();
  int pos = inc - cnt, total = 0;
  for (int u = 0; u < AT_NT / 64; ++u) {
    if (u < wv) pos += wtot[u];
    total += wtot[u];
  }
  for (int t = w0; t < w1; ++t) {
    uint32_t x = bits[t];
    while (x) {
      const int c = t * 32 + __ffs(x) - 1;
      uu[pos] = c;
      ub[1 + pos] = c;
      ++pos;
      x &= x - 1u;
    }
  }
  if (tid == 0) ub[0] = total;
  for (int e = total + tid; e < mk; e += AT_NT) ub[1 + e] = -1;   // no chunk past the union
  __syncthreads();
  for (int e = tid; e < total * M; e += AT_NT) {
    const int u = e / M, m = e - u * M;
    const int c = uu[u], n = kkm[m];
    const int p = lower_bound_i32(ids + m * K, n, c);
    us[e] = (int8_t)((p < n && ids[m * K + p] == c) ? p : -1);
  }
}

template <bool PAGED, int G>
__global__ void __launch_bounds__(AT_NT)
k_dec_attn_union(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, const int32_t* __restrict__ seqlen,
                 const int32_t* __restrict__ uni, float* __restrict__ part, int Hq, int Hkv, int N,
                 int W, int K, int NS, int nwin, float tau, int M, PageMap pm) {
  constexpr int D = DA_D, S = DA_S;
  __shared__ __align__(16) MfLds L;
  __shared__ int tsl[HILS_MAX_DECODE_QUERIES], tjn[HILS_MAX_DECODE_QUERIES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int bg = blockIdx.x, y = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const long long hbase = ((long long)b * Hq + (long long)g * G) * M;   // row (r, m): hbase + r M + m
  const int mk = M * K;
  const int sl = seqlen[b];
  long long j0;
  int jmax;
  if (y < mk) {
    // the chunk (-1 past the union) and, by thread m < M, token m's slot of
    // it: neither depends on the other, so both loads go out together
    const int c = uni[(long long)bg * (mk + 1) + 1 + y];
    const int8_t* us = reinterpret_cast<const int8_t*>(uni + (long long)gridDim.x * (mk + 1)) +
                       ((long long)bg * mk + y) * M;
    const int myslot = (tid < M) ? (int)us[tid] : -1;
    const int mu = y / K, su = y - mu * K;
    if (su >= min(K, n_cand(dec_pos(sl, N, M, mu), W, S))) split_empty<G>(part, hbase + mu, M, NS, su);
    if (c < 0) return;
    j0 = (long long)c * S;
    jmax = S;
    if (tid < M) { tsl[tid] = myslot; tjn[tid] = S; }
  } else {
    const int vt = y - mk;
    const long long i0 = dec_pos(sl, N, M, 0), iM = dec_pos(sl, N, M, M - 1);
    j0 = window_start(i0, W, S) + (long long)vt * S;   // tile start
    for (int m = 0; m < M; ++m) {                // window slots past a token's tiles
      const long long im = dec_pos(sl, N, M, m);
      const int cntm = (int)(im / S - window_start(im, W, S) / S) + 1;
      if (vt < nwin && vt >= cntm) split_empty<G>(part, hbase + m, M, NS, K + vt);
    }
    if (j0 > iM) return;
    jmax = (int)min((long long)S, iM - j0 + 1);
    if (tid < M) {                               // tokens whose windows hold the tile
      const long long im = dec_pos(sl, N, M, tid);
      const long long wsm = window_start(im, W, S);
      const bool in = j0 >= wsm && j0 <= im;
      tsl[tid] = in ? K + (int)((j0 - wsm) / S) : -1;
      tjn[tid] = in ? (int)min((long long)S, im - j0 + 1) : 0;
    }
  }
  const long long kvoff = PAGED ? (pm.page(b, j0 / S) * Hkv + g) * (long long)S * D
                                : ((b * (long long)Hkv + g) * N + j0) * D;
  uint4 ka[4];
  mf_load_k(k + kvoff, jmax, ka);
  mf_stage_v(L, v + kvoff, jmax);
  __syncthreads();                                // vt, tsl, tjn
  // rows (n-th token using the tile, head r) in passes of 16: row idx = G n + r
  int ntok = 0;
  for (int m = 0; m < M; ++m) ntok += (tsl[m] >= 0) ? 1 : 0;
  const int nrow = G * ntok;
  const float tau2 = tau * LOG2E;
  for (int base = 0; base < nrow; base += 16) {
    const int idx = base + (lane & 15);
    const bool ok = idx < nrow;
    const int n = ok ? idx / G : 0, r = ok ? idx % G : 0;
    int m = 0;
    for (int seen = -1; m < M; ++m) {            // the n-th token with a slot
      seen += (tsl[m] >= 0) ? 1 : 0;
      if (seen == n) break;
    }
    m = min(m, M - 1);
    const long long hrow = hbase + (long long)r * M + m;
    bf16x8_t qb[4];
    mf_load_q(q, ok, hrow, qb);
    mf_rows(L, qb, part, NS, tau2, ka, ok, hrow, tsl[m], tjn[m], base == 0);
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

template <typename T, bool PAGED, int MT, int WG = 0>
void launch_score(const HilsShape& s, const void* qr, const int32_t* seqlen, const void* ksum,
                  const float* bsum, float* scores, float* lsep, unsigned nsb, PageMap pm,
                  hipStream_t st, WinArgs wa = WinArgs{}) {
  const unsigned nz = (unsigned)((s.M + MT - 1) / MT);
  const unsigned nwx = WG > 0 ? (unsigned)((wa.nwin + WG - 1) / WG) : 0u;
  { HilsProfScope ps_("k_dec_score", st);
    hipLaunchKernelGGL((k_dec_score<T, PAGED, MT, WG>), dim3(nsb + nwx, s.B * s.Hq, nz), dim3(256), 0, st,
                       (const T*)qr, (const T*)ksum, bsum, seqlen, scores, lsep, s.Hq, s.nC, s.nmax,
                       (int)nsb, s.N, s.d, s.S, s.W, (float)s.tau, s.M, pm, wa); }
}

template <typename T, bool PAGED>
void launch_decode_t(const HilsShape& s, const void* q, const void* qr, const void* k, const void* v,
                     const int32_t* seqlen, const void* ksum, const float* bsum, void* out,
                     int32_t* sel, float* scores, uint32_t* keys, uint2* cand, int32_t* uni,
                     float* slog, float* part, float* lsep, PageMap pm, hipStream_t st) {
  const int NS = s.K + s.nwin;
  const float tau = (float)s.tau;
  const unsigned nsb = (unsigned)((s.nmax + SC_CPB - 1) / SC_CPB);
  const size_t esz = sizeof(T);
  const size_t ashm = 2 * (size_t)s.S * (s.d + 16 / esz) * esz + (size_t)s.G * s.d * 4 +
                      (size_t)s.G * ((s.S + 3) & ~3) * 4;
  const size_t cshm = (size_t)NS * 4;
  const bool fast_bf16 = std::is_same<T, bf16_t>::value && s.d == DA_D && s.S == DA_S &&
                         (s.G == 1 || s.G == 2 || s.G == 4);
  // single-token bf16 steps take their window splits inside the scoring launch
  const bool win_in_score = fast_bf16 && s.M == 1;
  if (win_in_score) {
    if constexpr (std::is_same<T, bf16_t>::value) {
      const WinArgs wa{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, part, s.Hkv, s.K, NS, s.nwin};
      if (s.G == 1) launch_score<T, PAGED, 1, 1>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st, wa);
      else if (s.G == 2) launch_score<T, PAGED, 1, 2>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st, wa);
      else launch_score<T, PAGED, 1, 4>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st, wa);
    }
  } else if (nsb > 0) {
    if (s.M == 1) launch_score<T, PAGED, 1>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
    else if (s.M == 2) launch_score<T, PAGED, 2>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
    else launch_score<T, PAGED, 4>(s, qr, seqlen, ksum, bsum, scores, lsep, nsb, pm, st);
  }
  int P = 1, span = 1;
  hils_dec_select_split(s, P, span);
  const int nm = s.nmax > 0 ? s.nmax : 1;
  const unsigned rows = (unsigned)(s.B * s.Hkv * s.M);
  auto select = [&](auto ph, dim3 grid, size_t shm, int sp) {
    constexpr int PH = decltype(ph)::value;
    auto launch = [&](auto kern) {
      hils_allow_lds((const void*)kern, shm);
      hipLaunchKernelGGL(kern, grid, dim3(SEL_NT), shm, st, scores, lsep, seqlen, keys, cand, sel, slog,
                         s.Hq, s.Hkv, s.G, nm, (int)nsb, s.N, s.S, s.W, s.K, s.M, sp, P);
    };
    if (s.G == 1) launch(k_dec_select<PH, 1>);
    else if (s.G == 2) launch(k_dec_select<PH, 2>);
    else if (s.G == 4) launch(k_dec_select<PH, 4>);
    else if (s.G == 8) launch(k_dec_select<PH, 8>);
    else launch(k_dec_select<PH, 0>);
  };
  if (P == 1) {
    HilsProfScope ps_("k_dec_select", st);
    select(std::integral_constant<int, SEL_WHOLE>(), dim3(rows), (size_t)4 * (size_t)min(nm, SEL_LDS_KEYS), nm);
  } else {
    HilsProfScope ps_("k_dec_select", st);
    select(std::integral_constant<int, SEL_PART>(), dim3(rows, P), (size_t)4 * (size_t)min(span, SEL_LDS_KEYS),
           span);
    // keys and chunk ids of the P * K candidates
    select(std::integral_constant<int, SEL_MERGE>(), dim3(rows), (size_t)8 * (size_t)P * s.K, span);
  }
  const dim3 agrid(s.B * s.Hkv * s.M, win_in_score ? s.K : NS);
  if (hils_dec_union(s)) {
    if constexpr (std::is_same<T, bf16_t>::value) {
      { HilsProfScope ps_("k_dec_union", st);
        hipLaunchKernelGGL(k_dec_union, dim3(s.B * s.Hkv), dim3(AT_NT), 0, st, sel, seqlen, uni, s.Hkv, s.N,
                           s.W, s.S, s.K, s.M, s.nC); }
      const dim3 ugrid(s.B * s.Hkv, s.M * s.K + s.nwin + 1);
      const bf16_t* qb = (const bf16_t*)q;
      const bf16_t* kb = (const bf16_t*)k;
      const bf16_t* vb = (const bf16_t*)v;
      HilsProfScope ps_("k_dec_attn", st);
      if (s.G == 1)
        hipLaunchKernelGGL((k_dec_attn_union<PAGED, 1>), ugrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen,
                           uni, part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, s.nwin, tau, s.M, pm);
      else if (s.G == 2)
        hipLaunchKernelGGL((k_dec_attn_union<PAGED, 2>), ugrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen,
                           uni, part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, s.nwin, tau, s.M, pm);
      else
        hipLaunchKernelGGL((k_dec_attn_union<PAGED, 4>), ugrid, dim3(AT_NT), 0, st, qb, kb, vb, seqlen,
                           uni, part, s.Hq, s.Hkv, s.N, s.W, s.K, NS, s.nwin, tau, s.M, pm);
    }
  } else if (fast_bf16) {
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
    hils_allow_lds((const void*)k_dec_attn<T, PAGED>, ashm);
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
                              uint32_t* keys, uint2* cand, int32_t* uni, float* slog, float* part,
                              float* lsep, const int32_t* page_table, int max_pages, int num_pages,
                              hipStream_t st) {
  const PageMap pm{page_table, max_pages, num_pages};
  const bool paged = page_table != nullptr;
  if (s.dtype == 0) {
    if (paged) launch_decode_t<bf16_t, true>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, cand, uni, slog, part, lsep, pm, st);
    else launch_decode_t<bf16_t, false>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, cand, uni, slog, part, lsep, pm, st);
  } else {
    if (paged) launch_decode_t<float, true>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, cand, uni, slog, part, lsep, pm, st);
    else launch_decode_t<float, false>(s, q, qr, k, v, seqlen, ksum, bsum, out, sel, scores, keys, cand, uni, slog, part, lsep, pm, st);
  }
  return hipGetLastError();
}
