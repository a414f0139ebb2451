// Fast-path chunk scoring + exact top-K selection (bf16, d = 128, S = 64).
//
// "Hierarchical Sparse Attention Done Right", section 3 routing equation
// (s_hat = q_hat . k'_c / sqrt(d) + b'_c, top-K over the candidate chunks C_i)
// and section 4.1 (GQA: per-head log-softmax over C_i, maximum over the heads
// of a group, one shared top-K).
//
// One workgroup (4 wavefronts) owns QB = 128/G query positions of one
// (batch, KV group).  Each wavefront loads its head's k' tiles of 32 chunks,
// stored beforehand in MFMA fragment order, straight into registers and
// computes a 32-chunk x 32-query score tile with v_mfma_f32_32x32x16_bf16
// (A = k' rows, B = q_hat).  Scores are kept in
// base-2 units (scaled by log2 e), which preserves their order.
//   pass 0: per (query, head) online log-sum-exp over C_i (G > 1), and the three
//           largest scores seen in each of the lane's 16 register slots.  Per
//           slot and rank r, u = max_h (r-th best of head h - L_h) is reached by
//           the group scores of r + 1 distinct chunks of the slot; the K-th
//           largest u of a query (96 per query) is then a lower bound T on its
//           K-th best group score.
//   pass 1: group score g = max_h (s_h - L_h) (cross-head max through LDS);
//           chunks whose score reaches the query's current K-th best (initially
//           T; a float compare) go to an LDS staging list, which is merged into
//           the query's sorted top-K list (wavefront bitonic sort of the staged
//           keys and one bitonic merge) before a step whose keys would not fit.
// The MFMA accumulator starts at b'_c / scale, so scores come out in units of
// 1 / (scale log2 e) with the bias already added.
// Keys are 64-bit: (order-preserving bits of g) << 32 | (~chunk id), so ties
// rank the lower chunk id first and every key is unique.  The selected ids
// are written ascending, -1 padded.
#include <cfloat>
#include <type_traits>

#include "fast_common.h"
#include "hils_internal.h"

using namespace fastp;

namespace {

constexpr int CT = 32;         // chunks per tile
constexpr int TRK = 128;       // pass-0 tracked scores per (query, head): 32 slots x ranks 0-2 (rank 3 unused)
constexpr int XROW = CT;       // row of the cross-head exchange buffer (floats); its 16-byte
                               // pieces are XOR-swizzled by the row's low 3 bits
// k' in MFMA fragment order: per (query head, 32-chunk tile) FRAGS fragments of
// 64 lanes x 16 bytes.  Fragment ks < 8 holds the A operand of k-step ks
// (lane l: chunk 32t + l % 32, elements 16 ks + 8 (l / 32) .. + 7); fragment
// 8 holds b' / scale split into three bf16 terms (lanes 0-31, elements 0-2),
// which a 32x32x8 MFMA against a constant operand of ones adds exactly (the
// scoring kernel reads only those 8 bytes of lanes 0-31).
constexpr int FRAGS = 9;

// Workgroup geometry.  Every wavefront scores 32 queries of one head; a
// workgroup of NW = 4 wavefronts covers QB = 32 NW / G queries with all G
// heads (the heads of a query meet in the workgroup's LDS exchange).  Each
// wavefront loads its own k' fragments, so a larger workgroup would only
// lengthen the exchange barrier (8 wavefronts measured slower).
template <int G>
struct Geo {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;      // threads
  static constexpr int QB = 32 * NW / G;  // queries per workgroup
  static constexpr int QW = QB / NW;      // queries per wavefront in the selection layout
  static constexpr int LQ = 64 / QW;      // lanes per query
  static constexpr int CL = CT / LQ;      // chunks per lane per tile (selection layout)
  // staging slots per query.  One selection step adds at most LQ * CL = 32
  // keys to a query, which merges its staged keys first when they would not
  // fit; a merge takes at most 64.  G = 2 keeps 56 to fit one CU's LDS;
  // G = 1 keeps 56 so that two workgroups share a CU when K <= 16 (the
  // workgroup's 128 queries hold K list keys and STG staged keys each).
  static constexpr int STG = (G <= 2) ? 56 : 64;
  static_assert(LQ * CL <= STG && STG <= 64, "staging area");
  static_assert(QW % 8 == 0, "merge rounds take 8 queries");
};

// The tracked scores of pass 0 (G*QB (query, head) pairs x TRK floats) are
// written at offset 0 once the pass's loop is done; they cover the exchange
// buffers, the lists and possibly the staging area, idle then.  tq and
// everything after it start past them.
template <int G>
struct Lds {
  size_t xb, lst, stg, tq, thf, tk, cnt, total;
  __host__ __device__ Lds(int K) {
    size_t o = 0;
    xb = o;    o += (G > 1) ? (size_t)2 * G * Geo<G>::QB * XROW * 4 : 0;   // two buffers
    lst = o;   o += (size_t)Geo<G>::QB * K * 8;
    stg = o;   o += (size_t)Geo<G>::QB * Geo<G>::STG * 8;
    const size_t scratch = (size_t)G * Geo<G>::QB * TRK * 4;
    o = o > scratch ? o : scratch;
    tq = o;    o += (size_t)G * Geo<G>::QB * 4;
    thf = o;   o += (size_t)Geo<G>::QB * 4;
    // tk lives between the passes only: it may share the idle staging array
    // when that starts past the tracked-score scratch; otherwise it needs room
    // of its own
    if (stg >= scratch) {
      tk = stg;
    } else {
      tk = o;  o += (size_t)G * Geo<G>::QB * 4;
    }
    cnt = o;   o += (size_t)Geo<G>::QB * 4;
    total = o;
  }
};

typedef __attribute__((ext_vector_type(4))) short bf16x4_bits;
// 32x32x8 bf16 MFMA on raw bf16 bits (same output layout as 32x32x16)
__device__ __forceinline__ f32x16_t mfma32x8(uint2 a, uint2 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(bf16x4_bits, a),
                                                  __builtin_bit_cast(bf16x4_bits, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a > b ? b : a; }

// The 64 keys of one query held by its 8 lanes (lg = lane & 7) x 8
// registers: the key of rank 8 lg + r sits in register r.  In the bitonic
// networks below, strides 8, 16 and 32 pair lane lg with lane lg ^ 1, 2, 4 of
// the group (DPP); strides 1, 2 and 4 pair registers of one lane.
__device__ __forceinline__ uint64_t mirror8_u64(uint64_t v) {     // lane lg ^ 7 of the group
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, 0x141, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), 0x141, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// one stage (block size k, stride j) of the descending bitonic network
template <int k, int j>
__device__ __forceinline__ void bitonic_stage8(uint64_t (&v)[8], int lg) {
  if constexpr (j >= 8) {
    constexpr int ls = j / 8;
    const bool lower = (lg & ls) == 0;
    const bool desc = (k >= 64) || ((8 * lg) & k) == 0;
    const bool keepmax = lower == desc;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint64_t p = xshfl_u64(v[r], ls);
      v[r] = keepmax ? umax64(v[r], p) : umin64(v[r], p);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if ((r & j) == 0) {
        const bool desc = (k >= 64) || ((8 * lg + r) & k) == 0;
        const uint64_t hi = umax64(v[r], v[r | j]), lo = umin64(v[r], v[r | j]);
        v[r] = desc ? hi : lo;
        v[r | j] = desc ? lo : hi;
      }
    }
  }
}

template <int k, int j>
__device__ __forceinline__ void bitonic_block8(uint64_t (&v)[8], int lg) {
  bitonic_stage8<k, j>(v, lg);
  if constexpr (j > 1) bitonic_block8<k, j / 2>(v, lg);
}

template <int k>
__device__ __forceinline__ void bitonic_sort8(uint64_t (&v)[8], int lg) {
  if constexpr (k > 2) bitonic_sort8<k / 2>(v, lg);
  bitonic_block8<k, k / 2>(v, lg);
}

// sort the 64 keys of each 8-lane group descending
__device__ __forceinline__ void sort8x8_desc(uint64_t (&v)[8], int lg) { bitonic_sort8<64>(v, lg); }

// a, b descending -> a = the 64 largest of a U b, descending
__device__ __forceinline__ void merge8x8_top(uint64_t (&a)[8], const uint64_t (&b)[8], int lg) {
#pragma unroll
  for (int r = 0; r < 8; ++r) a[r] = umax64(a[r], mirror8_u64(b[7 - r]));   // b reversed
  bitonic_block8<64, 32>(a, lg);
}

// wavefront-wide bitonic sort of 64 floats (1 per lane), descending
__device__ __forceinline__ float sort64_desc_f(float v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float p = xshfl_f(v, stride);
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0 || size == 64;
      v = (lower == desc) ? fmaxf(v, p) : fminf(v, p);
    }
  }
  return v;
}

// a, b descending across the wavefront -> the 64 largest of a U b, descending
__device__ __forceinline__ float merge_top64_f(float a, float b, int lane) {
  float v = fmaxf(a, __builtin_bit_cast(float, lane_reverse(__builtin_bit_cast(uint32_t, b))));
#pragma unroll
  for (int stride = 32; stride > 0; stride >>= 1) {
    const float p = xshfl_f(v, stride);
    v = ((lane & stride) == 0) ? fmaxf(v, p) : fminf(v, p);
  }
  return v;
}

template <int G>
__global__ void __launch_bounds__(Geo<G>::NT, 2)
k_score_fast(const bf16_t* __restrict__ qr, const uint4* __restrict__ frag,
             int32_t* __restrict__ sel, int Hq, int Hkv, int N, int W, int K, int ntg, float tau2,
             int nqb) {
  using GE = Geo<G>;
  constexpr int QB = GE::QB, QW = GE::QW, LQ = GE::LQ, CL = GE::CL;
  constexpr int STG = GE::STG, NT = GE::NT, NW = GE::NW;
  extern __shared__ __align__(16) unsigned char sm[];
  const Lds<G> L(K);
  float* xb = reinterpret_cast<float*>(sm + L.xb);           // [2][G][QB][XROW]
  float* tq = reinterpret_cast<float*>(sm + L.tq);           // [G][QB] log-sum-exp (base 2)
  float* tk = reinterpret_cast<float*>(sm + L.tk);           // [QB] bound T of the query
  float* trk = reinterpret_cast<float*>(sm);                 // [G*QB][TRK] between the passes
  uint64_t* lst = reinterpret_cast<uint64_t*>(sm + L.lst);   // [QB][K]
  uint2* stg = reinterpret_cast<uint2*>(sm + L.stg);         // [QB][STG] (score bits, chunk id)
  uint32_t* cnt_lst = reinterpret_cast<uint32_t*>(sm + L.cnt);
  float* thf = reinterpret_cast<float*>(sm + L.thf);        // [QB] staging bound (K-th key's score)

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

  // selection layout: lane -> (query qsel, CL chunks of the tile); nstg is
  // that query's staged-key count, held by every lane of its group
  const int qsel = (G == 1) ? (32 * w + col) : (w * QW + lane / LQ);
  const int cbase = (G == 1) ? 0 : CL * (lane % LQ);
  int nstg = 0;

  // this wavefront's k' fragments: coalesced 16-byte loads straight into the
  // MFMA operand registers (no LDS staging, no barrier)
  const uint4* fh = frag + ((hb + hw) * (long long)ntg) * (FRAGS * 64) + lane;
  // The bias fragment's data are its first 8 bytes in lanes 0-31: only those
  // are read, and they enter a 32x32x8 MFMA (four k per lane: lanes 0-31 hold
  // k = 0-3, lanes 32-63 k = 4-7, zero).
  auto load_frag = [&](int t, uint4 (&f)[FRAGS]) {
    const uint4* p = fh + (long long)t * (FRAGS * 64);
#pragma unroll
    for (int ks = 0; ks < FRAGS - 1; ++ks) f[ks] = p[ks * 64];
    uint2 bb = make_uint2(0u, 0u);
    if (half == 0) bb = *reinterpret_cast<const uint2*>(p + (FRAGS - 1) * 64);
    f[FRAGS - 1] = make_uint4(bb.x, bb.y, 0u, 0u);
  };
  // B operand of the bias MFMA: ones at k = 0, 1, 2 (lanes 0-31)
  const uint32_t one2 = 0x3F803F80u;                  // two bf16 1.0
  const uint2 bones = half ? make_uint2(0u, 0u) : make_uint2(one2, one2 & 0xFFFFu);

  // merge the staged keys of every query of this wavefront into its sorted
  // top-K list: each query in one 8-lane group (QW / 8 rounds), keys of rank
  // 8 lg + r in register r.  Staged counts pass through cnt_lst (the staging
  // lane groups need not be the merge groups).  An empty list slot holds 0,
  // which is below every key.
  auto merge_wave = [&](int ns_mine, bool leader) __attribute__((always_inline)) {
    if (leader) cnt_lst[qsel] = (uint32_t)ns_mine;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int lg = lane & 7;
#pragma unroll 1
    for (int rd = 0; rd < QW / 8; ++rd) {
      const int q = w * QW + 8 * rd + (lane >> 3);
      const int ns = (int)cnt_lst[q];
      uint64_t a[8], b[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = 8 * lg + r;
        a[r] = (i < K) ? lst[(size_t)q * K + i] : 0ull;
        b[r] = 0ull;
        if (i < ns) {
          const uint2 e = stg[(size_t)q * STG + i];
          b[r] = ((uint64_t)f32_order_key(__uint_as_float(e.x)) << 32) | (uint64_t)(0xffffffffu - e.y);
        }
      }
      sort8x8_desc(b, lg);
      merge8x8_top(a, b, lg);
      uint64_t kth = 0ull;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = 8 * lg + r;
        if (i < K) lst[(size_t)q * K + i] = a[r];
        kth = (r == ((K - 1) & 7)) ? a[r] : kth;
      }
      // key of rank K - 1 (0 while the list holds fewer than K keys)
      const int src = (lane & ~7) | ((K - 1) >> 3);
      const uint32_t khi = (uint32_t)__shfl((int)(uint32_t)(kth >> 32), src, 64);
      const uint32_t klo = (uint32_t)__shfl((int)(uint32_t)kth, src, 64);
      if (lg == 0 && (khi | klo) != 0u) thf[q] = fmaxf(thf[q], order_key_f32(khi));
    }
    // the lanes read the lists and bounds next: acquire-release keeps the
    // compiler from answering those reads with values from before the writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };

  // scores of tile t for this lane in accumulator units (score = tau2 * x, base
  // 2): x[i] <-> chunk 32t + 8(i>>2) + 4*half + (i&3).  The last MFMA of the
  // chain (32x32x8) adds the bias b' / tau2 of each chunk.
  const int n_lo = n_cand(i0, W, S);                 // every query of the block has >= n_lo
  auto tile_scores = [&](const uint4 (&f)[FRAGS], int t, float* x, float a0) {
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = a0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32(__builtin_bit_cast(bf16x8_t, f[ks]), bq[ks], acc);
    acc = mfma32x8(make_uint2(f[8].x, f[8].y), bones, acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = acc[i];
    if (CT * t + CT > n_lo) {                        // tile crosses some query's candidate range
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cl = 8 * (i >> 2) + 4 * half + (i & 3);
        x[i] = (CT * t + cl < nq) ? x[i] : -INFINITY;
      }
    }
  };

  float L2 = 0.0f;
  // the two passes are separate instantiations, so pass 1 does not keep
  // pass 0's trackers live
  auto run_pass = [&](auto pass_tag) {
    constexpr int pass = decltype(pass_tag)::value;
    // One head (G = 1) needs no log-sum-exp, and with at most four tiles of
    // candidates staging every chunk costs at most two merges, less than the
    // bound: pass 0 is skipped and the staging bound is -inf.
    if (pass == 0 && G == 1 && ntiles <= 4) {
      for (int t = tid; t < QB * K; t += NT) lst[t] = 0ull;
      for (int t = tid; t < QB; t += NT) thf[t] = -INFINITY;
      __syncthreads();
      return;
    }
    float m = -INFINITY, ssum = 0.0f;
    float t0[16], t1[16], t2[16];  // top 3 per register slot, descending (pass 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) { t0[i] = -INFINITY; t1[i] = -INFINITY; t2[i] = -INFINITY; }
    uint4 fA[FRAGS], fB[FRAGS];
    load_frag(0, fA);
    // pass 1 subtracts the head's log-sum-exp (L = -inf only for rows without
    // candidates, whose scores are all masked)
    const float nL = (L2 > -INFINITY) ? -L2 : 0.0f;
    // pass 0 takes the tiles in pairs: every register slot's trackers absorb
    // the larger of the pair's two scores (one chunk's score, so a slot's
    // tracked entries still belong to distinct chunks), and the log-sum-exp
    // takes both tiles against one running maximum
    auto absorb2 = [&](const float* xa, const float* xc) __attribute__((always_inline)) {
      float hi[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        hi[i] = fmaxf(xa[i], xc[i]);
        // insert hi into t0 >= t1 >= t2: each new entry is the median of its
        // old neighbours above and below and hi
        t2[i] = __builtin_amdgcn_fmed3f(t1[i], t2[i], hi[i]);
        t1[i] = __builtin_amdgcn_fmed3f(t0[i], t1[i], hi[i]);
        t0[i] = fmaxf(t0[i], hi[i]);
      }
      if (G > 1) {
        // online log-sum-exp; m is the running maximum in accumulator units
        float mt = hi[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, hi[i]);
        if (mt > m) { ssum = (m == -INFINITY) ? 0.0f : ssum * fast_exp2((m - mt) * tau2); m = mt; }
        if (m != -INFINITY) {
          const float mneg = -m * tau2;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            ssum += fast_exp2(fmaf(xa[i], tau2, mneg)) + fast_exp2(fmaf(xc[i], tau2, mneg));
        }
      }
    };
    // pass 1 starts the accumulators at -L / tau2, so its scores come out as
    // (s_h - L_h) / tau2: group scores in accumulator units
    const float a1 = (pass == 1 && G > 1) ? nL / tau2 : 0.0f;
    // one tile step of pass 1: cur holds the fragments of tile t, nxt receives
    // tile t + 1 (past the last tile: the last again, unused)
    auto step = [&](int t, const uint4 (&cur)[FRAGS], uint4 (&nxt)[FRAGS]) {
      load_frag(min(t + 1, ntiles - 1), nxt);
      float x[16];
      tile_scores(cur, t, x, a1);
      if constexpr (pass == 0) {
      } else {
        // group scores (s_h - L_h) / tau2, in accumulator units, which order
        // the chunks as s_h - L_h does; the heads of a group meet in LDS, in
        // one of two exchange buffers by step parity (a wavefront writes
        // buffer t & 1 only after every wavefront passed the barrier of step
        // t - 1, so after their reads of step t - 2).  G = 1 exchanges nothing.
        float* xbt = xb + (size_t)(t & 1) * G * QB * XROW;
        if (G > 1) {
          const int xrow = hw * QB + 32 * qw + col;
          float* xr = xbt + (size_t)xrow * XROW;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<float4*>(xr + 4 * ((2 * gq + half) ^ (xrow & 7))) =
                make_float4(x[4 * gq], x[4 * gq + 1], x[4 * gq + 2], x[4 * gq + 3]);
        }
        if (G > 1) __syncthreads();                      // exchange written
        float gs[CL];
        int cid0;
        if (G > 1) {
#pragma unroll
          for (int j4 = 0; j4 < CL; j4 += 4) {
            const int piece = (cbase + j4) >> 2;
            float4 mx = *reinterpret_cast<const float4*>(xbt + (size_t)qsel * XROW + 4 * (piece ^ (qsel & 7)));
#pragma unroll
            for (int h = 1; h < G; ++h) {
              const int xrow = h * QB + qsel;
              const float4 y = *reinterpret_cast<const float4*>(xbt + (size_t)xrow * XROW + 4 * (piece ^ (xrow & 7)));
              mx = make_float4(fmaxf(mx.x, y.x), fmaxf(mx.y, y.y), fmaxf(mx.z, y.z), fmaxf(mx.w, y.w));
            }
            gs[j4] = mx.x; gs[j4 + 1] = mx.y; gs[j4 + 2] = mx.z; gs[j4 + 3] = mx.w;
          }
          cid0 = CT * t + cbase;
        } else {
#pragma unroll
          for (int i = 0; i < CL; ++i) gs[i] = x[i];
          cid0 = CT * t;
        }
        // filter: stage the chunks whose group score reaches the query's current
        // bound (a float compare: a chunk tied with the K-th key may be staged,
        // and the merge drops it).  Masked chunks (-inf) never pass.
        const float tf = fmaxf(thf[qsel], -FLT_MAX);
        bool pj[CL];
        int c = 0;
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          pj[j] = gs[j] >= tf;
          c += pj[j] ? 1 : 0;
        }
        // this lane's slots: prefix of c over the query's lane group (xor
        // butterfly: lane l ^ s holds the total of the sibling block), and the
        // group's total
        int incl = c, tot = c;
        if (G == 1) {
          const int p = (int)xshfl((uint32_t)tot, 32);
          incl += half ? p : 0;
          tot += p;
        } else {
#pragma unroll
          for (int sh = 1; sh < LQ; sh <<= 1) {
            const int p = (int)xshfl((uint32_t)tot, sh);
            incl += (lane & sh) ? p : 0;
            tot += p;
          }
        }
        // merge the queries whose staged keys and this step's would not fit
        const bool leader = (G == 1) ? (half == 0) : (lane % LQ == 0);
        if (__ballot(leader && nstg + tot > STG)) {   // some query's keys would not fit
          merge_wave(nstg, leader);
          nstg = 0;
        }
        if (c > 0) {
          uint2* sq = stg + (size_t)qsel * STG;
          int pos = nstg + incl - c;
#pragma unroll
          for (int j = 0; j < CL; ++j) {
            const int cid = (G == 1) ? (cid0 + 8 * (j >> 2) + 4 * half + (j & 3)) : (cid0 + j);
            if (pj[j]) {
              sq[pos] = make_uint2(__float_as_uint(gs[j]), (uint32_t)cid);
              ++pos;
            }
          }
        }
        nstg += tot;
      }
    };
    if constexpr (pass == 0) {
      for (int t = 0; t < ntiles; t += 2) {
        float xa[16], xc[16];
        load_frag(min(t + 1, ntiles - 1), fB);
        tile_scores(fA, t, xa, 0.0f);
        load_frag(min(t + 2, ntiles - 1), fA);
        // with ntiles odd, tile t + 1 = ntiles lies past every query's
        // candidates and tile_scores masks all its scores to -inf (one extra
        // MFMA chain per workgroup; a branch around it made the compiler set
        // sixteen -inf scores on every iteration)
        tile_scores(fB, t + 1, xc, 0.0f);
        absorb2(xa, xc);
      }
    } else {
      for (int t = 0; t < ntiles; t += 2) {
        step(t, fA, fB);
        if (t + 1 < ntiles) step(t + 1, fB, fA);
      }
    }
    if constexpr (pass == 0) {
      // per (query, head): log-sum-exp and the tracked scores, by slot and rank
      const int pr = hw * QB + 32 * qw + col;        // (head, query) pair of this lane
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float* tr = trk + (size_t)pr * TRK + half * 64 + i;
        tr[0] = t0[i];
        tr[16] = t1[i];
        tr[32] = t2[i];
        tr[48] = -INFINITY;
      }
      if (G > 1) {
        const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(ssum, 32, 64);
        const float M = fmaxf(m, m2);
        float s = 0.0f;
        if (M != -INFINITY)
          s = (m == -INFINITY ? 0.0f : ssum * fast_exp2((m - M) * tau2)) +
              (m2 == -INFINITY ? 0.0f : s2 * fast_exp2((m2 - M) * tau2));
        L2 = M * tau2 + log2f(s);
      }
      if (half == 0) tq[pr] = L2;
      __syncthreads();
      // bound T of a query: every head tracks, in each register slot (a fixed
      // set of chunk positions, the same for all heads), its three best scores,
      // which belong to three distinct chunks.  u(slot, r) = max_h (t_r,h - L_h)
      // is thus reached by the group scores of at least r + 1 distinct chunks of
      // the slot, and slots share no chunk: at least K distinct chunks reach the
      // K-th largest u of the query, which bounds its K-th best group score.
      for (int j = 0; j < QB / NW; ++j) {
        const int q = w * (QB / NW) + j;
        float ua = -INFINITY, ub = -INFINITY;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float* tr = trk + (size_t)(h * QB + q) * TRK;
          const float lh = tq[(size_t)h * QB + q];
          const float va = tr[lane], vb = tr[64 + lane];
          if (G > 1) {
            // a finite tracked score implies candidates, hence a finite L
            if (va != -INFINITY) ua = fmaxf(ua, va * tau2 - lh);
            if (vb != -INFINITY) ub = fmaxf(ub, vb * tau2 - lh);
          } else {
            ua = va;
            ub = vb;
          }
        }
        const float v = merge_top64_f(sort64_desc_f(ua, lane), sort64_desc_f(ub, lane), lane);
        const float kth = __shfl(v, K - 1, 64);
        if (lane == 0) tk[q] = kth;
      }
      __syncthreads();
      for (int t = tid; t < QB * K; t += NT) lst[t] = 0ull;   // pass-0 scratch read above
      for (int t = tid; t < QB; t += NT) {
        const float T = tk[t];
        // pass 1 accumulates s_h - L_h in accumulator units (scores / tau2),
        // which rounds differently from the product above: lower the bound by
        // a margin far above that rounding so no chunk at the bound is lost,
        // then convert it to those units
        const float Tm = (T == -INFINITY) ? -INFINITY : T - (1e-3f + 1e-6f * fabsf(T));
        thf[t] = (G > 1) ? Tm / tau2 : Tm;
      }
      __syncthreads();
    }
  };
  run_pass(std::integral_constant<int, 0>{});
  run_pass(std::integral_constant<int, 1>{});

  // final merge, then each query's ids ascending (sorting (1 << 32 | ~id)
  // descending; empty slots, 0, go last) and the selection row
  merge_wave(nstg, (G == 1) ? (half == 0) : (lane % LQ == 0));
  {
    const int lg = lane & 7;
#pragma unroll 1
    for (int rd = 0; rd < QW / 8; ++rd) {
      const int q = w * QW + 8 * rd + (lane >> 3);
      uint64_t x[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int i = 8 * lg + r;
        const uint64_t e = (i < K) ? lst[(size_t)q * K + i] : 0ull;
        x[r] = e ? ((1ull << 32) | (uint64_t)(uint32_t)e) : 0ull;
      }
      sort8x8_desc(x, lg);
      const int i = i0 + q;
      if (i < N) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int rank = 8 * lg + r;
          if (rank < K)
            selg[(long long)i * K + rank] = (x[r] >> 32) ? (int)(0xffffffffu - (uint32_t)x[r]) : -1;
        }
      }
    }
  }
}

// k' and b' of every (sequence, query head) in MFMA fragment order (FRAGS per
// 32-chunk tile); chunks past nC are zero.  One thread per 16-byte piece.
// The bias term b' / tau2 is split as hi + mid + lo with each term a bf16
// (the sum equals the fp32 value to within its last bit).
__global__ void __launch_bounds__(256)
k_score_frag(const bf16_t* __restrict__ ksum, const float* __restrict__ bsum, uint4* __restrict__ frag,
             int nC, int ntg, float bscale, long long total) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const long long fi = gid >> 6;
  const int ks = (int)(fi % FRAGS);
  const long long rt = fi / FRAGS;
  const int t = (int)(rt % ntg);
  const long long row = rt / ntg;                    // sequence * Hq + head
  const int c = CT * t + (lane & 31), half = lane >> 5;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (c < nC) {
    if (ks < 8) {
      v = *reinterpret_cast<const uint4*>(ksum + (row * nC + c) * (long long)D + 16 * ks + 8 * half);
    } else if (half == 0) {
      const float bv = bsum[row * nC + c] * bscale;
      const float hi = (float)(__bf16)bv;
      const float r1 = bv - hi;
      const float mid = (float)(__bf16)r1;
      const float lo = (float)(__bf16)(r1 - mid);
      v.x = pack_bf16x2(hi, mid);
      v.y = pack_bf16x2(lo, 0.0f);
    }
  }
  frag[gid] = v;
}

template <int G>
hipError_t launch_score(const HilsShape& s, const void* qr, const uint4* frag, int ntg, int32_t* sel,
                        hipStream_t st) {
  const int QB = Geo<G>::QB, NT = Geo<G>::NT;
  const int nqb = (s.N + QB - 1) / QB;
  const Lds<G> L(s.K);
  auto f = k_score_fast<G>;
  hils_allow_lds((const void*)f, L.total);
  const float tau2 = (float)(s.tau * 1.4426950408889634);
  { HilsProfScope ps_("k_score_fast", st); hipLaunchKernelGGL(f, dim3((unsigned)((long long)s.B * s.Hkv * nqb)), dim3(NT), L.total, st,
                     (const bf16_t*)qr, frag, sel, s.Hq, s.Hkv, s.N, s.W, s.K, ntg, tau2, nqb); }
  return hipGetLastError();
}

int frag_tiles(const HilsShape& s) { return (s.nC + CT - 1) / CT; }

}  // namespace

size_t hils_fast_score_lds(int G, int K) {
  switch (G) {
    case 1: return Lds<1>(K).total;
    case 2: return Lds<2>(K).total;
    case 4: return Lds<4>(K).total;
  }
  return 0;
}

size_t hils_score_frag_bytes(const HilsShape& s) {
  return (size_t)s.B * s.Hq * frag_tiles(s) * FRAGS * 64 * 16;
}

hipError_t hils_launch_score_fast(const HilsShape& s, const void* qr, const void* ksum,
                                  const float* bsum, void* frag, int32_t* sel, hipStream_t st) {
  const int ntg = frag_tiles(s);
  if (ntg > 0) {
    const long long total = (long long)s.B * s.Hq * ntg * FRAGS * 64;
    HilsProfScope ps_("k_score_frag", st);
    hipLaunchKernelGGL(k_score_frag, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       (const bf16_t*)ksum, bsum, (uint4*)frag, s.nC, ntg, (float)(1.0 / s.tau), total);
  }
  const uint4* fr = (const uint4*)frag;
  switch (s.G) {
    case 1: return launch_score<1>(s, qr, fr, ntg, sel, st);
    case 2: return launch_score<2>(s, qr, fr, ntg, sel, st);
    case 4: return launch_score<4>(s, qr, fr, ntg, sel, st);
  }
  return hipErrorInvalidValue;
}
