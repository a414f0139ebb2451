// Prefill backward on the matrix cores, for bf16 inputs with d in {64, 128}
// and S a multiple of 16: everything that touches the attended keys runs per
// chunk over the chunk's contributions, as MFMA tiles.
//
// "Hierarchical Sparse Attention Done Right", section 3 (chunk attention, the
// sliding window, the routing equation and the fusion softmax).  A
// contribution is a (query i, head h) that attends keys of chunk c: a
// (query, slot) pair whose selection holds c, or a query whose window
// [window_start(i), i] meets c.  For a contribution with fusion weight alpha,
// log-normaliser lse of the softmax the chunk's keys take part in, g = dout.o
// of that softmax's output and, for the window, E = d log Z_swa (0 for a
// selected chunk), every key j it attends gets
//   p_j = exp(tau q.k_j - lse),  ds_j = alpha p_j (dout.v_j - g) + E p_j,
//   dv_j += alpha p_j dout,  dk_j += tau ds_j q,  dq += tau ds_j k_j.
//
// Four passes (plus the selection lists before and the summaries after):
//   k_bwd_mf<D, 0> (stats)  per chunk: lse and g of every selecting pair;
//                           for the window, per (query, chunk) the partial
//                           max / sum exp / sum exp dout.v over the chunk's
//                           keys in the window;
//   k_bwd_rowstat           per (query, head): the window's lse and g from
//                           its partials, the routing scores s_hat, the
//                           fusion weights and their gradients (d s_hat,
//                           d log Z_swa), and the routing query's gradient
//                           tau sum_t (d s_hat_t) k'_t;
//   k_bwd_mf<D, 1> (grads)  per chunk: dk, dv of its tokens, and one dq
//                           partial per contribution;
//   k_bwd_dq_reduce         per (query, head): dq = sum of its partials.
// The four run per query slice (one for most shapes) so that the partials fit
// a bounded workspace: a chunk pass then takes the contributions whose query
// lies in the slice, and dk, dv are written by the slice holding the chunk's
// first token and added to by the later ones.
//
// Layout of the chunk passes: one workgroup per (chunk, sequence, KV group),
// 4 wavefronts; wavefront w owns keys 16w .. 16w + 15 and keeps their K and V
// rows as MFMA operands in registers.  Contributions go in tiles of 32 whose
// q and dout rows are gathered into LDS row-major, double-buffered (the next
// tile's rows load while the current one is computed).  They are the operand
// of S = Q K^T and dP = dOut V^T (reduced over d) as they stand, and of
// dV^T = dOut^T P and dK^T = Q^T dS (reduced over the tile's queries) through
// LDS transpose loads.  S and dP take bf16 MFMA with exact products and
// fp32 sums.  P and tau dS are fp32 and enter their products as bf16 sums
// hi + lo (hi = bf16(x), lo = bf16(x - hi), within 2^-18 of x) in dv and dk,
// and hi + mid + lo (within 2^-27) in dq, whose error gathers over all of a
// query's keys: one MFMA per term, so the gradients keep fp32 accuracy.
// In the gradient pass the MFMA output layout of S (lane l: key l % 16,
// queries 4 (l / 16) + r of each 16-query half) is the B-operand layout of
// the second products once the tile's query positions are permuted
// (position 8 g + t <-> query 16 (t / 4) + 4 g + t % 4); the transpose loads
// gather the A operand in that order.  dq^T = K^T dS^T takes dS through LDS
// (key-contiguous per query) and K^T fragments built once per workgroup.  The
// stats pass takes S^T instead (one query, four keys per lane), whose sums
// over keys are short.  No floating-point atomics: every output element is
// written by one workgroup or wavefront, in a fixed order (the integer
// atomics of the work ordering change only the schedule).
#include <cstdlib>

#include "fast_common.h"
#include "hils_internal.h"
#include "hils_bwd.h"

namespace {

using fastp::ld_bf16x8;
using fastp::mfma16;
using fastp::pack_bf16x2;
using fastp::xshfl_f;

constexpr int MT = 256;     // threads of the chunk passes (4 wavefronts)
constexpr int QT = 32;      // contributions per tile
constexpr int SPLIT = 4096; // stats pass: contributions per workgroup at most (heavy chunks split)

template <int D, int PASS>
struct MfCol {
  static constexpr int RS = D + 8;                 // row-major tile: row stride (bf16), 16-byte pad
  static constexpr int TILE = 2 * QT * RS;         // one buffer: q rows, dout rows
  static constexpr int NPC = QT * (D / 8) / MT;    // 16-byte pieces per thread and tensor
  static constexpr int DSS = 72;                   // dS tile: row stride (bf16), 64 keys + pad
  static constexpr int DSN = 3 * QT * DSS;         // dS tile: three bf16 planes (hi, mid, lo)
  static constexpr int EXTRA = PASS ? DSN : 0;     // the dS tile, after both buffers
  static constexpr int DB = D / 64;                // 16-column blocks of dq per wavefront
  // contributions described per batch: each batch restarts the pipeline (two
  // dependent loads for the descriptors, then the first tile's rows), so the
  // gradient pass takes long batches; the stats pass keeps its LDS small for
  // occupancy
  static constexpr int CB = PASS ? 512 : 128;
  static_assert(CB % QT == 0 && CB >= 4 * QT, "whole tiles; the stats pass's [4][QT] sums fit dcf");
};

// A operand of a product reduced over the tile's queries (dV^T = dOut^T P,
// dK^T = Q^T dS) read from the row-major tile with two LDS transpose loads.
// ds_read_b64_tr_b16 gives output lane j of a 16-lane group, element t, the
// element j % 4 of the 4 read by lane 4 t + j / 4.  Lane 4 t + u of group g4
// reads columns 16 b + 4 u .. + 3 of query 16 c + 4 g4 + t (call c = 0, 1),
// so lane (g4, j) receives column 16 b + j of queries 16 c + 4 g4 + t: the
// fragment A[16 b + j][8 g4 + 4 c + t] in the permuted query order.
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t* lds_s4_ptr;
__device__ __forceinline__ bf16x8_t ld_tr_frag(const bf16_t* rows, int rs, int b, int g4, int l16) {
  const bf16_t* p = rows + (4 * g4 + (l16 >> 2)) * rs + 16 * b + 4 * (l16 & 3);
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(p));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(p + 16 * rs));
  const uint2 a = __builtin_bit_cast(uint2, lo), c = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, c.x, c.y));
}

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

template <int D, int PASS>
__global__ void __launch_bounds__(MT, PASS ? 2 : 4)
k_bwd_mf(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
         const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
         const uint32_t* __restrict__ off, const uint32_t* __restrict__ ent,
         float* __restrict__ pstat, const float* __restrict__ wstat, float* __restrict__ wpart,
         float* __restrict__ dqp, float* __restrict__ dk, float* __restrict__ dv,
         const uint32_t* __restrict__ srng, const uint32_t* __restrict__ order,
         const uint2* __restrict__ sitems, const uint32_t* __restrict__ nsi, int nbgp, int Hq,
         int Hkv, int G, int N, int S, int W, int K, int nC, int nwin, int qa, int qz, int QS,
         float tau) {
  using L = MfCol<D, PASS>;
  extern __shared__ __align__(16) unsigned char smm[];
  bf16_t* tiles = reinterpret_cast<bf16_t*>(smm);                        // [2][TILE]
  int* did = reinterpret_cast<int*>(smm + sizeof(bf16_t) * (2 * L::TILE + L::EXTRA));   // [CB] i << 4 | head
  int* dslot = did + L::CB;                                // [CB] slot, K + window chunk
  int2* dlim = reinterpret_cast<int2*>(dslot + L::CB);     // [CB] attended keys lo..hi
  float4* dcf = reinterpret_cast<float4*>(dlim + L::CB);   // [CB] alpha, lse, g, E; stats: [4][QT] partials
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  // work item (c, b, g) = c (B Hkv) + b Hkv + g.  The gradient pass takes the
  // items heaviest first (order); the stats pass takes their parts (sitems:
  // item, part), an item with more than SPLIT contributions cut into equal
  // parts (its outputs are per contribution), heaviest parts first
  const long long nbg = nbgp;                        // B * Hkv
  long long blk;
  int part = 0;
  if (PASS) {
    blk = order[blockIdx.x];
  } else {
    if (blockIdx.x >= nsi[0]) return;                // the grid bounds the part count
    const uint2 it = sitems[blockIdx.x];
    blk = it.x;
    part = (int)it.y;
  }
  const int c = (int)(blk / nbg);
  const long long bg = blk % nbg;
  const long long hb = (bg / Hkv) * Hq + (long long)(bg % Hkv) * G;
  const int j0 = c * S;
  const int jn = min(S, N - j0);                     // tokens of this chunk
  const int kk = 16 * wv + l16;                      // this lane's key in the MFMA layouts
  const bool kwave = 16 * wv < S;                    // the wavefront owns keys
  const bool kown = kwave && kk < jn;
  const int NS = K + nwin;                           // dq partial slots per (query, head)

  // lane: K[kk][32 s + 8 g4 ..], V likewise; the B operand of S = Q K^T in
  // the gradient pass, the A operand of S^T = K Q^T in the stats pass
  bf16x8_t kf[D / 32], vf[D / 32];
  {
    const long long ro = (bg * (long long)N + j0 + (kown ? kk : 0)) * D + 8 * g4;
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      kf[s2] = __builtin_bit_cast(bf16x8_t, kown ? fastp::ld_u4(k + ro + 32 * s2) : z);
      vf[s2] = __builtin_bit_cast(bf16x8_t, kown ? fastp::ld_u4(v + ro + 32 * s2) : z);
    }
  }
  // gradient pass: A operand of dq^T = K^T dS^T, K^T[16 db + l16][32 ks + 8 g4 ..]
  // for the wavefront's dq column blocks db = DB w ..
  bf16x8_t ktf[PASS ? L::DB : 1][2];
  f32x4_t accv[PASS ? D / 16 : 1], acck[PASS ? D / 16 : 1];
  if (PASS) {
    const unsigned short* k16 = reinterpret_cast<const unsigned short*>(k);
#pragma unroll
    for (int db = 0; db < L::DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t w2[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int k0 = 32 * ks + 8 * g4 + 2 * t;
          const long long e = (bg * (long long)N + j0) * D + 16 * (L::DB * wv + db) + l16;
          const uint32_t lo = k0 < jn ? k16[e + (long long)k0 * D] : 0u;
          const uint32_t hi = k0 + 1 < jn ? k16[e + (long long)(k0 + 1) * D] : 0u;
          w2[t] = lo | (hi << 16);
        }
        ktf[db][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(w2[0], w2[1], w2[2], w2[3]));
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < D / 16; ++b2) {
      accv[b2] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acck[b2] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // contributions of the query slice [qa, qz): the slice's part of the
  // chunk's list (srng, or the whole list for one slice) and its window
  // queries
  const bool summ = c < nC;
  const long long lc = bg * (long long)nC + c;
  const uint32_t p0 = !summ ? 0u : srng ? srng[2 * lc] : off[bg * (nC + 1) + c];
  const uint32_t p1 = !summ ? 0u : srng ? srng[2 * lc + 1] : off[bg * (nC + 1) + c + 1];
  const long long nsel = (long long)(p1 - p0) * G;                 // (pair, head)
  const int wa = max(j0, qa), wz = min(min(N, (c + 1) * S + W - 1), qz);
  const long long nwq = (long long)max(0, wz - wa) * G;          // window (query, head)
  const uint32_t* eg = ent + bg * (long long)N * K;
  // dk, dv: written by the slice holding the chunk's first token (its first
  // contribution), added to by the later ones
  const bool accum = j0 < qa;

  // staging: piece pc = tid + MT m of a tile: query pc / (D / 8), 16-byte part
  // pc % (D / 8), so that a load instruction reads whole rows
  uint4 pq[L::NPC], po[L::NPC];
  auto stage_load = [&](int tl, int nb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < L::NPC; ++m) {
      const int pc = tid + MT * m, qq = pc / (D / 8), part = pc % (D / 8);
      const int u = tl * QT + qq;
      pq[m] = make_uint4(0u, 0u, 0u, 0u);
      po[m] = pq[m];
      if (u < nb) {
        const int id = did[u];
        const long long o = ((hb + (id & 15)) * N + (id >> 4)) * (long long)D + 8 * part;
        pq[m] = fastp::ld_u4(q + o);
        po[m] = fastp::ld_u4(dout + o);
      }
    }
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
    bf16_t* tb = tiles + (size_t)buf * L::TILE;
#pragma unroll
    for (int m = 0; m < L::NPC; ++m) {
      const int pc = tid + MT * m, qq = pc / (D / 8), part = pc % (D / 8);
      fastp::st_u4(tb + qq * L::RS + 8 * part, pq[m]);
      fastp::st_u4(tb + (QT + qq) * L::RS + 8 * part, po[m]);
    }
  };
  // S and dP of the tile for this wavefront's 16 keys: sc[h][r], dp[h][r] for
  // query 16 h + 4 g4 + r, key kk
  auto scores = [&](const bf16_t* tb, f32x4_t* sc, f32x4_t* dp) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      dp[h] = sc[h];
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        const bf16x8_t aq = ld_bf16x8(tb + (16 * h + l16) * L::RS + 32 * s2 + 8 * g4);
        const bf16x8_t ao = ld_bf16x8(tb + (QT + 16 * h + l16) * L::RS + 32 * s2 + 8 * g4);
        sc[h] = mfma16(aq, kf[s2], sc[h]);
        dp[h] = mfma16(ao, vf[s2], dp[h]);
      }
    }
  };

  // stats pass: per query of the tile, max / sum exp / sum exp dout.v over
  // this wavefront's keys, combined over the wavefronts.  The pass takes
  // S^T = K Q^T and dP^T = V dOut^T (the same registers as operands in the
  // other order): lane (g4, l16) then holds keys 16 w + 4 g4 + r of query
  // 16 h + l16, so a query's sums over the wavefront's 16 keys are three
  // in-lane steps and two lane swaps (16 and 32 apart)
  auto compute_stats = [&](int tl, int buf, int nb) __attribute__((always_inline)) {
    float4* red = dcf;                               // [4][QT]
    if (kwave) {
      const bf16_t* tb = tiles + (size_t)buf * L::TILE;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, dp = sc;
#pragma unroll
        for (int s2 = 0; s2 < D / 32; ++s2) {
          const bf16x8_t aq = ld_bf16x8(tb + (16 * h + l16) * L::RS + 32 * s2 + 8 * g4);
          const bf16x8_t ao = ld_bf16x8(tb + (QT + 16 * h + l16) * L::RS + 32 * s2 + 8 * g4);
          sc = mfma16(kf[s2], aq, sc);
          dp = mfma16(vf[s2], ao, dp);
        }
        const int qq = 16 * h + l16;
        const int2 lm = dlim[tl * QT + qq];
        float x[4];
        bool ok[4];
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * wv + 4 * g4 + r;
          ok[r] = key < jn && key >= lm.x && key <= lm.y;
          x[r] = ok[r] ? tau * sc[r] : -INFINITY;
          m = fmaxf(m, x[r]);
        }
        m = fmaxf(m, xshfl_f(m, 16));
        m = fmaxf(m, xshfl_f(m, 32));
        float z = 0.0f, y = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = ok[r] ? __expf(x[r] - m) : 0.0f;
          z += e;
          y = fmaf(e, dp[r], y);
        }
        z += xshfl_f(z, 16);
        z += xshfl_f(z, 32);
        y += xshfl_f(y, 16);
        y += xshfl_f(y, 32);
        if (g4 == 0) red[wv * QT + qq] = make_float4(m, z, y, 0.0f);
      }
    }
    __syncthreads();
    if (tid < QT) {
      const int u = tl * QT + tid;
      if (u < nb) {
        const int nkw = (S + 15) / 16;
        float M = -INFINITY;
        for (int w = 0; w < nkw; ++w) M = fmaxf(M, red[w * QT + tid].x);
        float Z = 0.0f, Y = 0.0f;
        for (int w = 0; w < nkw; ++w) {
          const float4 p = red[w * QT + tid];
          if (p.x > -INFINITY) {
            const float f = __expf(p.x - M);
            Z = fmaf(p.y, f, Z);
            Y = fmaf(p.z, f, Y);
          }
        }
        const int id = did[u], slot = dslot[u];
        const int i = id >> 4, r = id & 15;
        if (slot < K) {
          float* ps = pstat + (((bg * N + i) * (long long)K + slot) * G + r) * 4;
          ps[1] = M + __logf(Z);
          ps[2] = Y / Z;
        } else {
          *reinterpret_cast<float4*>(wpart + (((hb + r) * QS + (i - qa)) * (long long)nwin + (slot - K)) * 4) =
              make_float4(M, Z, Y, 0.0f);
        }
      }
    }
  };

  // gradient pass
  auto compute_grads = [&](int tl, int buf, int nb) __attribute__((always_inline)) {
    bf16_t* tb = tiles + (size_t)buf * L::TILE;
    uint32_t ph[4], pl[4], dh[4], dl[4], d3[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { ph[t] = 0u; pl[t] = 0u; dh[t] = 0u; dl[t] = 0u; d3[t] = 0u; }
    if (kwave) {
      f32x4_t sc[2], dp[2];
      scores(tb, sc, dp);
      // weights of the (query, key) pairs this lane holds
      float ap[8], ds[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = tl * QT + 16 * h + 4 * g4 + r;
          const float4 cf = dcf[u];
          const int2 lm = dlim[u];
          const bool ok = kown && kk >= lm.x && kk <= lm.y;
          const float p = ok ? __expf(tau * sc[h][r] - cf.y) : 0.0f;
          const float a = cf.x * p;
          ap[4 * h + r] = a;
          ds[4 * h + r] = tau * fmaf(a, dp[h][r] - cf.z, cf.w * p);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ph[t] = pack_bf16x2(ap[2 * t], ap[2 * t + 1]);
        pl[t] = pack_bf16x2(ap[2 * t] - bf_lo(ph[t]), ap[2 * t + 1] - bf_hi(ph[t]));
        dh[t] = pack_bf16x2(ds[2 * t], ds[2 * t + 1]);
        dl[t] = pack_bf16x2(ds[2 * t] - bf_lo(dh[t]), ds[2 * t + 1] - bf_hi(dh[t]));
        // third term for dq (its error is summed over all of a query's keys)
        d3[t] = pack_bf16x2(ds[2 * t] - bf_lo(dh[t]) - bf_lo(dl[t]),
                            ds[2 * t + 1] - bf_hi(dh[t]) - bf_hi(dl[t]));
      }
    }
    // dS (hi, mid, lo): [3][QT][DSS], key-contiguous; the previous tile's dq
    // products read it before the barrier that ended that tile
    bf16_t* dst = tiles + 2 * L::TILE;
    {
      unsigned short* dsl = reinterpret_cast<unsigned short*>(dst);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int e = 2 * t + x, qq = 16 * (e >> 2) + 4 * g4 + (e & 3);
          dsl[qq * L::DSS + kk] = (unsigned short)(dh[t] >> (16 * x));
          dsl[(QT + qq) * L::DSS + kk] = (unsigned short)(dl[t] >> (16 * x));
          dsl[(2 * QT + qq) * L::DSS + kk] = (unsigned short)(d3[t] >> (16 * x));
        }
      }
    }
    if (kwave) {
      const bf16x8_t bph = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      const bf16x8_t bpl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
      const bf16x8_t bdh = __builtin_bit_cast(bf16x8_t, make_uint4(dh[0], dh[1], dh[2], dh[3]));
      const bf16x8_t bdl = __builtin_bit_cast(bf16x8_t, make_uint4(dl[0], dl[1], dl[2], dl[3]));
#pragma unroll
      for (int b2 = 0; b2 < D / 16; ++b2) {
        const bf16x8_t ao = ld_tr_frag(tb + QT * L::RS, L::RS, b2, g4, l16);
        const bf16x8_t aq = ld_tr_frag(tb, L::RS, b2, g4, l16);
        accv[b2] = mfma16(ao, bph, accv[b2]);
        accv[b2] = mfma16(ao, bpl, accv[b2]);
        acck[b2] = mfma16(aq, bdh, acck[b2]);
        acck[b2] = mfma16(aq, bdl, acck[b2]);
      }
    }
    __syncthreads();                                 // the dS tile is complete
    // dq^T[16 db + 4 g4 + r][query 16 qb + l16] = sum over the chunk's keys
    const bf16_t* dsl = dst;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int u = tl * QT + 16 * qb + l16;
      long long prow = 0;
      if (u < nb) {
        const int id = did[u];
        prow = ((hb + (id & 15)) * QS + ((id >> 4) - qa)) * (long long)NS + dslot[u];
      }
      bf16x8_t bh[2], bl[2], b3[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bh[ks] = ld_bf16x8(dsl + (16 * qb + l16) * L::DSS + 32 * ks + 8 * g4);
        bl[ks] = ld_bf16x8(dsl + (QT + 16 * qb + l16) * L::DSS + 32 * ks + 8 * g4);
        b3[ks] = ld_bf16x8(dsl + (2 * QT + 16 * qb + l16) * L::DSS + 32 * ks + 8 * g4);
      }
#pragma unroll
      for (int db = 0; db < L::DB; ++db) {
        f32x4_t a = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          a = mfma16(ktf[db][ks], bh[ks], a);
          a = mfma16(ktf[db][ks], bl[ks], a);
          a = mfma16(ktf[db][ks], b3[ks], a);
        }
        if (u < nb)
          *reinterpret_cast<float4*>(dqp + prow * D + 16 * (L::DB * wv + db) + 4 * g4) =
              make_float4(a[0], a[1], a[2], a[3]);
      }
    }
  };

  long long clo = 0, chi = nsel + nwq;              // this workgroup's contributions
  if (!PASS) {
    const long long np = max(1LL, (chi + SPLIT - 1) / SPLIT);
    clo = chi * part / np;
    chi = chi * (part + 1) / np;
  }
  for (long long base = clo; base < chi; base += L::CB) {
    const int nb = (int)min((long long)L::CB, chi - base);
    __syncthreads();                                 // the previous batch is consumed
    for (int t = tid; t < L::CB; t += MT) {
      const long long idx = base + t;
      int id = 0, slot = 0;
      float4 cf = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      int2 lm = make_int2(1, 0);                     // no key
      if (t < nb) {
        if (idx < nsel) {
          const uint32_t e = eg[p0 + idx / G];
          const int r = (int)(idx % G), i = (int)(e >> 8);
          slot = (int)(e & 255u);
          id = (i << 4) | r;
          lm = make_int2(0, S);
          if (PASS) {
            const float4 ps = *reinterpret_cast<const float4*>(
                pstat + (((bg * N + i) * (long long)K + slot) * G + r) * 4);
            cf = make_float4(ps.x, ps.y, ps.z, 0.0f);
          }
        } else {
          const long long widx = idx - nsel;
          const int i = wa + (int)(widx / G), r = (int)(widx % G);
          const int ws = (int)window_start(i, W, S);
          id = (i << 4) | r;
          slot = K + (c - ws / S);
          lm = make_int2(ws - j0, i - j0);
          if (PASS) cf = *reinterpret_cast<const float4*>(wstat + ((hb + r) * N + i) * 4);
        }
      }
      did[t] = id;
      dslot[t] = slot;
      dlim[t] = lm;
      if (PASS) dcf[t] = cf;
    }
    __syncthreads();
    const int ntl = (nb + QT - 1) / QT;
    stage_load(0, nb);
    stage_store(0);
    __syncthreads();
    for (int tl = 0; tl < ntl; ++tl) {
      if (tl + 1 < ntl) stage_load(tl + 1, nb);
      if (PASS) compute_grads(tl, tl & 1, nb);
      else compute_stats(tl, tl & 1, nb);
      // buffer (tl + 1) & 1 was last read in tile tl - 1, before the barrier
      // that ended it
      if (tl + 1 < ntl) stage_store((tl + 1) & 1);
      __syncthreads();
    }
  }
  if (PASS && kown) {
    const long long ro = (bg * (long long)N + j0 + kk) * D + 4 * g4;
#pragma unroll
    for (int b2 = 0; b2 < D / 16; ++b2) {
      float4* pv = reinterpret_cast<float4*>(dv + ro + 16 * b2);
      float4* pk = reinterpret_cast<float4*>(dk + ro + 16 * b2);
      float4 av = make_float4(accv[b2][0], accv[b2][1], accv[b2][2], accv[b2][3]);
      float4 ak = make_float4(acck[b2][0], acck[b2][1], acck[b2][2], acck[b2][3]);
      if (accum) {
        const float4 ov = *pv, ok = *pk;
        av = make_float4(ov.x + av.x, ov.y + av.y, ov.z + av.z, ov.w + av.w);
        ak = make_float4(ok.x + ak.x, ok.y + ak.y, ok.z + ak.z, ok.w + ak.w);
      }
      *pv = av;
      *pk = ak;
    }
  }
}

template <int D, int PASS>
size_t mf_lds() {
  return sizeof(bf16_t) * (2 * MfCol<D, PASS>::TILE + MfCol<D, PASS>::EXTRA) +
         (size_t)MfCol<D, PASS>::CB * (2 * sizeof(int) + sizeof(int2) + sizeof(float4));
}

// ---------------------------------------------------------------------------
// per (query, head): window statistics from the partials, routing scores,
// fusion weights and their gradients; one wavefront per row, K <= 128.
// NI > 0: the k' rows of the selected slots are read once, as PR = D / 8
// pieces of 16 bytes (lane (rr, pc) = (lane / PR, lane % PR) holds piece pc of
// the rows of slots RPI x + rr, x < NI, RPI = 64 / PR, all in flight), and
// serve both the routing scores (piece dot products summed over the PR lanes
// of a row) and tau sum_t (d s_hat_t) k'_t (summed over x, then over the RPI
// row groups).  NI = 0: one lane per slot for the scores, the k' rows read
// again for the routing query's gradient (K > 16 RPI).
template <int D, int NI>
__global__ void __launch_bounds__(256)
k_bwd_rowstat(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ ksum,
              const float* __restrict__ bsum, const int32_t* __restrict__ sel,
              float* __restrict__ pstat, float* __restrict__ wstat, const float* __restrict__ wpart,
              float* __restrict__ dqo, int Hq, int Hkv, int G, int N, int d, int S, int W, int K,
              int nC, int nwin, int qa, int QN, int QS, long long nrows, float tau) {
  extern __shared__ __align__(16) float smq[];       // [4][d] routing query rows
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long item = (long long)blockIdx.x * 4 + wv;   // (b, h, i - qa), slice rows
  if (item >= nrows) return;                         // whole wavefronts; no barriers below
  const int i = qa + (int)(item % QN);
  const long long bh = item / QN;
  const int h = (int)(bh % Hq);
  const long long b = bh / Hq;
  const int g = h / G, r = h - g * G;
  const long long row = (b * Hkv + g) * N + i;       // selection row
  const long long arow = bh * N + i;                 // (b, h, i)
  const long long srow = bh * QS + (i - qa);         // its row of the slice's partials
  float* qs = smq + wv * d;
  for (int e = lane; e < d; e += 64) qs[e] = bf16_to_f32(qr[arow * d + e]);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // selected chunks: lanes t and t + 64
  float sh[2], lt[2], gt[2];
  bool vt[2];
  int cs[2];                                         // chunk of slot lane + 64 m, -1 if none
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = lane + 64 * m;
    vt[m] = false;
    sh[m] = -INFINITY;
    lt[m] = 0.0f;
    gt[m] = 0.0f;
    cs[m] = -1;
    if (t < K) {
      const int c = sel[row * K + t];
      if (c >= 0 && c < nC) {
        cs[m] = c;
        vt[m] = true;
        if constexpr (NI == 0) {
          const bf16_t* kp = ksum + (bh * nC + c) * (long long)d;
          float a = 0.0f;
          for (int e = 0; e < d; e += 8) {
            const uint4 u = fastp::ld_u4(kp + e);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              a = fmaf(qs[e + 2 * x], bf_lo(w4[x]), a);
              a = fmaf(qs[e + 2 * x + 1], bf_hi(w4[x]), a);
            }
          }
          sh[m] = fmaf(tau, a, bsum[bh * nC + c]);
        } else {
          sh[m] = bsum[bh * nC + c];                 // the score is added below
        }
        const float* ps = pstat + ((row * K + t) * G + r) * 4;
        lt[m] = ps[1];
        gt[m] = ps[2];
      }
    }
  }
  constexpr int PR = D / 8, RPI = 64 / PR;
  const int rr = lane / PR, pc = lane % PR;
  uint4 kr[NI > 0 ? NI : 1];
  if constexpr (NI > 0) {
    // slot RPI x + rr of this lane: its chunk from the slot lanes, its k' piece
    float qv[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) qv[x] = qs[8 * pc + x];
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const int t = RPI * x + rr;
      const int ca = __shfl(cs[0], t & 63, 64), cb = __shfl(cs[1], t & 63, 64);
      const int c = t < 64 ? ca : cb;
      kr[x] = make_uint4(0u, 0u, 0u, 0u);
      if (t < K && c >= 0) kr[x] = fastp::ld_u4(ksum + (bh * nC + c) * (long long)D + 8 * pc);
    }
    float a[NI];
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const uint32_t w4[4] = {kr[x].x, kr[x].y, kr[x].z, kr[x].w};
      float acc = 0.0f;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        acc = fmaf(qv[2 * y], bf_lo(w4[y]), acc);
        acc = fmaf(qv[2 * y + 1], bf_hi(w4[y]), acc);
      }
#pragma unroll
      for (int msk = 1; msk < PR; msk <<= 1) acc += fastp::xshfl_f(acc, msk);
      a[x] = acc;
    }
    // slot lane + 64 m takes the sum of its row group
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const float v = __shfl(a[x], PR * (lane % RPI), 64);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (vt[m] && (lane + 64 * m) / RPI == x) sh[m] = fmaf(tau, v, sh[m]);
    }
  }
  // the window: partials of its chunks
  const int ws = (int)window_start(i, W, S);
  const int nw = i / S - ws / S + 1;
  float wm = -INFINITY, wz = 0.0f, wy = 0.0f;      // this lane's chunks, online
  for (int w = lane; w < nw; w += 64) {
    const float4 p = *reinterpret_cast<const float4*>(wpart + (srow * nwin + w) * 4);
    if (p.x > wm) {
      const float f = __expf(wm - p.x);
      wz = fmaf(wz, f, p.y);
      wy = fmaf(wy, f, p.z);
      wm = p.x;
    } else if (p.x > -INFINITY) {
      const float f = __expf(p.x - wm);
      wz = fmaf(p.y, f, wz);
      wy = fmaf(p.z, f, wy);
    }
  }
  const float Mw = wave_max_f(wm);
  const float fw = wm > -INFINITY ? __expf(wm - Mw) : 0.0f;
  const float Zw = wave_sum_f(wz * fw);
  const float Yw = wave_sum_f(wy * fw);
  const float lse_w = Mw + __logf(Zw);
  const float g_w = Yw / Zw;
  // fusion softmax over {s_hat_t} U {log Z_swa}
  const float Mf = fmaxf(wave_max_f(fmaxf(sh[0], sh[1])), lse_w);
  float ez[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) ez[m] = vt[m] ? __expf(sh[m] - Mf) : 0.0f;
  const float ew = __expf(lse_w - Mf);
  const float Zf = wave_sum_f(ez[0] + ez[1]) + ew;
  const float aw = ew / Zf;
  float at[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) at[m] = ez[m] / Zf;
  const float gbar = fmaf(aw, g_w, wave_sum_f(fmaf(at[0], gt[0], at[1] * gt[1])));
  float dsh[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    dsh[m] = at[m] * (gt[m] - gbar);
    if (vt[m])
      *reinterpret_cast<float4*>(pstat + ((row * K + lane + 64 * m) * G + r) * 4) =
          make_float4(at[m], lt[m], gt[m], dsh[m]);
  }
  if (lane == 0)
    *reinterpret_cast<float4*>(wstat + arow * 4) = make_float4(aw, lse_w, g_w, aw * (g_w - gbar));
  if constexpr (NI > 0) {
    // routing query: tau sum_t (d s_hat_t) k'_t from the k' pieces in registers
    float qa8[8];
#pragma unroll
    for (int y = 0; y < 8; ++y) qa8[y] = 0.0f;
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const int t = RPI * x + rr;
      const float da = __shfl(dsh[0], t & 63, 64), db = __shfl(dsh[1], t & 63, 64);
      const float w = t < K ? (t < 64 ? da : db) : 0.0f;   // empty slots: zero piece
      const uint32_t w4[4] = {kr[x].x, kr[x].y, kr[x].z, kr[x].w};
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        qa8[2 * y] = fmaf(w, bf_lo(w4[y]), qa8[2 * y]);
        qa8[2 * y + 1] = fmaf(w, bf_hi(w4[y]), qa8[2 * y + 1]);
      }
    }
#pragma unroll
    for (int msk = PR; msk < 64; msk <<= 1)
#pragma unroll
      for (int y = 0; y < 8; ++y) qa8[y] += fastp::xshfl_f(qa8[y], msk);
    if (rr == 0) {
      float* o = dqo + arow * D + 8 * pc;
      *reinterpret_cast<float4*>(o) = make_float4(tau * qa8[0], tau * qa8[1], tau * qa8[2], tau * qa8[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(tau * qa8[4], tau * qa8[5], tau * qa8[6], tau * qa8[7]);
    }
    return;
  }
  // routing query: tau sum_t (d s_hat_t) k'_t; lane takes elements 2 lane,
  // 2 lane + 1; slots in order, eight k' rows in flight, the chunk ids and
  // d s_hat from the slot lanes
  float q0 = 0.0f, q1 = 0.0f;
  const int e = 2 * lane;
  for (int t0 = 0; t0 < K; t0 += 8) {
    uint32_t kv[8];
    float xs[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int t = min(t0 + x, K - 1);
      const int c = __shfl(t < 64 ? cs[0] : cs[1], t & 63, 64);
      const float ds = __shfl(t < 64 ? dsh[0] : dsh[1], t & 63, 64);
      const bool ok = t0 + x < K && c >= 0;
      xs[x] = ok ? ds : 0.0f;
      kv[x] = (ok && e < d) ? *reinterpret_cast<const uint32_t*>(ksum + (bh * nC + c) * (long long)d + e) : 0u;
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      q0 = fmaf(xs[x], bf_lo(kv[x]), q0);
      q1 = fmaf(xs[x], bf_hi(kv[x]), q1);
    }
  }
  if (e < d) *reinterpret_cast<float2*>(dqo + arow * d + e) = make_float2(tau * q0, tau * q1);
}

// streaming 16-byte load: the dq partials are read once
typedef float f4nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_f4_nt(const float* p) {
  const f4nt_t w = __builtin_nontemporal_load(reinterpret_cast<const f4nt_t*>(p));
  return make_float4(w.x, w.y, w.z, w.w);
}

// per (query, head): dq = (add ? dq : 0) + the partials of its selected
// chunks and window chunks; one wavefront per row.  A partial row is read as
// PR = D / 4 pieces of 16 bytes, so one load instruction covers SPI = 64 / PR
// partial rows: lane (sub, e) = (lane / PR, 4 (lane % PR)) takes every SPI-th
// slot of the row's slot sequence, eight of them in flight, and the SPI
// partial sums meet by lane swaps at the end
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_dq_reduce(const float* __restrict__ dqp, const int32_t* __restrict__ sel, float* __restrict__ dq,
                int Hq, int Hkv, int G, int N, int S, int W, int K, int nC, int nwin,
                int qa, int QN, int QS, long long nrows, int add) {
  constexpr int PR = D / 4, SPI = 64 / PR;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long item = (long long)blockIdx.x * 4 + wv;
  if (item >= nrows) return;
  const int sub = lane / PR, e = 4 * (lane % PR);
  const int i = qa + (int)(item % QN);
  const long long bh = item / QN;
  const int h = (int)(bh % Hq);
  const long long b = bh / Hq;
  const long long row = (b * Hkv + h / G) * N + i;
  const long long arow = bh * N + i;
  const float* pp = dqp + (bh * QS + (i - qa)) * (long long)(K + nwin) * D + e;
  float4 acc = (add && sub == 0) ? *reinterpret_cast<const float4*>(dq + arow * D + e)
                                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // the selected slots that hold a chunk (one ballot bit per slot, K <= 128),
  // then the window chunks, in this order; the sequence is the same in every
  // lane (ballots and counters are uniform)
  const int c0 = lane < K ? sel[row * K + lane] : -1;
  const int c1 = lane + 64 < K ? sel[row * K + lane + 64] : -1;
  uint64_t m0 = __ballot(c0 >= 0 && c0 < nC), m1 = __ballot(c1 >= 0 && c1 < nC);
  const int ws = (int)window_start(i, W, S);
  const int nw = i / S - ws / S + 1;
  int wn = 0;
  for (;;) {
    int sl[8], first = -1;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      int mine = -1;
#pragma unroll
      for (int y = 0; y < SPI; ++y) {
        int t = -1;
        if (m0) { t = __ffsll((unsigned long long)m0) - 1; m0 &= m0 - 1; }
        else if (m1) { t = 64 + __ffsll((unsigned long long)m1) - 1; m1 &= m1 - 1; }
        else if (wn < nw) t = K + wn++;
        if (x == 0 && y == 0) first = t;
        if (y == sub) mine = t;
      }
      sl[x] = mine;
    }
    if (first < 0) break;
    float4 v[8];
#pragma unroll
    for (int x = 0; x < 8; ++x)
      v[x] = sl[x] >= 0 ? ld_f4_nt(pp + (long long)sl[x] * D) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      acc.x += v[x].x;
      acc.y += v[x].y;
      acc.z += v[x].z;
      acc.w += v[x].w;
    }
  }
#pragma unroll
  for (int msk = PR; msk < 64; msk <<= 1) {
    acc.x += __shfl_xor(acc.x, msk, 64);
    acc.y += __shfl_xor(acc.y, msk, 64);
    acc.z += __shfl_xor(acc.z, msk, 64);
    acc.w += __shfl_xor(acc.w, msk, 64);
  }
  if (sub == 0) *reinterpret_cast<float4*>(dq + arow * D + e) = acc;
}

// per (sequence, KV group, chunk with a summary): the part of the chunk's
// query-ordered list whose queries lie in [qa, qz) (entries are i << 8 | slot)
__global__ void __launch_bounds__(256)
k_bwd_slice_ranges(const uint32_t* __restrict__ off, const uint32_t* __restrict__ ent,
                   uint32_t* __restrict__ srng, int N, int K, int nC, long long nlists, int qa,
                   int qz) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= nlists) return;
  const long long bg = t / nC;
  const int c = (int)(t % nC);
  const uint32_t* eg = ent + bg * (long long)N * K;
  const uint32_t p0 = off[bg * (nC + 1) + c], p1 = off[bg * (nC + 1) + c + 1];
  auto lower = [&](uint32_t key) {
    uint32_t lo = p0, hi = p1;
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (eg[mid] < key) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  srng[2 * t] = lower((uint32_t)qa << 8);
  srng[2 * t + 1] = lower((uint32_t)qz << 8);
}

// Work items (chunk, sequence, KV group) of a slice in decreasing order of
// their contribution counts (bucketed by powers of two), so that the chunk
// passes start the longest workgroups first: a chunk's count depends on its
// position and on the routing (a chunk many queries select takes several
// times the mean).  For the stats pass the same, by part: an item with w
// contributions is cut into ceil(w / SPLIT) parts (none when w = 0), listed
// in sitems (item, part), their number in nsi[0].  The orders change only the
// schedule, not any result.
__global__ void __launch_bounds__(1024)
k_bwd_order(const uint32_t* __restrict__ off, const uint32_t* __restrict__ srng,
            uint32_t* __restrict__ order, uint2* __restrict__ sitems, uint32_t* __restrict__ nsi,
            int nbg, int ncs, int nC, int G, int N, int S, int W, int qa, int qz) {
  __shared__ uint32_t hist[33], cur[33], hist2[33], cur2[33];
  const int tid = threadIdx.x;
  const long long n = (long long)nbg * ncs;
  auto work = [&](long long t) {
    const int c = (int)(t / nbg);
    const long long bg = t % nbg;
    long long w = 0;
    if (c < nC) {
      const long long lc = bg * nC + c;
      w = srng ? (long long)srng[2 * lc + 1] - srng[2 * lc]
               : (long long)off[bg * (nC + 1) + c + 1] - off[bg * (nC + 1) + c];
    }
    const int j0 = c * S;
    w += max(0, min(min(N, (c + 1) * S + W - 1), qz) - max(j0, qa));
    return w * G;
  };
  auto bucket = [](long long w) {                    // 0 .. 32 (w < 2^32)
    return min(w > 0 ? 64 - __clzll((unsigned long long)w) : 0, 32);
  };
  auto parts = [](long long w) { return (w + SPLIT - 1) / SPLIT; };
  if (tid < 33) { hist[tid] = 0u; hist2[tid] = 0u; }
  __syncthreads();
  for (long long t = tid; t < n; t += 1024) {
    const long long w = work(t), np = parts(w);
    atomicAdd(&hist[bucket(w)], 1u);
    if (np > 0) atomicAdd(&hist2[bucket((w + np - 1) / np)], (uint32_t)np);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0, run2 = 0;
    for (int b = 32; b >= 0; --b) {
      cur[b] = run;
      run += hist[b];
      cur2[b] = run2;
      run2 += hist2[b];
    }
    nsi[0] = run2;
  }
  __syncthreads();
  for (long long t = tid; t < n; t += 1024) {
    const long long w = work(t), np = parts(w);
    order[atomicAdd(&cur[bucket(w)], 1u)] = (uint32_t)t;
    if (np > 0) {
      const uint32_t p0 = atomicAdd(&cur2[bucket((w + np - 1) / np)], (uint32_t)np);
      for (long long p = 0; p < np; ++p) sitems[p0 + p] = make_uint2((uint32_t)t, (uint32_t)p);
    }
  }
}

// upper bound of the stats pass's parts in a slice of QN queries: one per
// item plus one per SPLIT of the most contributions the slice can have
// (every query and head with K selected chunks and nwin window chunks)
long long stats_parts_max(const HilsShape& s, int QN) {
  return (long long)s.B * s.Hkv * s.nCc +
         ((long long)s.B * s.Hq * QN * (s.K + s.nwin) + SPLIT - 1) / SPLIT;
}

template <int D>
hipError_t launch_mf(const HilsShape& s, const void* q, const void* qr, const void* k, const void* v,
                     const void* dout, const int32_t* sel, const void* ksum, const float* bsum,
                     float* dq, float* dqr, float* dk, float* dv, const HilsBwdBufs& wb,
                     hipStream_t st) {
  const float tau = (float)s.tau;
  const int QS = hils_bwd_mf_slice(s);
  const size_t sh0 = mf_lds<D, 0>(), sh1 = mf_lds<D, 1>();
  // row pass: the selected slots' k' pieces in registers, NI rows per lane
  // (a power of two covering K), while NI <= 16
  constexpr int RPI = 64 / (D / 8);
  const int need = (s.K + RPI - 1) / RPI;
  auto rowstat = need <= 1 ? k_bwd_rowstat<D, 1> : need <= 2 ? k_bwd_rowstat<D, 2>
               : need <= 4 ? k_bwd_rowstat<D, 4> : need <= 8 ? k_bwd_rowstat<D, 8>
               : need <= 16 ? k_bwd_rowstat<D, 16> : k_bwd_rowstat<D, 0>;
  hils_allow_lds((const void*)k_bwd_mf<D, 0>, sh0);
  hils_allow_lds((const void*)k_bwd_mf<D, 1>, sh1);
  for (int qa = 0; qa < s.N; qa += QS) {
    const int qz = min(s.N, qa + QS), QN = qz - qa;
    const uint32_t* srng = nullptr;
    if (QS < s.N && s.nC > 0) {
      const long long nl = (long long)s.B * s.Hkv * s.nC;
      HilsProfScope ps_("k_bwd_slice_ranges", st);
      hipLaunchKernelGGL(k_bwd_slice_ranges, dim3((unsigned)((nl + 255) / 256)), dim3(256), 0, st,
                         wb.off, wb.ent, wb.srng, s.N, s.K, s.nC, nl, qa, qz);
      srng = wb.srng;
    }
    // chunks with a token before qz (the others have no contribution yet)
    const int ncs = min(s.nCc, (qz + s.S - 1) / s.S);
    const long long nblk = (long long)s.B * s.Hkv * ncs;
    { HilsProfScope ps_("k_bwd_order", st);
      hipLaunchKernelGGL(k_bwd_order, dim3(1), dim3(1024), 0, st, wb.off, srng, wb.order,
                         wb.sitems, wb.nsi, s.B * s.Hkv, ncs, s.nC, s.G, s.N, s.S, s.W, qa, qz); }
    const long long nrows = (long long)s.B * s.Hq * QN;
    const unsigned rgrid = (unsigned)((nrows + 3) / 4);
    { HilsProfScope ps_("k_bwd_stats", st);
      hipLaunchKernelGGL((k_bwd_mf<D, 0>), dim3((unsigned)stats_parts_max(s, QN)), dim3(MT), sh0, st,
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)dout,
                         wb.off, wb.ent, wb.pstat, wb.wstat, wb.wpart, wb.dqp, dk, dv, srng,
                         wb.order, wb.sitems, wb.nsi, s.B * s.Hkv, s.Hq, s.Hkv, s.G, s.N, s.S, s.W,
                         s.K, s.nC, s.nwin, qa, qz, QS, tau); }
    // the routing query's gradient goes to dq_route, or to dq (then the
    // partials are added to it)
    { HilsProfScope ps_("k_bwd_rowstat", st);
      hipLaunchKernelGGL(rowstat, dim3(rgrid), dim3(256), sizeof(float) * 4 * s.d, st,
                         (const bf16_t*)qr, (const bf16_t*)ksum, bsum, sel, wb.pstat, wb.wstat,
                         wb.wpart, dqr ? dqr : dq, s.Hq, s.Hkv, s.G, s.N, s.d, s.S, s.W, s.K, s.nC,
                         s.nwin, qa, QN, QS, nrows, tau); }
    { HilsProfScope ps_("k_bwd_cols", st);
      hipLaunchKernelGGL((k_bwd_mf<D, 1>), dim3((unsigned)nblk), dim3(MT), sh1, st,
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)dout,
                         wb.off, wb.ent, wb.pstat, wb.wstat, wb.wpart, wb.dqp, dk, dv, srng,
                         wb.order, wb.sitems, wb.nsi, s.B * s.Hkv, s.Hq, s.Hkv, s.G, s.N, s.S, s.W,
                         s.K, s.nC, s.nwin, qa, qz, QS, tau); }
    { HilsProfScope ps_("k_bwd_dq", st);
      hipLaunchKernelGGL(k_bwd_dq_reduce<D>, dim3(rgrid), dim3(256), 0, st, wb.dqp, sel, dq, s.Hq,
                         s.Hkv, s.G, s.N, s.S, s.W, s.K, s.nC, s.nwin, qa, QN, QS, nrows,
                         dqr ? 0 : 1); }
  }
  return hipGetLastError();
}

}  // namespace

// Queries per slice: the slice's dq and window partials stay within 4 GiB
// (all of prefill_8k in one slice; about 2.6K query rows of 32 heads at
// K = 64, W = 2048).  HILS_BWD_SLICE_QUERIES, when set to a positive count,
// caps it (tests use it to run several slices at small sizes).
int hils_bwd_mf_slice(const HilsShape& s) {
  const size_t per_q = (size_t)s.B * s.Hq * ((size_t)(s.K + s.nwin) * s.d * 4 + (size_t)s.nwin * 16);
  size_t qs = ((size_t)4 << 30) / (per_q ? per_q : 1);
  if (const char* e = getenv("HILS_BWD_SLICE_QUERIES")) {
    const long v = atol(e);
    if (v > 0 && (size_t)v < qs) qs = (size_t)v;
  }
  if (qs < 1) qs = 1;
  return qs >= (size_t)s.N ? s.N : (int)qs;
}

size_t hils_bwd_mf_wpart_bytes(const HilsShape& s) {
  return (size_t)s.B * s.Hq * hils_bwd_mf_slice(s) * s.nwin * 16;
}
size_t hils_bwd_mf_dqp_bytes(const HilsShape& s) {
  return (size_t)s.B * s.Hq * hils_bwd_mf_slice(s) * (s.K + s.nwin) * s.d * 4;
}
size_t hils_bwd_mf_order_bytes(const HilsShape& s) { return (size_t)s.B * s.Hkv * s.nCc * 4; }
size_t hils_bwd_mf_sitems_bytes(const HilsShape& s) {
  return (size_t)stats_parts_max(s, hils_bwd_mf_slice(s)) * 8 + 16;   // parts, then the count
}
size_t hils_bwd_mf_srng_bytes(const HilsShape& s) {
  return hils_bwd_mf_slice(s) < s.N ? (size_t)s.B * s.Hkv * s.nC * 8 : 0;
}

bool hils_bwd_mf_ok(const HilsShape& s) {
  return s.dtype == 0 && (s.d == 64 || s.d == 128) && s.S % 16 == 0 && s.S <= 64 && s.G <= 16 &&
         s.K <= 128 && s.N < (1 << 24);
}

hipError_t hils_launch_backward_mf(const HilsShape& s, const void* q, const void* qr, const void* k,
                                   const void* v, const void* dout, const int32_t* sel,
                                   const void* ksum, const float* bsum, float* dq, float* dqr,
                                   float* dk, float* dv, const HilsBwdBufs& wb, hipStream_t st) {
  if (!hils_bwd_mf_ok(s) || !wb.wpart || !wb.dqp || !wb.order || !wb.sitems || !wb.nsi)
    return hipErrorInvalidValue;
  if (hils_bwd_mf_slice(s) < s.N && s.nC > 0 && !wb.srng) return hipErrorInvalidValue;
  if ((long long)s.B * s.Hkv * s.nCc <= 0) return hipSuccess;
  return s.d == 128 ? launch_mf<128>(s, q, qr, k, v, dout, sel, ksum, bsum, dq, dqr, dk, dv, wb, st)
                    : launch_mf<64>(s, q, qr, k, v, dout, sel, ksum, bsum, dq, dqr, dk, dv, wb, st);
}
