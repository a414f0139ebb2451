// Prefill backward, column pass on the matrix cores: dk and dv of one chunk's
// tokens over every (query, head) that attends them, for bf16 inputs with
// d in {64, 128} and S a multiple of 16.
//
// "Hierarchical Sparse Attention Done Right", section 3 (chunk attention, the
// sliding window and the fusion softmax).  With the row pass's statistics of
// a contribution (query i, head h) to chunk c - the fusion weight alpha, the
// log-normaliser lse of the softmax the chunk's keys take part in, g = dout.o
// of that softmax's output and, for the window, d log Z_swa = E - every key j
// of the chunk it attends gets
//   p_j = exp(tau q.k_j - lse),  dv_j += alpha p_j dout,
//   ds_j = alpha p_j (dout.v_j - g) + E p_j,  dk_j += tau ds_j q.
// The contributions are the (query, slot) pairs that selected the chunk (E = 0)
// and the queries whose window holds any of its keys (each key j counts only
// where window_start(i) <= j <= i).
//
// One workgroup per (chunk, sequence, KV group), 4 wavefronts; wavefront w owns
// keys 16w .. 16w + 15 and keeps their K and V rows as MFMA operands in
// registers.  Contributions go in tiles of 32: their q and dout rows are
// gathered into LDS both row-major (operand of S = Q K^T and dP = dOut V^T,
// reduced over d) and transposed (operand of dV^T = dOut^T P and
// dK^T = Q^T dS, reduced over the tile's queries), double-buffered, the next
// tile's rows loaded while the current one is computed.  S and dP take bf16
// MFMA with exact products and fp32 sums; P and tau dS are fp32 and enter
// their products as a bf16 pair hi + lo (hi = bf16(x), lo = bf16(x - hi),
// within 2^-18 of x), two MFMAs each, so the gradients keep fp32 accuracy.
// The MFMA output layout of S (lane l: key l % 16, queries 4 (l / 16) + r of
// each 16-query half) is the B-operand layout of the second products once the
// tile's query positions are permuted (position 8 g + t <-> query
// 16 (t / 4) + 4 g + t % 4); the transposed LDS tiles store queries at those
// positions.  No atomics: every dk, dv row is written by one workgroup.
#include "fast_common.h"
#include "hils_internal.h"
#include "hils_bwd.h"

namespace {

using fastp::ld_bf16x8;
using fastp::mfma16;
using fastp::pack_bf16x2;

constexpr int MT = 256;     // threads (4 wavefronts)
constexpr int QT = 32;      // contributions per tile
constexpr int CB = 128;     // contributions described per batch

template <int D>
struct MfCol {
  static constexpr int RS = D + 8;     // row-major tile: row stride (bf16), 16-byte pad
  static constexpr int TS = QT + 8;    // transposed tile: row stride (bf16), 16-byte pad
  // one buffer: q rows, dout rows, q^T, dout^T
  static constexpr int TILE = 2 * QT * RS + 2 * D * TS;
  static constexpr int NPC = QT * (D / 8) / MT;   // 16-byte pieces per thread per tensor
};

// position of tile query q in the transposed tiles (see above)
__device__ __forceinline__ int tpos(int q) { return 8 * ((q & 15) >> 2) + 4 * (q >> 4) + (q & 3); }

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

template <int D>
__global__ void __launch_bounds__(MT, 2)
k_bwd_cols_mf(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
              const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
              const uint32_t* __restrict__ off, const uint32_t* __restrict__ ent,
              const float* __restrict__ pstat, const float* __restrict__ wstat,
              float* __restrict__ dk, float* __restrict__ dv, int Hq, int Hkv, int G, int N,
              int S, int W, int K, int nC, int nCc, float tau) {
  using L = MfCol<D>;
  extern __shared__ __align__(16) unsigned char smm[];
  bf16_t* tiles = reinterpret_cast<bf16_t*>(smm);                      // [2][TILE]
  int* did = reinterpret_cast<int*>(smm + sizeof(bf16_t) * 2 * L::TILE); // [CB] i << 4 | head
  float4* dcf = reinterpret_cast<float4*>(did + CB);                    // [CB] alpha, lse, g, E
  int2* dlim = reinterpret_cast<int2*>(dcf + CB);                       // [CB] attended keys lo..hi
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  // chunk-major order (c, b, g), as in the VALU column pass
  const long long nbg = gridDim.x / nCc;             // B * Hkv
  const long long blk = blockIdx.x;
  const int c = (int)(blk / nbg);
  const long long bg = blk % nbg;
  const int gq = (int)(bg % Hkv);
  const long long hb = (bg / Hkv) * Hq + (long long)gq * G;
  const int j0 = c * S;
  const int jn = min(S, N - j0);                     // tokens of this chunk
  const int kk = 16 * wv + l16;                      // this lane's key in the MFMA layouts
  const bool kwave = 16 * wv < S;                    // the wavefront owns keys
  const bool kown = kwave && kk < jn;

  bf16x8_t kf[D / 32], vf[D / 32];                   // B operand: K[kk][32 s + 8 g4 ..]
  {
    const long long ro = (bg * (long long)N + j0 + (kown ? kk : 0)) * D + 8 * g4;
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      kf[s2] = __builtin_bit_cast(bf16x8_t, kown ? fastp::ld_u4(k + ro + 32 * s2) : z);
      vf[s2] = __builtin_bit_cast(bf16x8_t, kown ? fastp::ld_u4(v + ro + 32 * s2) : z);
    }
  }
  f32x4_t accv[D / 16], acck[D / 16];
#pragma unroll
  for (int b2 = 0; b2 < D / 16; ++b2) {
    accv[b2] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    acck[b2] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const bool summ = c < nC;
  const uint32_t p0 = summ ? off[bg * (nC + 1) + c] : 0u;
  const uint32_t p1 = summ ? off[bg * (nC + 1) + c + 1] : 0u;
  const long long nsel = (long long)(p1 - p0) * G;                 // (pair, head)
  const int i1 = min(N, (c + 1) * S + W - 1);
  const long long nwin = (long long)(i1 - j0) * G;                // window (query, head)
  const uint32_t* eg = ent + bg * (long long)N * K;

  // staging: piece pc = tid + MT m of a tile: query pc % QT, 16-byte part pc / QT
  uint4 pq[L::NPC], po[L::NPC];
  auto stage_load = [&](int tl, int nb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < L::NPC; ++m) {
      const int pc = tid + MT * m, qq = pc % QT, part = pc / QT;
      const int u = tl * QT + qq;
      pq[m] = make_uint4(0u, 0u, 0u, 0u);
      po[m] = pq[m];
      if (u < nb) {
        const int id = did[u];
        const int i = (id >> 4) & 0x7ffffff, r = id & 15;
        const long long o = ((hb + r) * N + i) * (long long)D + 8 * part;
        pq[m] = fastp::ld_u4(q + o);
        po[m] = fastp::ld_u4(dout + o);
      }
    }
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
    bf16_t* tb = tiles + (size_t)buf * L::TILE;
    unsigned short* tq = reinterpret_cast<unsigned short*>(tb + 2 * QT * L::RS);
    unsigned short* to = tq + D * L::TS;
#pragma unroll
    for (int m = 0; m < L::NPC; ++m) {
      const int pc = tid + MT * m, qq = pc % QT, part = pc / QT;
      fastp::st_u4(tb + qq * L::RS + 8 * part, pq[m]);
      fastp::st_u4(tb + (QT + qq) * L::RS + 8 * part, po[m]);
      const int ps = tpos(qq);
      const uint32_t wq[4] = {pq[m].x, pq[m].y, pq[m].z, pq[m].w};
      const uint32_t wo[4] = {po[m].x, po[m].y, po[m].z, po[m].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = 8 * part + e;
        tq[row * L::TS + ps] = (unsigned short)(wq[e >> 1] >> (16 * (e & 1)));
        to[row * L::TS + ps] = (unsigned short)(wo[e >> 1] >> (16 * (e & 1)));
      }
    }
  };
  auto compute = [&](int tl, int buf) __attribute__((always_inline)) {
    const bf16_t* tb = tiles + (size_t)buf * L::TILE;
    const bf16_t* tqt = tb + 2 * QT * L::RS;
    const bf16_t* tot = tqt + D * L::TS;
    f32x4_t sc[2], dp[2];
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
    // weights of the (query, key) pairs this lane holds: query 16 h + 4 g4 + r
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
    uint32_t ph[4], pl[4], dh[4], dl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      ph[t] = pack_bf16x2(ap[2 * t], ap[2 * t + 1]);
      pl[t] = pack_bf16x2(ap[2 * t] - bf_lo(ph[t]), ap[2 * t + 1] - bf_hi(ph[t]));
      dh[t] = pack_bf16x2(ds[2 * t], ds[2 * t + 1]);
      dl[t] = pack_bf16x2(ds[2 * t] - bf_lo(dh[t]), ds[2 * t + 1] - bf_hi(dh[t]));
    }
    const bf16x8_t bph = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8_t bpl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    const bf16x8_t bdh = __builtin_bit_cast(bf16x8_t, make_uint4(dh[0], dh[1], dh[2], dh[3]));
    const bf16x8_t bdl = __builtin_bit_cast(bf16x8_t, make_uint4(dl[0], dl[1], dl[2], dl[3]));
#pragma unroll
    for (int b2 = 0; b2 < D / 16; ++b2) {
      const bf16x8_t ao = ld_bf16x8(tot + (16 * b2 + l16) * L::TS + 8 * g4);
      const bf16x8_t aq = ld_bf16x8(tqt + (16 * b2 + l16) * L::TS + 8 * g4);
      accv[b2] = mfma16(ao, bph, accv[b2]);
      accv[b2] = mfma16(ao, bpl, accv[b2]);
      acck[b2] = mfma16(aq, bdh, acck[b2]);
      acck[b2] = mfma16(aq, bdl, acck[b2]);
    }
  };

  for (long long base = 0; base < nsel + nwin; base += CB) {
    const int nb = (int)min((long long)CB, nsel + nwin - base);
    __syncthreads();                                 // the previous batch is consumed
    for (int t = tid; t < CB; t += MT) {
      const long long idx = base + t;
      int id = 0;
      float4 cf = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      int2 lm = make_int2(1, 0);                     // no key
      if (t < nb) {
        if (idx < nsel) {
          const uint32_t e = eg[p0 + idx / G];
          const int r = (int)(idx % G), i = (int)(e >> 8), s2 = (int)(e & 255u);
          const float4 ps = *reinterpret_cast<const float4*>(pstat + (((bg * N + i) * (long long)K + s2) * G + r) * 4);
          id = (i << 4) | r;
          cf = make_float4(ps.x, ps.y, ps.z, 0.0f);
          lm = make_int2(0, S);
        } else {
          const long long widx = idx - nsel;
          const int i = j0 + (int)(widx / G), r = (int)(widx % G);
          const float4 ws = *reinterpret_cast<const float4*>(wstat + ((hb + r) * N + i) * 4);
          id = (i << 4) | r;
          cf = ws;
          lm = make_int2((int)(window_start(i, W, S) - j0), i - j0);
        }
      }
      did[t] = id;
      dcf[t] = cf;
      dlim[t] = lm;
    }
    __syncthreads();
    const int ntl = (nb + QT - 1) / QT;
    stage_load(0, nb);
    stage_store(0);
    __syncthreads();
    for (int tl = 0; tl < ntl; ++tl) {
      if (tl + 1 < ntl) stage_load(tl + 1, nb);
      if (kwave) compute(tl, tl & 1);
      // buffer (tl + 1) & 1 was last read in tile tl - 1, before the barrier
      // that ended it
      if (tl + 1 < ntl) stage_store((tl + 1) & 1);
      __syncthreads();
    }
  }
  if (kown) {
    const long long ro = (bg * (long long)N + j0 + kk) * D + 4 * g4;
#pragma unroll
    for (int b2 = 0; b2 < D / 16; ++b2) {
      *reinterpret_cast<float4*>(dv + ro + 16 * b2) =
          make_float4(accv[b2][0], accv[b2][1], accv[b2][2], accv[b2][3]);
      *reinterpret_cast<float4*>(dk + ro + 16 * b2) =
          make_float4(acck[b2][0], acck[b2][1], acck[b2][2], acck[b2][3]);
    }
  }
}

template <int D>
size_t cols_mf_lds() {
  return sizeof(bf16_t) * 2 * MfCol<D>::TILE + (size_t)CB * (sizeof(int) + sizeof(float4) + sizeof(int2));
}

}  // namespace

bool hils_bwd_cols_mf_ok(const HilsShape& s) {
  return s.dtype == 0 && (s.d == 64 || s.d == 128) && s.S % 16 == 0 && s.S <= 64 && s.G <= 16;
}

hipError_t hils_launch_bwd_cols_mf(const HilsShape& s, const void* q, const void* k, const void* v,
                                   const void* dout, const HilsBwdBufs& wb, float* dk, float* dv,
                                   hipStream_t st) {
  if (!hils_bwd_cols_mf_ok(s)) return hipErrorInvalidValue;
  const long long nblk = (long long)s.B * s.Hkv * s.nCc;
  if (nblk <= 0) return hipSuccess;
  const float tau = (float)s.tau;
  HilsProfScope ps_("k_bwd_cols", st);
  if (s.d == 128) {
    const size_t shm = cols_mf_lds<128>();
    hils_allow_lds((const void*)k_bwd_cols_mf<128>, shm);
    hipLaunchKernelGGL(k_bwd_cols_mf<128>, dim3((unsigned)nblk), dim3(MT), shm, st,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)dout,
                       wb.off, wb.ent, wb.pstat, wb.wstat, dk, dv, s.Hq, s.Hkv, s.G, s.N, s.S, s.W,
                       s.K, s.nC, s.nCc, tau);
  } else {
    const size_t shm = cols_mf_lds<64>();
    hils_allow_lds((const void*)k_bwd_cols_mf<64>, shm);
    hipLaunchKernelGGL(k_bwd_cols_mf<64>, dim3((unsigned)nblk), dim3(MT), shm, st,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)dout,
                       wb.off, wb.ent, wb.pstat, wb.wstat, dk, dv, s.Hq, s.Hkv, s.G, s.N, s.S, s.W,
                       s.K, s.nC, s.nCc, tau);
  }
  return hipGetLastError();
}
