// Fast-path window + selected-chunk attention with chunk-level fusion
// (bf16, d = 128, S = 64).
//
// "Hierarchical Sparse Attention Done Right", section 3 (hierarchical
// softmax): each query attends inside its chunk-aligned window and,
// independently, inside each selected chunk; the parts are mixed by a softmax
// over {s_hat_c : c selected} U {log Z_swa}.  Section 4.2 groups adjacent
// queries and loads the union of their chunks once; here one workgroup owns
// 64 (query, head) rows = 64/G adjacent queries of one KV group, walks the
// window tiles and then the sorted union of the rows' selected chunks.  Each
// chunk's K (64 x 128) and V^T (128 x 64, pre-transposed per chunk) are staged
// in LDS once and used by every wavefront whose rows selected it.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): S^T = K Q^T, so a lane holds 16 key
// logits of one (query, head) column and the per-column max/sum need only
// two cross-lane steps; P^T stays in registers as the B operand of
// O^T = V^T P^T.  Logits are in base-2 units (scale * log2 e).
// Because the fusion weights are known before a chunk is visited (the
// window's log-mass and every selected chunk's score are computed first),
// each chunk's normalised probabilities are scaled by its fusion weight and
// accumulated straight into the output accumulator.
#include "fast_common.h"
#include "hils_internal.h"

using namespace fastp;

namespace {

constexpr int NT = 256;
constexpr int KSTR = D;       // K tile row stride (elements); 16-byte parts XOR-swizzled per row

// physical 16-byte part of logical part p in K-tile row r: the rows read by one
// 16-lane group (see the key order in qk) land in 16 distinct bank groups
__device__ __forceinline__ int kswz(int r, int p) { return p ^ (((r >> 1) & 12) | (r & 3)); }
constexpr int VSTR = S + 8;   // V^T tile row stride (elements)
constexpr int MAXW = 512;     // bitmap words: chunk ids < 16384

struct ALds {
  size_t kt, vt, sel, bm, wp, ul, um, lam, total;
  __host__ __device__ ALds(int QA, int K) {
    size_t o = 0;
    kt = o;  o += (size_t)S * KSTR * 2;
    vt = o;  o += (size_t)D * VSTR * 2;
    sel = o; o += (size_t)QA * K * 4;
    bm = o;  o += (size_t)MAXW * 4;
    wp = o;  o += (size_t)MAXW * 4;
    ul = o;  o += (size_t)QA * K * 4;
    o = (o + 15) & ~(size_t)15;
    um = o;  o += (size_t)QA * K * 8;
    lam = o; o += (size_t)64 * (K + 1) * 4;   // rows padded to K+1 floats
    total = o;
  }
};

// V [B][Hkv][N][D] -> V^T per chunk [B][Hkv][nCc][D][S], zero beyond N
__global__ void __launch_bounds__(NT)
k_vt(const bf16_t* __restrict__ v, bf16_t* __restrict__ vt, int N, int nCc) {
  __shared__ bf16_t tile[S][D + 8];
  const int tid = threadIdx.x;
  const long long bgc = blockIdx.x;
  const int c = (int)(bgc % nCc);
  const long long bg = bgc / nCc;
  const bf16_t* src = v + (bg * N + (long long)c * S) * D;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int piece = tid + NT * p, row = piece / 16, part = piece % 16;
    const uint4 val = ((long long)c * S + row < N) ? ld_u4(src + (long long)row * D + part * 8)
                                                    : make_uint4(0, 0, 0, 0);
    st_u4(&tile[row][part * 8], val);
  }
  __syncthreads();
  bf16_t* dst = vt + bgc * (long long)D * S;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int piece = tid + NT * p, e = piece / 8, part = piece % 8;
    uint32_t w4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w4[t] = (uint32_t)tile[part * 8 + 2 * t][e] | ((uint32_t)tile[part * 8 + 2 * t + 1][e] << 16);
    st_u4(dst + (long long)e * S + part * 8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
  }
}

template <int G>
__global__ void __launch_bounds__(NT, 2)
k_attn_fast(const bf16_t* __restrict__ q, const bf16_t* __restrict__ qr,
            const bf16_t* __restrict__ k, const bf16_t* __restrict__ vt,
            const bf16_t* __restrict__ ksum, const float* __restrict__ bsum,
            const int32_t* __restrict__ sel, bf16_t* __restrict__ out, int Hq, int Hkv, int N,
            int W, int K, int nC, int nCc, float tau2, int nqb) {
  constexpr int QA = 64 / G;
  extern __shared__ __align__(16) unsigned char sm[];
  const ALds L(QA, K);
  bf16_t* ktile = reinterpret_cast<bf16_t*>(sm + L.kt);
  bf16_t* vtile = reinterpret_cast<bf16_t*>(sm + L.vt);
  int* sel_s = reinterpret_cast<int*>(sm + L.sel);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(sm + L.bm);
  int* wpref = reinterpret_cast<int*>(sm + L.wp);
  int* ulist = reinterpret_cast<int*>(sm + L.ul);
  unsigned long long* umask = reinterpret_cast<unsigned long long*>(sm + L.um);
  float* lam = reinterpret_cast<float*>(sm + L.lam);
  __shared__ int scan[NT];
  __shared__ int sh_nunion;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int qb = nqb - 1 - (blk % nqb);
  const int bg = blk / nqb;
  const int g = bg % Hkv;
  const long long b = bg / Hkv;
  const int i0 = qb * QA;
  const int qcount = min(QA, N - i0);
  const long long hb = b * Hq + (long long)g * G;
  const long long kvbase = (b * Hkv + g);

  // ---- selections of the block and their sorted union --------------------
  for (int t = tid; t < QA * K; t += NT) {
    const int qa = t / K;
    sel_s[t] = (qa < qcount) ? sel[(kvbase * N + i0 + qa) * K + t % K] : -1;
  }
  const int ncmax = n_cand(i0 + qcount - 1, W, S);
  const int nwords = (ncmax + 31) / 32;
  for (int t = tid; t < MAXW; t += NT) bitmap[t] = 0;
  __syncthreads();
  for (int t = tid; t < QA * K; t += NT) {
    const int c = sel_s[t];
    if (c >= 0) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  {
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    const int c0 = (w0 < nwords) ? __popc(bitmap[w0]) : 0;
    const int c1 = (w1 < nwords) ? __popc(bitmap[w1]) : 0;
    scan[tid] = c0 + c1;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int add = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int excl = scan[tid] - (c0 + c1);
    if (w0 < MAXW) wpref[w0] = excl;
    if (w1 < MAXW) wpref[w1] = excl + c0;
    if (tid == NT - 1) sh_nunion = scan[NT - 1];
  }
  __syncthreads();
  const int nunion = sh_nunion;
  for (int t = tid; t < nwords; t += NT) {
    uint32_t word = bitmap[t];
    int pos = wpref[t];
    while (word) {
      const int j = __ffs(word) - 1;
      ulist[pos++] = t * 32 + j;
      word &= word - 1;
    }
  }
  for (int t = tid; t < nunion; t += NT) umask[t] = 0ull;
  __syncthreads();
  for (int t = tid; t < QA * K; t += NT) {
    const int c = sel_s[t];
    if (c >= 0) {
      const int u = wpref[c >> 5] + __popc(bitmap[c >> 5] & ((1u << (c & 31)) - 1u));
      atomicOr(&umask[u], 1ull << (t / K));
    }
  }
  // ---- fusion logits s_hat (base 2) of every (row, selected chunk) ----------
  for (int idx = tid; idx < 64 * K; idx += NT) {
    const int r = idx / K, kx = idx % K, qa = r / G, h = r % G;
    const int li = r * (K + 1) + kx;
    const int c = (qa < qcount) ? sel_s[qa * K + kx] : -1;
    float val = -INFINITY;
    if (c >= 0) {
      const bf16_t* qp = qr + ((hb + h) * N + i0 + qa) * (long long)D;
      const bf16_t* kp = ksum + ((hb + h) * nC + c) * (long long)D;
      float acc = 0.0f;
#pragma unroll 4
      for (int e = 0; e < D; e += 8) {
        const uint4 a = ld_u4(qp + e), bb = ld_u4(kp + e);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc = fmaf(__uint_as_float(av[t] << 16), __uint_as_float(bv[t] << 16), acc);
          acc = fmaf(__uint_as_float(av[t] & 0xffff0000u), __uint_as_float(bv[t] & 0xffff0000u), acc);
        }
      }
      val = fmaf(acc, tau2, bsum[(hb + h) * nC + c] * LOG2E);
    }
    lam[li] = val;
  }
  __syncthreads();

  // ---- per-lane column: (query, head) row of this wavefront ----------------
  const int colr = 16 * w + (lane & 15);
  const int qa = colr / G, h = colr % G;
  const int lq = lane >> 4;
  const bool vcol = qa < qcount;
  const int iq = i0 + qa;
  bf16x8_t bq[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (vcol) bq[ks] = ld_bf16x8(q + ((hb + h) * N + iq) * (long long)D + 32 * ks + 8 * lq);
    else bq[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }
  const long long wlo = vcol ? window_start(iq, W, S) : 0;

  // chunk staging through registers (two chunks in flight) into one LDS tile
  // Unconditional loads (rows past N read row N-1: such keys are always masked,
  // and V^T is zero there), so no load result is ever merged or copied while
  // it is still in flight.
  auto load_chunk = [&](uint4* r, int c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 16, part = piece % 16;
      const long long t = min((long long)c * S + row, (long long)N - 1);
      r[p] = ld_u4(k + (kvbase * N + t) * D + part * 8);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 8, part = piece % 8;
      r[4 + p] = ld_u4(vt + ((kvbase * nCc + c) * D + row) * (long long)S + part * 8);
    }
  };
  auto store_chunk = [&](const uint4* r) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 16, part = piece % 16;
      st_u4(ktile + row * KSTR + kswz(row, part) * 8, r[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = tid + NT * p, row = piece / 8, part = piece % 8;
      st_u4(vtile + row * VSTR + part * 8, r[4 + p]);
    }
  };
  // S^T tile: s[kt][e] <-> key 32*(kt>>1) + 8*lq + 4*(kt&1) + e
  auto qk = [&](f32x4_t* s) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int m = lane & 15;
      const int key = 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3);
      f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a4 = mfma16(ld_bf16x8(ktile + key * KSTR + kswz(key, 4 * ks + lq) * 8), bq[ks], a4);
      s[kt] = a4;
    }
  };
  f32x4_t acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto pv = [&](const float* p) {   // p[kt*4+e]
    bf16x8_t pb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 u = make_uint4(pack_bf16x2(p[8 * kb + 0], p[8 * kb + 1]),
                                 pack_bf16x2(p[8 * kb + 2], p[8 * kb + 3]),
                                 pack_bf16x2(p[8 * kb + 4], p[8 * kb + 5]),
                                 pack_bf16x2(p[8 * kb + 6], p[8 * kb + 7]));
      pb[kb] = __builtin_bit_cast(bf16x8_t, u);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc[dt] = mfma16(ld_bf16x8(vtile + (16 * dt + (lane & 15)) * VSTR + 32 * kb + 8 * lq),
                         pb[kb], acc[dt]);
    }
  };

  // ---- one pipelined pass over the block's window tiles, then its union ------
  float m = -INFINITY, l = 0.0f;
  float M2 = 0.0f, invZ = 0.0f;
  const int cw_lo = (int)(window_start(i0, W, S) / S);
  const int cw_hi = (i0 + qcount - 1) / S;
  const int nw = cw_hi - cw_lo + 1;
  const int total = nw + nunion;
  unsigned long long wq = 0ull;   // queries with a row in this wavefront
  for (int r = 16 * w; r < 16 * w + 16; ++r) wq |= 1ull << (r / G);
  int kptr = 0;
  auto chunk_of = [&](int idx) { return idx < nw ? cw_lo + idx : ulist[idx - nw]; };

  auto window_tile = [&](int c) {
    f32x4_t s[4];
    qk(s);
    float x[16];
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long long j = (long long)c * S + 32 * (kt >> 1) + 8 * lq + 4 * (kt & 1) + e;
        const bool ok = vcol && j >= wlo && j <= iq;
        const float v2 = ok ? s[kt][e] * tau2 : -INFINITY;
        x[kt * 4 + e] = v2;
        mt = fmaxf(mt, v2);
      }
    mt = max_x32(max_x16(mt));
    // the reference m moves only when the tile's maximum passes it by more
    // than 8 (base-2 logits; always on the first finite tile), so weights
    // stay below 2^8 and the outputs are rescaled rarely; a row without a
    // finite score yet keeps m = -inf and weights 0
    const float mnew = (mt > m + 8.0f) ? mt : m;
    const float scale = (mnew == m) ? 1.0f : fast_exp2(m - mnew);   // 0 when m = -inf
    const float mref = (mnew == -INFINITY) ? 0.0f : mnew;
    float p[16];
    float ps = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) { p[t] = fast_exp2(x[t] - mref); ps += p[t]; }
    ps = sum_x32(sum_x16(ps));
    l = l * scale + ps;
    m = mnew;
    if (__ballot(scale != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= scale;
    }
    float pk[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 8; ++t) pk[8 * kb + t] = p[(2 * kb + (t >> 2)) * 4 + (t & 3)];
    pv(pk);
  };

  // chunk-level fusion weights once the window is done: softmax over
  // {s_hat_c : c selected} U {log Z_swa}
  auto fusion_setup = [&]() {
    const float logz2 = m + log2f(l);
    int kk = 0;
    M2 = logz2;
    for (int kx = 0; kx < K; ++kx) {
      const float lv = lam[colr * (K + 1) + kx];
      if (lv != -INFINITY) { M2 = fmaxf(M2, lv); ++kk; }
    }
    float Z = fast_exp2(logz2 - M2);
    for (int kx = 0; kx < kk; ++kx) Z += fast_exp2(lam[colr * (K + 1) + kx] - M2);
    invZ = 1.0f / Z;
    const float a_swa = vcol ? fast_exp2(logz2 - M2) * invZ / l : 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] *= a_swa;
  };

  auto selected_chunk = [&](int u) {
    const unsigned long long mk = umask[u];
    if (!(mk & wq)) return;
    f32x4_t s[4];
    qk(s);
    const bool here = vcol && ((mk >> qa) & 1ull);
    float x[16];
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v2 = here ? s[kt][e] * tau2 : -INFINITY;
        x[kt * 4 + e] = v2;
        mt = fmaxf(mt, v2);
      }
    mt = max_x32(max_x16(mt));
    float p[16];
    float ps = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) { p[t] = here ? fast_exp2(x[t] - mt) : 0.0f; ps += p[t]; }
    ps = sum_x32(sum_x16(ps));
    float coef = 0.0f;
    if (here) {
      coef = fast_exp2(lam[colr * (K + 1) + kptr] - M2) * invZ / ps;
      ++kptr;
    }
    float pk[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 8; ++t) pk[8 * kb + t] = p[(2 * kb + (t >> 2)) * 4 + (t & 3)] * coef;
    pv(pk);
  };

  // invariant at step idx: LDS holds chunk idx, `nxt` holds chunk idx+1 (loads
  // in flight), `far` is free and receives chunk idx+2
  // (past the end, loads repeat the last chunk and the final store is unused)
  uint4 ra[8], rb[8];
  auto step = [&](int idx, uint4* nxt, uint4* far) {
    load_chunk(far, chunk_of(min(idx + 2, total - 1)));
    if (idx < nw) {
      window_tile(cw_lo + idx);
      if (idx == nw - 1) fusion_setup();
    } else {
      selected_chunk(idx - nw);
    }
    __syncthreads();
    store_chunk(nxt);
    __syncthreads();
  };
  load_chunk(ra, chunk_of(0));
  load_chunk(rb, chunk_of(min(1, total - 1)));
  store_chunk(ra);
  __syncthreads();
  int idx = 0;
  for (; idx + 1 < total; idx += 2) {
    step(idx, rb, ra);
    step(idx + 1, ra, rb);
  }
  if (idx < total) step(idx, rb, ra);

  // ---- store ------------------------------------------------------------
  if (vcol) {
    bf16_t* op = out + ((hb + h) * N + iq) * (long long)D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint2 u = make_uint2(pack_bf16x2(acc[dt][0], acc[dt][1]), pack_bf16x2(acc[dt][2], acc[dt][3]));
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * lq) = u;
    }
  }
}

template <int G>
hipError_t launch_attn(const HilsShape& s, const void* q, const void* qr, const void* k,
                       const void* vt, const void* ksum, const float* bsum, const int32_t* sel,
                       void* out, hipStream_t st) {
  constexpr int QA = 64 / G;
  const int nqb = (s.N + QA - 1) / QA;
  const ALds L(QA, s.K);
  auto f = k_attn_fast<G>;
  hils_allow_lds((const void*)f, L.total);
  const float tau2 = (float)(s.tau * 1.4426950408889634);
  { HilsProfScope ps_("k_attn_fast", st); hipLaunchKernelGGL(f, dim3((unsigned)((long long)s.B * s.Hkv * nqb)), dim3(NT), L.total, st,
                     (const bf16_t*)q, (const bf16_t*)qr, (const bf16_t*)k, (const bf16_t*)vt,
                     (const bf16_t*)ksum, bsum, sel, (bf16_t*)out, s.Hq, s.Hkv, s.N, s.W, s.K, s.nC,
                     s.nCc, tau2, nqb); }
  return hipGetLastError();
}

}  // namespace

hipError_t hils_launch_vt(const HilsShape& s, const void* v, void* vt, hipStream_t st) {
  { HilsProfScope ps_("k_vt", st); hipLaunchKernelGGL(k_vt, dim3((unsigned)((long long)s.B * s.Hkv * s.nCc)), dim3(NT), 0, st,
                     (const bf16_t*)v, (bf16_t*)vt, s.N, s.nCc); }
  return hipGetLastError();
}

size_t hils_fast_attn_lds(int G, int K) { return ALds(64 / G, K).total; }

hipError_t hils_launch_attn_fast(const HilsShape& s, const void* q, const void* qr, const void* k,
                                 const void* vt, const void* ksum, const float* bsum,
                                 const int32_t* sel, void* out, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_attn<1>(s, q, qr, k, vt, ksum, bsum, sel, out, st);
    case 2: return launch_attn<2>(s, q, qr, k, vt, ksum, bsum, sel, out, st);
    case 4: return launch_attn<4>(s, q, qr, k, vt, ksum, bsum, sel, out, st);
  }
  return hipErrorInvalidValue;
}
