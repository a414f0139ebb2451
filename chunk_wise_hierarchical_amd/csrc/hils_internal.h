// Host-side shape record and kernel launchers (internal to libhils).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hils.h"

struct HilsShape {
  int B, N, Hq, Hkv, G, d, S, W, K;
  int dtype;   // 0 bf16, 1 fp32
  int mode;    // 0 surrogate, 1 landmark key, 2 exact
  int nC;      // floor(N/S): chunks with a landmark / summary
  int nCc;     // ceil(N/S): chunks holding tokens
  int nmax;    // |C_{N-1}|: most candidate chunks of any position
  int nwin;    // max number of S-token tiles a window spans
  double tau;  // logit scale
  int M = 1;   // decode: new tokens (queries) per sequence
};

// Lets `kernel` launch with up to `bytes` of dynamic LDS on the current
// device.  The attribute is set only when a launch needs more than was set
// before (per kernel and device); setting it on every launch has stalled the
// host's enqueueing.
void hils_allow_lds(const void* kernel, size_t bytes);

// Kernel timing (hils_profile_enable): records a HIP event pair around each launch.
struct HilsProfScope {
  HilsProfScope(const char* name, hipStream_t st);
  ~HilsProfScope();
  int slot;
  hipStream_t st;
};

// summarize.hip
hipError_t hils_launch_summarize(const HilsShape& s, const void* k, const void* lm, int c0, int c1,
                                 void* ksum, float* bsum, hipStream_t st);

// prefill_generic.hip: vector-ALU score/select and attention, any supported shape
hipError_t hils_launch_select_generic(const HilsShape& s, const void* qr, const void* k,
                                      const void* ksum, const float* bsum, int32_t* sel,
                                      float* slog, hipStream_t st);
hipError_t hils_launch_attn_generic(const HilsShape& s, const void* q, const void* k, const void* v,
                                    const int32_t* sel, const float* slog, void* out, hipStream_t st);

// fast path (bf16, d = 128, S = 64, G in {1,2,4}, K <= 64): fast_score.hip, fast_attn.hip
hipError_t hils_launch_vt(const HilsShape& s, const void* v, void* vt, hipStream_t st);
// frag: workspace of hils_score_frag_bytes(s) for k' in MFMA fragment order
hipError_t hils_launch_score_fast(const HilsShape& s, const void* qr, const void* ksum,
                                  const float* bsum, void* frag, int32_t* sel, hipStream_t st);
size_t hils_score_frag_bytes(const HilsShape& s);
hipError_t hils_launch_attn_fast(const HilsShape& s, const void* q, const void* qr, const void* k,
                                 const void* vt, const void* ksum, const float* bsum,
                                 const int32_t* sel, void* out, hipStream_t st);
size_t hils_fast_score_lds(int G, int K);

// fast_pairs.hip: prefill attention organised by selected chunk.  Buffers of
// one slice of at most qs_max queries (workspace):
struct HilsPairBufs {
  uint32_t *cnt, *loff, *toff, *cur, *tot;  // [B*Hkv*nC] x4, [4]
  uint32_t* bsum;                           // [2 * ceil(B*Hkv*nC / HILS_PAIR_SB)]
  uint2* tinfo;                             // [hils_pair_tiles_max]
  uint32_t* list;                           // [B*Hkv*qs_max*K]
  float* lam;                               // [B*Hkv*qs_max*K*G] fusion logits (base 2)
  uint16_t* part;                           // [B*Hkv*qs_max*K*G*d] bf16 per-chunk outputs
  int qs_max;
};
constexpr int HILS_PAIR_SLICE = 131072;     // queries per slice
constexpr int HILS_PAIR_TPW = 16;           // tiles per attention workgroup
constexpr int HILS_PAIR_SB = 4096;          // buckets per scan workgroup
long long hils_pair_tiles_max(const HilsShape& s, int qs);
hipError_t hils_launch_attn_pairs(const HilsShape& s, const void* q, const void* qr, const void* k,
                                  const void* vt, const void* ksum, const float* bsum,
                                  const int32_t* sel, void* out, const HilsPairBufs& pb,
                                  hipStream_t st);
size_t hils_fast_attn_lds(int G, int K);
constexpr int HILS_FAST_NCMAX = 16384;   // chunk ids the fast attention bitmap covers

// decode.hip
hipError_t hils_launch_decode(const HilsShape& s, const void* q, const void* qr, const void* k,
                              const void* v, const int32_t* seqlen, const void* ksum,
                              const float* bsum, void* out, int32_t* sel, float* scores,
                              uint32_t* keys, uint2* cand, int32_t* uni, float* slog, float* part,
                              float* lsep,
                              const int32_t* page_table, int max_pages, int num_pages,
                              hipStream_t st);
// Decode selection: one workgroup per (sequence, KV group, query) takes the
// whole candidate list when there are enough such rows to fill the chip and
// the list's keys fit in LDS.  Otherwise P partitions of `span` chunks each
// find their own top-K, then one merge of the P * K candidates; the merge
// keeps its P * K keys and ids in LDS, so P * K stays within
// HILS_DEC_MERGE_MAX.
constexpr int HILS_DEC_SEL_SPAN = 4096;
constexpr int HILS_DEC_MERGE_MAX = 8192;
constexpr int HILS_DEC_SEL_ROWS_WHOLE = 128;
constexpr int HILS_DEC_SEL_LDS_KEYS = 24576;
// Multi-token blocks take the union attention when M K <= HILS_DEC_UNION_IDS
// and the cache has at most HILS_DEC_UNION_CHUNKS chunks (an LDS bitmap over
// chunk ids); other blocks attend token by token.
constexpr int HILS_DEC_UNION_IDS = HILS_MAX_DECODE_QUERIES * 64;
constexpr int HILS_DEC_UNION_CHUNKS = 65536;
inline bool hils_dec_union(const HilsShape& s) {
  return s.dtype == 0 && s.d == 128 && s.S == 64 && (s.G == 1 || s.G == 2 || s.G == 4) && s.M > 1 &&
         s.M * s.K <= HILS_DEC_UNION_IDS && s.nC <= HILS_DEC_UNION_CHUNKS;
}
// per (sequence, KV group): the union's size and its ids ascending (M K + 1
// ints), then per union element and token the token's slot of that chunk (M K
// x M bytes, -1 where the token did not select it)
inline size_t hils_dec_union_bytes(const HilsShape& s) {
  if (!hils_dec_union(s)) return 8;
  const size_t bg = (size_t)s.B * s.Hkv, mk = (size_t)s.M * s.K;
  return bg * (mk + 1) * 4 + bg * mk * s.M;
}
inline void hils_dec_select_split(const HilsShape& s, int& P, int& span) {
  const long long nm = s.nmax > 0 ? s.nmax : 1;
  const long long rows = (long long)s.B * s.Hkv * s.M;
  if (rows >= HILS_DEC_SEL_ROWS_WHOLE && nm <= HILS_DEC_SEL_LDS_KEYS) {
    P = 1;
    span = (int)nm;
    return;
  }
  span = HILS_DEC_SEL_SPAN;
  P = (int)((nm + span - 1) / span);
  if (P > 1 && (long long)P * s.K > HILS_DEC_MERGE_MAX) {
    const long long pmax = HILS_DEC_MERGE_MAX / s.K;             // >= 64 (K <= 128)
    span = (int)(((nm + pmax - 1) / pmax + 1023) / 1024 * 1024);
    P = (int)((nm + span - 1) / span);
  }
}
hipError_t hils_launch_summarize_paged(const HilsShape& s, const void* k_pages, const void* lm_pages,
                                       const int32_t* pages, int npages_listed, int num_pages,
                                       void* ksum_pages, float* bsum_pages, hipStream_t st);

// chunk rows per decode scoring workgroup (one (max, sum exp) partial each)
constexpr int HILS_DEC_SCORE_ROWS = 256;
// the decode scoring grid puts (sequence, query head) on grid dimension y
constexpr long long HILS_DEC_MAX_ROWS_Y = 65535;

// maximum candidates the generic select kernel keeps in LDS
constexpr int HILS_GENERIC_NMAX = 8192;
