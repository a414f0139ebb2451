// C ABI of libhils: argument validation, workspace layout and kernel dispatch.
// See include/hils.h for the contract of every entry point.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/hils.h"
#include "hils_bwd.h"
#include "hils_internal.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int n_cand_host(long long i, int W, int S) {
  long long t = i - W + 1;
  long long q = (t >= 0) ? t / S : -((-t + S - 1) / S);
  long long l = q * S;
  return l > 0 ? (int)(l / S) : 0;
}

// Validates a configuration and fills the shape record.
hils_status make_shape(const hils_cfg* c, HilsShape& s) {
  if (!c) return HILS_E_ARG;
  if (c->B < 1 || c->N < 1 || c->Hq < 1 || c->Hkv < 1 || c->d < 1 || c->S < 1 || c->W < 1 ||
      c->K < 1)
    return HILS_E_ARG;
  if (c->Hq % c->Hkv != 0) return HILS_E_ARG;
  if (c->dtype != HILS_BF16 && c->dtype != HILS_F32) return HILS_E_ARG;
  if (c->mode < HILS_SCORE_SURROGATE || c->mode > HILS_SCORE_MEAN_POOL) return HILS_E_ARG;
  if (!(c->scale >= 0.0f) || isinf(c->scale)) return HILS_E_ARG;
  if (c->d > 256 || c->S > 64 || c->K > 128 || c->Hq / c->Hkv > 8) return HILS_E_UNSUPPORTED;
  const long long elems = (long long)c->B * c->Hq * c->N * c->d;
  if (elems <= 0 || elems > (1LL << 40)) return HILS_E_UNSUPPORTED;
  s.B = c->B; s.N = c->N; s.Hq = c->Hq; s.Hkv = c->Hkv; s.G = c->Hq / c->Hkv;
  s.d = c->d; s.S = c->S; s.W = c->W; s.K = c->K;
  s.dtype = c->dtype; s.mode = c->mode;
  s.nC = c->N / c->S;
  s.nCc = (c->N + c->S - 1) / c->S;
  s.nmax = n_cand_host((long long)c->N - 1, c->W, c->S);
  s.nwin = (c->W + c->S - 1 + c->S - 1) / c->S;   // ceil((W + S - 1) / S)
  s.tau = (c->scale == 0.0f) ? 1.0 / sqrt((double)c->d) : (double)c->scale;
  return HILS_OK;
}

inline size_t esize(const HilsShape& s) { return s.dtype == HILS_BF16 ? 2 : 4; }

// The MFMA fast path covers bf16, d = 128, S = 64, G in {1, 2, 4}, K <= 64.
bool fast_eligible(const HilsShape& s, uint32_t flags) {
  if (flags & HILS_FLAG_GENERIC) return false;
  if (s.mode == HILS_SCORE_EXACT) return false;   // test mode: generic kernels only
  if (s.dtype != HILS_BF16 || s.d != 128 || s.S != 64 || s.K > 64) return false;
  if (!(s.G == 1 || s.G == 2 || s.G == 4)) return false;
  if (s.nC > HILS_FAST_NCMAX) return false;
  if ((long long)s.B * s.Hkv * s.nC >= (1LL << 25)) return false;   // bucket id in 25 bits
  return true;
}

inline bool pair_path(const HilsShape& s, uint32_t flags, bool fast) {
  return fast && !(flags & HILS_FLAG_UNION);
}

struct PrefillLayout {
  size_t ks, bs, sel, slog, vt, kf, total;
  // per-chunk bucket path
  size_t cnt, loff, toff, cur, tot, bsum, tinfo, list, lam, part;
  int qs_max;
};
// generic path: summaries, selection, fusion logits; fast path: summaries,
// selection, the per-chunk transposed V and k' in MFMA fragment order (fusion
// logits are recomputed in the attention kernel)
PrefillLayout prefill_layout(const HilsShape& s, bool fast, bool pairs) {
  PrefillLayout L{};
  size_t off = 0;
  L.ks = off;   off += align_up((size_t)s.B * s.Hq * s.nC * s.d * esize(s));
  L.bs = off;   off += align_up((size_t)s.B * s.Hq * s.nC * 4);
  L.sel = off;  off += align_up((size_t)s.B * s.Hkv * s.N * s.K * 4);
  if (fast) {
    L.slog = 0;
    L.vt = off; off += align_up((size_t)s.B * s.Hkv * s.nCc * s.d * s.S * 2);
    L.kf = off; off += align_up(hils_score_frag_bytes(s));
    if (pairs) {
      const int qs = s.N < HILS_PAIR_SLICE ? s.N : HILS_PAIR_SLICE;
      const size_t F = (size_t)s.B * s.Hkv * s.nC;
      const size_t P = (size_t)s.B * s.Hkv * qs * s.K;   // pair slots of a slice
      L.qs_max = qs;
      L.cnt = off;   off += align_up(F * 4);
      L.loff = off;  off += align_up(F * 4);
      L.toff = off;  off += align_up(F * 4);
      L.cur = off;   off += align_up(F * 4);
      L.tot = off;   off += align_up(16);
      L.bsum = off;  off += align_up((F + HILS_PAIR_SB - 1) / HILS_PAIR_SB * 8);
      L.tinfo = off; off += align_up((size_t)hils_pair_tiles_max(s, qs) * 8);
      L.list = off;  off += align_up(P * 4);
      L.lam = off;   off += align_up(P * s.G * 4);
      L.part = off;  off += align_up(P * s.G * s.d * 2);
    }
  } else {
    L.slog = off; off += align_up((size_t)s.B * s.Hq * s.N * s.K * 4);
    L.vt = 0;
  }
  L.total = off;
  return L;
}

struct DecodeLayout {
  size_t scores, keys, cand, uni, slog, sel, part, lsep, total;
};
DecodeLayout decode_layout(const HilsShape& s) {
  DecodeLayout L{};
  const size_t nm = (size_t)(s.nmax > 0 ? s.nmax : 1);
  size_t off = 0;
  const size_t BM = (size_t)s.B * s.M;          // (sequence, query) rows
  L.scores = off; off += align_up(BM * s.Hq * nm * 4);
  L.keys = off;   off += align_up(BM * s.Hkv * nm * 4);
  int P = 1, span = 1;
  hils_dec_select_split(s, P, span);
  L.cand = off;   off += align_up(P > 1 ? BM * s.Hkv * (size_t)P * s.K * 8 : 8);
  L.uni = off;    off += align_up(hils_dec_union_bytes(s));
  L.slog = off;   off += align_up(BM * s.Hq * s.K * 4);
  L.sel = off;    off += align_up(BM * s.Hkv * s.K * 4);
  L.part = off;   off += align_up(BM * s.Hq * (s.K + s.nwin) * (s.d + 2) * 4);
  L.lsep = off;   off += align_up(BM * s.Hq * ((nm + HILS_DEC_SCORE_ROWS - 1) / HILS_DEC_SCORE_ROWS) * 8);
  L.total = off;
  return L;
}

struct BwdLayout {
  size_t ks, bs, off, ent, pstat, wstat, wpart, dqp, srng, order, sitems, lcnt, total;
};
BwdLayout bwd_layout(const HilsShape& s) {
  BwdLayout L{};
  const size_t BG = (size_t)s.B * s.Hkv;
  size_t off = 0;
  L.ks = off;    off += align_up((size_t)s.B * s.Hq * s.nC * s.d * (s.dtype == HILS_BF16 ? 2 : 4));
  L.bs = off;    off += align_up((size_t)s.B * s.Hq * s.nC * 4);
  L.off = off;   off += align_up(BG * (s.nC + 1) * 4);
  L.ent = off;   off += align_up(BG * s.N * s.K * 4);
  L.pstat = off; off += align_up(BG * s.N * s.K * s.G * 16);
  L.wstat = off; off += align_up((size_t)s.B * s.Hq * s.N * 16);
  const bool mf = hils_bwd_mf_ok(s);
  L.wpart = off; off += align_up(mf ? hils_bwd_mf_wpart_bytes(s) : 0);
  L.dqp = off;   off += align_up(mf ? hils_bwd_mf_dqp_bytes(s) : 0);
  L.srng = off;  off += align_up(mf ? hils_bwd_mf_srng_bytes(s) : 0);
  L.order = off; off += align_up(mf ? hils_bwd_mf_order_bytes(s) : 0);
  L.sitems = off; off += align_up(mf ? hils_bwd_mf_sitems_bytes(s) : 0);
  L.lcnt = off;  off += align_up(hils_bwd_list_count_bytes(s));
  L.total = off;
  return L;
}

// shapes the backward kernels take
hils_status bwd_supported(const HilsShape& s) {
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_UNSUPPORTED;
  // the column pass gives each thread d / 8 elements of a row, read as whole
  // 16-byte vectors (8 bf16 or 4 fp32 elements)
  if (s.d > 128 || s.d % (s.dtype == HILS_BF16 ? 64 : 32) != 0) return HILS_E_UNSUPPORTED;
  if (s.S > 64 || s.G > 8 || s.K > 128) return HILS_E_UNSUPPORTED;
  if (s.N >= (1 << 24)) return HILS_E_UNSUPPORTED;
  if ((long long)s.B * s.Hkv * s.N * s.K >= (1LL << 31)) return HILS_E_UNSUPPORTED;
  if ((long long)s.B * s.Hkv * s.N >= (1LL << 31)) return HILS_E_UNSUPPORTED;
  if (hils_bwd_rows_lds(s) > 160 * 1024) return HILS_E_UNSUPPORTED;
  if ((size_t)s.nC * 4 > 160 * 1024) return HILS_E_UNSUPPORTED;
  return HILS_OK;
}

inline hils_status hip_status(hipError_t e) { return e == hipSuccess ? HILS_OK : HILS_E_HIP; }

// ---- scratch of the allocation-free decode entry point --------------------
// Device addresses of `scratch` (defined below, outside this namespace), one
// per device: each GPU holds its own copy of the array at its own address,
// which only hipGetSymbolAddress with that device current can tell.  In host
// code the array's name is a host-side stand-in and is never passed to a
// kernel or a copy.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hils_status scratch_ptr_current_device(void** out);

// ---- kernel timing record ------------------------------------------------
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::atomic<int> g_prof_on{0};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;        // recorded this period
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

// Scratch of hils_decode_noalloc: file scope, 256-byte aligned, the size the
// header states; zero-initialised once at load and never freed.
static __device__ __align__(256) unsigned char scratch[HILS_NOALLOC_SCRATCH_BYTES];

namespace {
hils_status scratch_ptr_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HILS_E_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HILS_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HILS_OK;
}
}  // namespace

namespace {
std::mutex g_lds_mu;
std::map<std::pair<const void*, int>, size_t> g_lds_set;   // (kernel, device) -> bytes allowed
}  // namespace

void hils_allow_lds(const void* kernel, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lk(g_lds_mu);
  size_t& have = g_lds_set[std::make_pair(kernel, dev)];
  if (bytes <= have) return;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess)
    have = bytes;
}

HilsProfScope::HilsProfScope(const char* name, hipStream_t s) : slot(-1), st(s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r{name, prof_event(), prof_event()};
  if (!r.a || !r.b) return;
  hipEventRecord(r.a, st);
  slot = (int)g_prof.size();
  g_prof.push_back(r);
}

HilsProfScope::~HilsProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot < (int)g_prof.size()) hipEventRecord(g_prof[slot].b, st);
}

extern "C" {

const char* hils_strerror(hils_status st) {
  switch (st) {
    case HILS_OK: return "ok";
    case HILS_E_ARG: return "invalid argument";
    case HILS_E_UNSUPPORTED: return "unsupported configuration";
    case HILS_E_WORKSPACE: return "workspace too small";
    case HILS_E_HIP: return "HIP runtime or launch error";
  }
  return "unknown status";
}

int hils_abi_version(void) { return HILS_ABI_VERSION; }

void hils_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on.store(on ? 1 : 0);
  if (!on) {
    for (auto& r : g_prof) { hipEventDestroy(r.a); hipEventDestroy(r.b); }
    g_prof.clear();
    for (auto e : g_prof_pool) hipEventDestroy(e);
    g_prof_pool.clear();
  }
}

int hils_profile_read(const char** names, float* ms, int cap) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int n = (int)g_prof.size();
  for (int i = 0; i < n; ++i) {
    if (i < cap) {
      float t = 0.0f;
      if (hipEventElapsedTime(&t, g_prof[i].a, g_prof[i].b) != hipSuccess) t = -1.0f;
      if (names) names[i] = g_prof[i].name;
      if (ms) ms[i] = t;
    }
    g_prof_pool.push_back(g_prof[i].a);
    g_prof_pool.push_back(g_prof[i].b);
  }
  g_prof.clear();
  return n;
}

size_t hils_workspace_bytes(const hils_cfg* cfg, int is_decode) {
  HilsShape s;
  if (make_shape(cfg, s) != HILS_OK) return 0;
  return is_decode ? decode_layout(s).total : prefill_layout(s, fast_eligible(s, cfg->flags),
                                    pair_path(s, cfg->flags, fast_eligible(s, cfg->flags))).total;
}

hils_status hils_summarize(const hils_cfg* cfg, const void* k, const void* lm_q, int32_t c0,
                           int32_t c1, void* k_sum, float* b_sum, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_ARG;   // exact mode has no summaries
  if (c0 < 0 || c1 < c0 || c1 > s.nC) return HILS_E_ARG;
  if (c1 == c0) return HILS_OK;
  const bool need_lm = s.mode != HILS_SCORE_MEAN_POOL;
  if (!k || (need_lm && !lm_q) || !k_sum || !b_sum) return HILS_E_ARG;
  if (!aligned16(k) || (lm_q && !aligned16(lm_q)) || !aligned16(k_sum) || !aligned16(b_sum))
    return HILS_E_ARG;
  if ((long long)s.B * s.Hq * (c1 - c0) >= (1LL << 31)) return HILS_E_UNSUPPORTED;
  return hip_status(hils_launch_summarize(s, k, lm_q, c0, c1, k_sum, b_sum, (hipStream_t)stream));
}

hils_status hils_prefill(const hils_cfg* cfg, const void* q, const void* q_route, const void* k,
                         const void* v, const void* lm_q, void* out, int32_t* sel, void* k_sum,
                         float* b_sum, void* ws, size_t ws_bytes, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  const bool exact = s.mode == HILS_SCORE_EXACT;
  if (!q || !k || !v || !out) return HILS_E_ARG;
  if (s.nC > 0 && !lm_q && s.mode != HILS_SCORE_MEAN_POOL && !exact) return HILS_E_ARG;
  if ((k_sum == nullptr) != (b_sum == nullptr)) return HILS_E_ARG;
  const void* ptrs[] = {q, q_route, k, v, lm_q, out, sel, k_sum, b_sum, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  const bool fast = fast_eligible(s, cfg->flags);
  if (!fast && s.nmax > HILS_GENERIC_NMAX) return HILS_E_UNSUPPORTED;
  if ((long long)s.B * s.Hkv * s.N >= (1LL << 31)) return HILS_E_UNSUPPORTED;
  const bool pairs = pair_path(s, cfg->flags, fast);
  const PrefillLayout L = prefill_layout(s, fast, pairs);
  if (ws_bytes < L.total || (L.total > 0 && !ws)) return HILS_E_WORKSPACE;
  char* w = static_cast<char*>(ws);
  void* ks = k_sum ? k_sum : (void*)(w + L.ks);
  float* bs = b_sum ? b_sum : (float*)(w + L.bs);
  int32_t* sl = sel ? sel : (int32_t*)(w + L.sel);
  // exact mode scores chunks with the token query and needs no summaries
  const void* qr = exact ? q : (q_route ? q_route : q);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!exact) {
    e = hils_launch_summarize(s, k, lm_q, 0, s.nC, ks, bs, st);
    if (e != hipSuccess) return HILS_E_HIP;
  }
  if (fast) {
    void* vt = (void*)(w + L.vt);
    e = hils_launch_vt(s, v, vt, st);
    if (e != hipSuccess) return HILS_E_HIP;
    e = hils_launch_score_fast(s, qr, ks, bs, w + L.kf, sl, st);
    if (e != hipSuccess) return HILS_E_HIP;
    if (!pairs) return hip_status(hils_launch_attn_fast(s, q, qr, k, vt, ks, bs, sl, out, st));
    HilsPairBufs pb{};
    pb.cnt = (uint32_t*)(w + L.cnt);
    pb.loff = (uint32_t*)(w + L.loff);
    pb.toff = (uint32_t*)(w + L.toff);
    pb.cur = (uint32_t*)(w + L.cur);
    pb.tot = (uint32_t*)(w + L.tot);
    pb.bsum = (uint32_t*)(w + L.bsum);
    pb.tinfo = (uint2*)(w + L.tinfo);
    pb.list = (uint32_t*)(w + L.list);
    pb.lam = (float*)(w + L.lam);
    pb.part = (uint16_t*)(w + L.part);
    pb.qs_max = L.qs_max;
    return hip_status(hils_launch_attn_pairs(s, q, qr, k, vt, ks, bs, sl, out, pb, st));
  }
  float* slog = (float*)(w + L.slog);
  e = hils_launch_select_generic(s, qr, k, ks, bs, sl, slog, st);
  if (e != hipSuccess) return HILS_E_HIP;
  e = hils_launch_attn_generic(s, q, k, v, sl, slog, out, st);
  return hip_status(e);
}

hils_status hils_decode(const hils_cfg* cfg, const void* q, const void* q_route,
                        const void* k_cache, const void* v_cache, const int32_t* seqlen,
                        const void* k_sum, const float* b_sum, void* out, int32_t* sel, void* ws,
                        size_t ws_bytes, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !seqlen || !out) return HILS_E_ARG;
  if (s.nmax > 0 && (!k_sum || !b_sum)) return HILS_E_ARG;
  const void* ptrs[] = {q, q_route, k_cache, v_cache, seqlen, k_sum, b_sum, out, sel, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  if (s.d % (s.dtype == HILS_BF16 ? 8 : 4) != 0) return HILS_E_UNSUPPORTED;
  const DecodeLayout L = decode_layout(s);
  if (ws_bytes < L.total || (L.total > 0 && !ws)) return HILS_E_WORKSPACE;
  char* w = static_cast<char*>(ws);
  int32_t* sl = sel ? sel : (int32_t*)(w + L.sel);
  const void* qr = q_route ? q_route : q;
  if ((long long)s.B * s.Hq > HILS_DEC_MAX_ROWS_Y) return HILS_E_UNSUPPORTED;
  return hip_status(hils_launch_decode(s, q, qr, k_cache, v_cache, seqlen, k_sum, b_sum, out, sl,
                                       (float*)(w + L.scores), (uint32_t*)(w + L.keys),
                                       (uint2*)(w + L.cand), (int32_t*)(w + L.uni),
                                       (float*)(w + L.slog), (float*)(w + L.part),
                                       (float*)(w + L.lsep), nullptr, 0, 0, (hipStream_t)stream));
}

hils_status hils_decode_noalloc(const hils_cfg* cfg, const void* q, const void* q_route,
                                const void* k_cache, const void* v_cache, const int32_t* seqlen,
                                const void* k_sum, const float* b_sum, void* out, int32_t* sel,
                                void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !seqlen || !out) return HILS_E_ARG;
  // the scratch must hold this configuration's decode workspace
  const size_t need = decode_layout(s).total;
  if (need > HILS_NOALLOC_SCRATCH_BYTES) return HILS_E_WORKSPACE;
  void* ws = nullptr;
  r = scratch_ptr_current_device(&ws);
  if (r != HILS_OK) return r;
  // the regular entry point validates the rest and enqueues the same kernels
  return hils_decode(cfg, q, q_route, k_cache, v_cache, seqlen, k_sum, b_sum, out, sel, ws,
                     HILS_NOALLOC_SCRATCH_BYTES, stream);
}

size_t hils_decode_multi_workspace_bytes(const hils_cfg* cfg, int32_t M) {
  HilsShape s;
  if (make_shape(cfg, s) != HILS_OK || M < 1 || M > HILS_MAX_DECODE_QUERIES) return 0;
  s.M = M;
  return decode_layout(s).total;
}

hils_status hils_decode_multi(const hils_cfg* cfg, int32_t M, const void* q, const void* q_route,
                              const void* k_cache, const void* v_cache, const int32_t* seqlen,
                              const void* k_sum, const float* b_sum, void* out, int32_t* sel,
                              void* ws, size_t ws_bytes, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (M < 1 || M > s.N) return HILS_E_ARG;
  if (M > HILS_MAX_DECODE_QUERIES) return HILS_E_UNSUPPORTED;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_UNSUPPORTED;
  s.M = M;
  if ((long long)s.B * s.Hkv * M >= (1LL << 31) || (long long)s.B * s.Hq * M >= (1LL << 31))
    return HILS_E_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !seqlen || !out) return HILS_E_ARG;
  if (s.nmax > 0 && (!k_sum || !b_sum)) return HILS_E_ARG;
  const void* ptrs[] = {q, q_route, k_cache, v_cache, seqlen, k_sum, b_sum, out, sel, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  if (s.d % (s.dtype == HILS_BF16 ? 8 : 4) != 0) return HILS_E_UNSUPPORTED;
  const DecodeLayout L = decode_layout(s);
  if (ws_bytes < L.total || (L.total > 0 && !ws)) return HILS_E_WORKSPACE;
  char* w = static_cast<char*>(ws);
  int32_t* sl = sel ? sel : (int32_t*)(w + L.sel);
  const void* qr = q_route ? q_route : q;
  if ((long long)s.B * s.Hq > HILS_DEC_MAX_ROWS_Y) return HILS_E_UNSUPPORTED;
  return hip_status(hils_launch_decode(s, q, qr, k_cache, v_cache, seqlen, k_sum, b_sum, out, sl,
                                       (float*)(w + L.scores), (uint32_t*)(w + L.keys),
                                       (uint2*)(w + L.cand), (int32_t*)(w + L.uni),
                                       (float*)(w + L.slog), (float*)(w + L.part),
                                       (float*)(w + L.lsep), nullptr, 0, 0, (hipStream_t)stream));
}

size_t hils_prefill_backward_workspace_bytes(const hils_cfg* cfg) {
  HilsShape s;
  if (make_shape(cfg, s) != HILS_OK || bwd_supported(s) != HILS_OK) return 0;
  return bwd_layout(s).total;
}

hils_status hils_prefill_backward(const hils_cfg* cfg, const void* q, const void* q_route,
                                  const void* k, const void* v, const void* lm_q, const void* dout,
                                  const int32_t* sel, const void* k_sum, const float* b_sum,
                                  float* dq, float* dq_route, float* dk, float* dv, float* dlm,
                                  void* ws, size_t ws_bytes, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  r = bwd_supported(s);
  if (r != HILS_OK) return r;
  const bool need_lm = s.mode != HILS_SCORE_MEAN_POOL;
  if (!q || !k || !v || !dout || !sel || !dq || !dk || !dv) return HILS_E_ARG;
  if (s.nC > 0 && need_lm && (!lm_q || !dlm)) return HILS_E_ARG;
  if ((q_route == nullptr) != (dq_route == nullptr)) return HILS_E_ARG;
  if ((k_sum == nullptr) != (b_sum == nullptr)) return HILS_E_ARG;
  const void* ptrs[] = {q, q_route, k, v, lm_q, dout, sel, k_sum, b_sum, dq, dq_route, dk, dv, dlm, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  const BwdLayout L = bwd_layout(s);
  if (ws_bytes < L.total || !ws) return HILS_E_WORKSPACE;
  char* w = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  const void* ks = k_sum;
  const float* bs = b_sum;
  if (!k_sum && s.nC > 0) {
    hipError_t e = hils_launch_summarize(s, k, lm_q, 0, s.nC, w + L.ks, (float*)(w + L.bs), st);
    if (e != hipSuccess) return HILS_E_HIP;
    ks = w + L.ks;
    bs = (const float*)(w + L.bs);
  }
  const bool mf = hils_bwd_mf_ok(s);
  HilsBwdBufs wb{(uint32_t*)(w + L.off), (uint32_t*)(w + L.ent), (float*)(w + L.pstat),
                 (float*)(w + L.wstat), mf ? (float*)(w + L.wpart) : nullptr,
                 mf ? (float*)(w + L.dqp) : nullptr,
                 mf && hils_bwd_mf_srng_bytes(s) ? (uint32_t*)(w + L.srng) : nullptr,
                 mf ? (uint32_t*)(w + L.order) : nullptr,
                 mf ? (uint2*)(w + L.sitems) : nullptr,
                 mf ? (uint32_t*)(w + L.sitems + hils_bwd_mf_sitems_bytes(s) - 16) : nullptr,
                 hils_bwd_list_count_bytes(s) ? (uint32_t*)(w + L.lcnt) : nullptr};
  return hip_status(hils_launch_backward(s, q, q_route ? q_route : q, k, v, lm_q, dout, sel, ks, bs,
                                         dq, dq_route, dk, dv, dlm, wb, st));
}

hils_status hils_summarize_paged(const hils_cfg* cfg, const void* k_pages, const void* lm_pages,
                                 const int32_t* pages, int32_t npages, int32_t num_pages,
                                 void* k_sum_pages, float* b_sum_pages, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_ARG;
  if (npages < 0 || num_pages < 1) return HILS_E_ARG;
  if (npages == 0) return HILS_OK;
  const bool need_lm = s.mode != HILS_SCORE_MEAN_POOL;
  if (!k_pages || (need_lm && !lm_pages) || !pages || !k_sum_pages || !b_sum_pages)
    return HILS_E_ARG;
  const void* ptrs[] = {k_pages, lm_pages, pages, k_sum_pages, b_sum_pages};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  if ((long long)npages * s.Hq >= (1LL << 31)) return HILS_E_UNSUPPORTED;
  return hip_status(hils_launch_summarize_paged(s, k_pages, lm_pages, pages, npages, num_pages,
                                                k_sum_pages, b_sum_pages, (hipStream_t)stream));
}

hils_status hils_decode_paged(const hils_cfg* cfg, const void* q, const void* q_route,
                              const void* k_pages, const void* v_pages, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seqlen,
                              const void* k_sum_pages, const float* b_sum_pages, void* out,
                              int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  HilsShape s;
  hils_status r = make_shape(cfg, s);
  if (r != HILS_OK) return r;
  if (s.mode == HILS_SCORE_EXACT) return HILS_E_UNSUPPORTED;
  if (num_pages < 1 || max_pages < 1 || (long long)max_pages * s.S < s.N) return HILS_E_ARG;
  if (!q || !k_pages || !v_pages || !page_table || !seqlen || !out) return HILS_E_ARG;
  if (s.nmax > 0 && (!k_sum_pages || !b_sum_pages)) return HILS_E_ARG;
  const void* ptrs[] = {q, q_route, k_pages, v_pages, page_table, seqlen, k_sum_pages, b_sum_pages,
                        out, sel, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HILS_E_ARG;
  if (s.d % (s.dtype == HILS_BF16 ? 8 : 4) != 0) return HILS_E_UNSUPPORTED;
  if ((long long)num_pages * s.Hq * s.d >= (1LL << 40)) return HILS_E_UNSUPPORTED;
  const DecodeLayout L = decode_layout(s);
  if (ws_bytes < L.total || (L.total > 0 && !ws)) return HILS_E_WORKSPACE;
  char* w = static_cast<char*>(ws);
  int32_t* sl = sel ? sel : (int32_t*)(w + L.sel);
  const void* qr = q_route ? q_route : q;
  if ((long long)s.B * s.Hq > HILS_DEC_MAX_ROWS_Y) return HILS_E_UNSUPPORTED;
  return hip_status(hils_launch_decode(s, q, qr, k_pages, v_pages, seqlen, k_sum_pages, b_sum_pages,
                                       out, sl, (float*)(w + L.scores), (uint32_t*)(w + L.keys),
                                       (uint2*)(w + L.cand), (int32_t*)(w + L.uni),
                                       (float*)(w + L.slog), (float*)(w + L.part),
                                       (float*)(w + L.lsep), page_table, max_pages, num_pages,
                                       (hipStream_t)stream));
}

}  // extern "C"
