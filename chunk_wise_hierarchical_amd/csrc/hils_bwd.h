// Prefill backward (backward.hip): launcher and workspace buffers (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hils_internal.h"

struct HilsBwdBufs {
  uint32_t* off;    // [B*Hkv][nC+1] start of each chunk's list of selecting pairs
  uint32_t* ent;    // [B*Hkv][N*K]  pairs (query << 8 | slot), query order per chunk
  float* pstat;     // [B*Hkv*N][K][G][4] alpha, log-normaliser, g = dout.o, d s_hat
  float* wstat;     // [B*Hq*N][4]        the same for the window (d log Z_swa last)
  // matrix-core backward only (else null):
  // (QS = queries per slice, hils_bwd_mf_slice)
  float* wpart;     // [B*Hq*QS][nwin][4]  window partials per chunk: max, sum exp, sum exp dout.v
  float* dqp;       // [B*Hq*QS][K + nwin][d] dq partial per selected slot and window chunk
  uint32_t* srng;   // [B*Hkv*nC][2] each list's part in the slice (several slices only)
  uint32_t* order;  // [B*Hkv*nCc]    the gradient pass's work items, heaviest first
  uint2* sitems;    // the stats pass's (item, part) entries, heaviest first
  uint32_t* nsi;    // [1]            their number
  // list kernels over several workgroups per (sequence, KV group) (else null):
  uint32_t* lcnt;   // [B*Hkv][16 P][nC] per sub-range counts, then cursors
};

// workgroups per (sequence, KV group) of the list kernels, and their counts buffer
int hils_bwd_list_parts(const HilsShape& s);
size_t hils_bwd_list_count_bytes(const HilsShape& s);

// LDS bytes of the row kernel (window logits of G heads live in LDS)
size_t hils_bwd_rows_lds(const HilsShape& s);

hipError_t hils_launch_backward(const HilsShape& s, const void* q, const void* qr, const void* k,
                                const void* v, const void* lm, const void* dout, const int32_t* sel,
                                const void* ksum, const float* bsum, float* dq, float* dqr,
                                float* dk, float* dv, float* dlm, const HilsBwdBufs& wb,
                                hipStream_t st);

// Matrix-core backward (backward_mf.hip) for bf16 inputs with d in {64, 128}
// and S a multiple of 16: per-chunk statistics, per-row fusion gradients,
// per-chunk dk, dv and dq partials, per-row dq.  The selection lists come
// before it and the summaries' share of dk and dlm after it.
// It runs in query slices [qa, qa + QS) (one for most shapes) whose partials
// fit 4 GiB; dk, dv accumulate over the slices.
bool hils_bwd_mf_ok(const HilsShape& s);
int hils_bwd_mf_slice(const HilsShape& s);
size_t hils_bwd_mf_wpart_bytes(const HilsShape& s);
size_t hils_bwd_mf_dqp_bytes(const HilsShape& s);
size_t hils_bwd_mf_srng_bytes(const HilsShape& s);
size_t hils_bwd_mf_order_bytes(const HilsShape& s);
size_t hils_bwd_mf_sitems_bytes(const HilsShape& s);
hipError_t hils_launch_backward_mf(const HilsShape& s, const void* q, const void* qr, const void* k,
                                   const void* v, const void* dout, const int32_t* sel,
                                   const void* ksum, const float* bsum, float* dq, float* dqr,
                                   float* dk, float* dv, const HilsBwdBufs& wb, hipStream_t st);
