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
};

// LDS bytes of the row kernel (window logits of G heads live in LDS)
size_t hils_bwd_rows_lds(const HilsShape& s);

hipError_t hils_launch_backward(const HilsShape& s, const void* q, const void* qr, const void* k,
                                const void* v, const void* lm, const void* dout, const int32_t* sel,
                                const void* ksum, const float* bsum, float* dq, float* dqr,
                                float* dk, float* dv, float* dlm, const HilsBwdBufs& wb,
                                hipStream_t st);
