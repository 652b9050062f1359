// Host-side helpers of the C ABI shared between its source files.
#pragma once

#include <stdint.h>

namespace osattn {

// Records the thread-local text osattn_last_error_message() returns; returns status.
int set_error(int status, const char *fmt, ...);

// Every host check of osattn_bwd that does not involve the workspace:
// OSATTN_OK, or the failing status with the error text set.
int bwd_check_args(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d, const void *q,
                   const void *k, const void *v, const void *o, const void *d_o,
                   int64_t q_stride_h, int64_t q_stride_n, int64_t kv_stride_h,
                   int64_t kv_stride_n, int64_t o_stride_h, int64_t o_stride_n, const float *m,
                   const float *l, float scale, int causal, const int32_t *cu_seqlens,
                   int num_seqs, int max_seqlen, void *dq, void *dk, void *dv);

}  // namespace osattn
