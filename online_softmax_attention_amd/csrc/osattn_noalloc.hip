// Backward entry point for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid allocation): osattn_bwd_noalloc runs the
// same kernels as osattn_bwd with the workspace taken from a file-scope
// device array instead of a caller buffer.  Declared in osattn.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/osattn.h"
#include "api_internal.h"

namespace {

// The backward's workspace for every call on a device: per-row statistics and
// split partial sums (32 MiB covers causal N=4096 H=16 D=128, whose plan needs
// under 1 MiB, and the f32 SQ=8192 SK=2048 D=64 backward, 24 MiB).  Every GPU
// the library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = OSATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == ((size_t)32 << 20), "the header states 32 MiB");
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on each device, found once per device with that
// device current.  In host code the array's name is only a stand-in for the
// symbol, never a device address: kernels get these pointers.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_ptr[kMaxDevices];
std::mutex g_init;

int scratch_ptr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return osattn::set_error(OSATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return osattn::set_error(OSATTN_ERR_UNSUPPORTED, "device index %d is above %d", dev,
                                 kMaxDevices - 1);
    void *p = g_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_init);
        p = g_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return osattn::set_error(OSATTN_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                                         hipGetErrorString(e));
            g_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return OSATTN_OK;
}

}  // namespace

extern "C" {

int osattn_bwd_noalloc(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
                       const void *q, const void *k, const void *v, const void *o,
                       const void *d_o, int64_t q_stride_h, int64_t q_stride_n,
                       int64_t kv_stride_h, int64_t kv_stride_n, int64_t o_stride_h,
                       int64_t o_stride_n, const float *m, const float *l, float scale,
                       int causal, const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
                       void *dq, void *dk, void *dv, void *stream) {
    const int st = osattn::bwd_check_args(dtype, o_dtype, H, n_q, n_k, d, q, k, v, o, d_o,
                                          q_stride_h, q_stride_n, kv_stride_h, kv_stride_n,
                                          o_stride_h, o_stride_n, m, l, scale, causal,
                                          cu_seqlens, num_seqs, max_seqlen, dq, dk, dv);
    if (st != OSATTN_OK) return st;
    const size_t need = osattn_bwd_workspace_bytes(dtype, H, n_q, n_k, d, causal, cu_seqlens,
                                                   num_seqs, max_seqlen);
    if (need > kScratchBytes)
        return osattn::set_error(OSATTN_ERR_WORKSPACE,
                                 "this backward needs %zu bytes of scratch, above the static "
                                 "maximum of %zu; call osattn_bwd with a workspace",
                                 need, kScratchBytes);
    void *ws = nullptr;
    const int sp = scratch_ptr(&ws);
    if (sp != OSATTN_OK) return sp;
    return osattn_bwd(dtype, o_dtype, H, n_q, n_k, d, q, k, v, o, d_o, q_stride_h, q_stride_n,
                      kv_stride_h, kv_stride_n, o_stride_h, o_stride_n, m, l, scale, causal,
                      cu_seqlens, num_seqs, max_seqlen, dq, dk, dv, ws, kScratchBytes, stream);
}

}  // extern "C"
