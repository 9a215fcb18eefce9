// qmm_noalloc.hip -- qmm_w4a16_g128 for callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid allocation): the split's
// bf16 partial planes live in a static device array of this library instead of a workspace
// the caller passes.
//
// `scratch` is one file-scope device array; every GPU the library runs on holds its own copy
// at its own address until the process ends. In host code the array's name stands for a host
// shadow, not a device address, so the host never hands it to a kernel: the first call on a
// device looks up that device's address once (hipGetSymbolAddress, with the device current)
// and every call passes that address to the existing entry point as its workspace. After the
// look-up a call allocates nothing.
//
// Every call on one GPU shares that GPU's array: the partial planes of a call are completely
// written by its split kernel before its reduce reads them, so nothing has to start at zero
// and the array keeps the last call's planes; two calls that overlap in time on one GPU (on
// different streams, or from different threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmm.h"

static __device__ __align__(256) unsigned char scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMM_ERR_HIP;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QMM_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QMM_OK;
}

}  // namespace

extern "C" int qmm_w4a16_g128_noalloc(const void *A, const void *Wq, const void *scale, const void *bias, void *C,
                                      int M, int N, int K, int s, void *stream)
{
    void *ws = nullptr;
    int rc = scratch_address(&ws);
    if (rc != QMM_OK) return rc;
    // The split the call runs and its planes' size, with the existing entry point's checks
    // of the shape (argument, alignment and split errors are its own).
    if (s < 0) return QMM_ERR_ARG;
    size_t need = 0;
    if (s == 0) {
        qmm_plan plan;
        rc = qmm_splitk_plan(M, N, K, 128, nullptr, &plan);
        if (rc != QMM_OK) return rc;
        need = plan.workspace_bytes;
    } else if (s > 1 && M > 0 && N > 0) {
        need = (size_t)2 * (size_t)s * (size_t)M * (size_t)N;
    }
    if (need > (size_t)QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_SCRATCH;
    return qmm_w4a16_g128(A, Wq, scale, bias, C, M, N, K, s, need ? ws : nullptr,
                          need ? (size_t)QMM_NOALLOC_SCRATCH_BYTES : 0, stream);
}
