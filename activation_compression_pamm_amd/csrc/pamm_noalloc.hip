// pamm_noalloc.hip -- pamm_wgrad_noalloc: the weight-gradient call for
// callers that cannot allocate device memory (code under stream capture,
// serving loops, harnesses that forbid allocation).
//
// Its workspace is `scratch`, a file-scope device array of
// PAMM_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs on holds its own
// copy from module load until the process ends.  In host code the array's
// name is only a host-side stand-in; its device address is looked up once
// per device with hipGetSymbolAddress (with that device current) and kept,
// and only that address is ever handed to kernels.
#include <mutex>

#include "pamm.h"
#include "pamm_kernels.hpp"

static __device__ __align__(256) unsigned char scratch[PAMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr on failure.
void* scratch_address(int* status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = PAMM_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *status = PAMM_ERR_HIP;
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

int pamm_wgrad_noalloc(const void* C, const int32_t* f, const float* alpha, int64_t n, int64_t k, int64_t d,
                       const void* dY, int64_t d_out, int64_t lddy, int dtype, float* dW, int64_t lddw,
                       int accumulate, int transpose_out, void* stream) {
    // every argument, then the size, before any device query: a problem
    // whose workspace exceeds the array is refused with nothing enqueued
    const int st = pamm::wgrad_check(C, f, alpha, n, k, d, dY, d_out, lddy, dtype, dW, lddw, transpose_out);
    if (st != PAMM_OK) return st;
    const size_t need = pamm_wgrad_workspace_size(n, k, d, d_out, dtype);
    if (need > (size_t)PAMM_NOALLOC_SCRATCH_BYTES) return PAMM_ERR_TOO_LARGE;
    int status = PAMM_OK;
    void* ws = scratch_address(&status);
    if (!ws) return status;
    // every part of the workspace that pamm_wgrad's kernels read is written
    // earlier in the same call, so the array needs no clearing between calls
    return pamm_wgrad(C, f, alpha, n, k, d, dY, d_out, lddy, dtype, dW, lddw, accumulate, transpose_out, ws,
                      (size_t)PAMM_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
