// Allocation-free chunked forward: loglin_fwd_chunked with its workspace in a
// static device array owned by the library, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Declared in include/loglin.h.
//
// The array `scratch` exists once per GPU the library runs on (it is part of
// the code object loaded on that device) and lives until the process ends.
// Host code never passes the array's name to a kernel: on the first call on a
// device, with that device current, hipGetSymbolAddress gives the device
// address of that device's copy, which is kept per device and used from then
// on.  The forward's kernels write every part of the workspace they read
// before reading it, so nothing in the array needs clearing between calls.
#include "loglin.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace loglin {
// error reporting of the C ABI (loglin_api.cpp): sets the calling thread's
// error text and returns the status
loglin_status api_fail(loglin_status s, const char* fmt, ...);
}  // namespace loglin

namespace {

constexpr size_t kScratchBytes = LOGLIN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's copy of `scratch` (nullptr on error,
// with the status in *st and the error text set).
void* device_scratch(loglin_status* st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *st = loglin::api_fail(LOGLIN_EHIP, "loglin_fwd_chunked_noalloc: hipGetDevice: %s",
                               hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *st = loglin::api_fail(LOGLIN_EUNSUPPORTED,
                               "loglin_fwd_chunked_noalloc: device %d (at most %d devices)", dev,
                               kMaxDevices);
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev]) {
        *st = loglin::api_fail(LOGLIN_EHIP,
                               "loglin_fwd_chunked_noalloc: address of the scratch array on "
                               "device %d: %s",
                               dev, hipGetErrorString(g_scratch_err[dev]));
        return nullptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

loglin_status loglin_fwd_chunked_noalloc(const void* q, const void* k, const void* v,
                                         const float* log_decay, const float* lambda, float* out,
                                         int B, int H, int T, int dk, int dv, int L, int C,
                                         loglin_dtype in_dtype, void* stream) {
    const size_t need = loglin_fwd_workspace_bytes(B, H, T, dk, dv, C, in_dtype);
    if (need == (size_t)-1) {
        // sizes or dtype the forward rejects: let it report them (it checks
        // them before anything else and enqueues nothing)
        return loglin_fwd_chunked(q, k, v, log_decay, lambda, out, B, H, T, dk, dv, L, C,
                                  in_dtype, nullptr, 0, stream);
    }
    if (need > kScratchBytes)
        return loglin::api_fail(LOGLIN_EUNSUPPORTED,
                                "loglin_fwd_chunked_noalloc: these sizes need %zu bytes of "
                                "workspace; the allocation-free forward holds %zu",
                                need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        loglin_status st = LOGLIN_OK;
        ws = device_scratch(&st);
        if (!ws) return st;
    }
    return loglin_fwd_chunked(q, k, v, log_decay, lambda, out, B, H, T, dk, dv, L, C, in_dtype,
                              ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
