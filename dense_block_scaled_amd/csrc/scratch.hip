// scratch.hip -- gemm_nvfp4_fp8_noalloc: the FP8-rate NVFP4 GEMM for callers
// that cannot allocate device memory.  Its requantisation workspace is a
// static device array of this file instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "dbs.h"
#include "launch.h"

namespace {

// The workspace.  Every GPU the library runs on holds its own copy from the
// first call on that GPU until the process ends.  In host code the name
// stands for a host-side shadow, not for device memory: only its device
// address, looked up below, may reach a kernel or a copy.
constexpr size_t kScratchBytes = DBS_NOALLOC_WORKSPACE_BYTES;
static __device__ __attribute__((used)) __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];      // device address of `scratch` per device, null until looked up

// The current device's copy of the array (looked up on the first call on
// that device, with the device current).
dbs_status scratch_of_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        char msg[256];
        std::snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
        dbs::set_error(msg);
        return DBS_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        dbs::set_error("device index out of range");
        return DBS_EHIP;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[256];
            std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            dbs::set_error(msg);
            return DBS_EHIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DBS_OK;
}

}  // namespace

extern "C" {

dbs_status gemm_nvfp4_fp8_noalloc(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB,
                                  float tB, void *D, int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb,
                                  hipStream_t stream)
{
    dbs_status st = static_cast<dbs_status>(dbs::nvfp4_fp8_check(A, sA, B, sB, D, M, N, K, la, lb));
    if (st != DBS_OK) return st;
    const int64_t need = dbs::nvfp4_fp8_workspace_bytes(M, N, K);
    if (need > (int64_t)kScratchBytes) {
        char msg[256];
        std::snprintf(msg, sizeof(msg),
                      "gemm_nvfp4_fp8_noalloc: this M, N, K needs %lld workspace bytes, above the static %zu; "
                      "call gemm_nvfp4_fp8 with a caller workspace",
                      (long long)need, kScratchBytes);
        dbs::set_error(msg);
        return DBS_EINVAL;
    }
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != DBS_OK) return st;
    return static_cast<dbs_status>(dbs::nvfp4_fp8_run(A, sA, tA, B, sB, tB, D, M, N, K, ws, kScratchBytes, stream));
}

}  // extern "C"
