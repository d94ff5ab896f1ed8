// kda_noalloc.hip -- kda_prefill_noalloc: the prefill of include/kda.h for
// callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation).  It is kda_prefill
// with the segmented path's workspace (the segment plan, the identity runs'
// outputs and the per-segment states) taken from a fixed device array of
// this library instead of a caller's buffer.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kda.h"
#include "kda_launch.hpp"

namespace {

// The fixed workspace.  Each device the library runs on holds its own copy
// for the life of the process.  In host code the array's name is only a
// host-side stand-in: its device address comes from hipGetSymbolAddress,
// looked up once per device and kept in g_scratch.
constexpr size_t kScratchBytes = KDA_PREFILL_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
hipError_t scratch_address(void** out) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
    });
    *out = g_scratch[dev];
    return g_scratch_status[dev];
}

}  // namespace

extern "C" kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                          const float* beta, const float* S0, const int32_t* cu_seqlens,
                                          int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                          kda_dtype dtype, void* o, float* S_T, void* stream) {
    int32_t split = 0;
    size_t need = 0;
    const kda_status st = kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, 0, &split, &need);
    if (st != KDA_OK) return st;
    if (need > kScratchBytes) {
        const std::string msg = "kda_prefill_noalloc: these sizes need " + std::to_string(need) +
                                " bytes of workspace; the fixed workspace holds " + std::to_string(kScratchBytes) +
                                " (use kda_prefill with a caller workspace)";
        kda::set_last_error(msg.c_str());
        return KDA_ERR_INVALID_ARG;
    }
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess || ws == nullptr) {
            const std::string msg = std::string("kda_prefill_noalloc: device address of the fixed workspace: ") +
                                    hipGetErrorString(e);
            kda::set_last_error(msg.c_str());
            return KDA_ERR_HIP;
        }
    }
    return kda_prefill_ex(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T, ws,
                          need > 0 ? kScratchBytes : 0, 0, 0u, stream);
}
