// kda_launch.hpp -- internal host interface between the C ABI layer and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S0;  // may be null
    const int32_t* cu_seqlens;
    int32_t N;
    int64_t T_tot;
    int32_t H, d_k, d_v;
    bool bf16;
    void* o;
    float* S_T;
    int32_t v_split;  // 1, 2, 4, 8; d_v / v_split >= 16
    void* stream;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    float* S;
    int32_t N, H, d_k, d_v;
    bool bf16;
    void* o;
    void* stream;
};

hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

// Launch shape kda_prefill picks for these sizes (see kda_prefill.hip).
int32_t default_v_split(int32_t N, int32_t H, int32_t d_k, int32_t d_v, bool bf16);

}  // namespace kda
