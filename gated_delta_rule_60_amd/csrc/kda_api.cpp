// kda_api.cpp -- the C ABI declared in include/kda.h: host-side argument
// validation (before any HIP call), launch-shape selection and error text.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <string>

#include "kda_launch.hpp"

namespace kda {

// Compute units of the current device, queried once per device (relaxed
// atomics: concurrent callers may both query and store the same value).
hipError_t device_cus(int* cus) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (*cus < 1) *cus = 1;
    if (dev >= 0 && dev < 64) cached[dev].store(*cus, std::memory_order_relaxed);
    return hipSuccess;
}

int device_cus_or_default() {
    int cus = 0;
    if (device_cus(&cus) != hipSuccess) {
        (void)hipGetLastError();  // the failed query must not surface as a later call's error
        return kDefaultCUs;
    }
    return cus;
}

}  // namespace kda

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

bool supported_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_dims(int32_t d_k, int32_t d_v, kda_dtype dtype) {
    if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32)
        return fail(KDA_ERR_UNSUPPORTED, "dtype must be KDA_DTYPE_BF16 or KDA_DTYPE_F32");
    if (!supported_dim(d_k) || !supported_dim(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "d_k and d_v must each be 32, 64 or 128 (got " +
                                             std::to_string(d_k) + ", " + std::to_string(d_v) + ")");
    return KDA_OK;
}

kda_status hip_fail(hipError_t e, const char* what) {
    return fail(KDA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace kda {
void set_last_error(const char* msg) { g_last_error = msg; }
}  // namespace kda

extern "C" {

int32_t kda_version(void) { return KDA_VERSION; }

const char* kda_status_string(kda_status status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported size or dtype";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
        default: return "unknown kda_status";
    }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status kda_prefill_plan(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                            int32_t compute_units, int32_t* v_split, size_t* workspace_bytes) {
    g_last_error.clear();
    if (N < 1 || H < 1 || T_tot < 0) return fail(KDA_ERR_INVALID_ARG, "need N >= 1, H >= 1 and T_tot >= 0");
    if (compute_units < 0) return fail(KDA_ERR_INVALID_ARG, "compute_units must be >= 0");
    if (!v_split || !workspace_bytes) return fail(KDA_ERR_INVALID_ARG, "v_split and workspace_bytes must not be NULL");
    const kda_status ds = check_dims(d_k, d_v, dtype);
    if (ds != KDA_OK) return ds;
    const int cus = compute_units > 0 ? compute_units : kda::device_cus_or_default();
    *v_split = kda::default_v_split(N, T_tot, H, d_k, d_v, dtype == KDA_DTYPE_BF16, cus);
    *workspace_bytes = kda::prefill_workspace_bytes(N, T_tot, H, d_k, d_v, dtype == KDA_DTYPE_BF16, cus);
    return KDA_OK;
}

size_t kda_prefill_workspace_size(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype dtype) {
    int32_t split = 0;
    size_t bytes = 0;
    const std::string keep = g_last_error;  // a query leaves the last error text alone
    const kda_status st = kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, 0, &split, &bytes);
    g_last_error = keep;
    return st == KDA_OK ? bytes : 0;
}

int32_t kda_prefill_default_split(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype dtype) {
    int32_t split = 0;
    size_t bytes = 0;
    const std::string keep = g_last_error;
    const kda_status st = kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, 0, &split, &bytes);
    g_last_error = keep;
    return st == KDA_OK ? split : 0;
}

size_t kda_prefill_workspace_size_ex(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                     kda_dtype dtype, uint32_t flags) {
    if ((flags & ~static_cast<uint32_t>(KDA_PREFILL_SCALAR_GATE | KDA_PREFILL_WIDE_DECAY | KDA_PREFILL_ANY_DECAY)) != 0 ||
        ((flags & KDA_PREFILL_WIDE_DECAY) && (flags & KDA_PREFILL_ANY_DECAY)))
        return 0;
    if (N < 1 || H < 1 || T_tot < 0 || !supported_dim(d_k) || !supported_dim(d_v) ||
        (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32))
        return 0;
    if (flags & KDA_PREFILL_ANY_DECAY) return kda::any_map_bytes(N, T_tot, H);
    return kda_prefill_workspace_size(N, T_tot, H, d_k, d_v, dtype);
}

size_t kda_prefill_backward_workspace_size_ex(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                              kda_dtype dtype, uint32_t flags) {
    if (N < 1 || H < 1 || T_tot < 0 || !supported_dim(d_k) || !supported_dim(d_v) ||
        (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32))
        return 0;
    if (flags & KDA_PREFILL_ANY_DECAY) return kda::prefill_bwd_workspace_bytes(N, T_tot, H, d_k, d_v);
    return kda::prefill_bwd_chunk_workspace_bytes(N, T_tot, H, d_k, d_v, dtype == KDA_DTYPE_BF16);
}

size_t kda_prefill_backward_workspace_size(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                           kda_dtype dtype) {
    return kda_prefill_backward_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, 0u);
}

}  // extern "C"

namespace {

// Shared by both backward entry points; scalar_gate: log_alpha and
// d_log_alpha are [T_tot, H] (4-byte aligned).
kda_status backward_impl(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const float* S0, const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                         int32_t d_k, int32_t d_v, kda_dtype dtype, const void* d_o, const float* d_S_T, float* d_q,
                         float* d_k_out, float* d_v_out, float* d_log_alpha, float* d_beta, float* d_S0,
                         void* workspace, size_t workspace_bytes, void* stream, uint32_t flags) {
    g_last_error.clear();
    if ((flags & ~static_cast<uint32_t>(KDA_PREFILL_SCALAR_GATE | KDA_PREFILL_ANY_DECAY)) != 0)
        return fail(KDA_ERR_INVALID_ARG, "unknown or unsupported bits in flags (the backward takes "
                                         "KDA_PREFILL_SCALAR_GATE and KDA_PREFILL_ANY_DECAY)");
    const bool scalar_gate = (flags & KDA_PREFILL_SCALAR_GATE) != 0;
    if (N < 1 || H < 1 || T_tot < 0)
        return fail(KDA_ERR_INVALID_ARG, "need N >= 1, H >= 1 and T_tot >= 0");
    const kda_status ds = check_dims(d_k, d_v, dtype);
    if (ds != KDA_OK) return ds;
    if (!cu_seqlens || !d_S0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens and d_S0 must not be NULL");
    if (T_tot > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !d_q || !d_k_out || !d_v_out ||
                      !d_log_alpha || !d_beta))
        return fail(KDA_ERR_INVALID_ARG,
                    "inputs, d_o and every token gradient must not be NULL when T_tot > 0");
    if (T_tot > INT32_MAX) return fail(KDA_ERR_INVALID_ARG, "T_tot must fit in int32 (cu_seqlens is int32)");
    if (static_cast<int64_t>(N) * H * (d_v / 8) > (int64_t{1} << 22))
        return fail(KDA_ERR_INVALID_ARG, "N * H too large");
    if (!(flags & KDA_PREFILL_ANY_DECAY)) {  // the chunked path runs the prefill kernel
        if (T_tot * H * static_cast<int64_t>(d_k > d_v ? d_k : d_v) > INT32_MAX)
            return fail(KDA_ERR_INVALID_ARG, "q, k, v, d_o and log_alpha must each hold fewer than 2^31 elements");
        if (static_cast<int64_t>(H) * (d_k > d_v ? d_k : d_v) > (int64_t{1} << 20))
            return fail(KDA_ERR_INVALID_ARG, "H * max(d_k, d_v) must not exceed 2^20");
    }
    const void* ptrs[] = {q, k, v, scalar_gate ? nullptr : log_alpha, d_o, S0, d_S_T, d_q, d_k_out, d_v_out,
                          scalar_gate ? nullptr : d_log_alpha, d_S0};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const void* ptrs4[] = {d_beta, scalar_gate ? log_alpha : nullptr, scalar_gate ? d_log_alpha : nullptr};
    for (const void* p : ptrs4)
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u) != 0)
            return fail(KDA_ERR_INVALID_ARG, scalar_gate ? "d_beta, log_alpha and d_log_alpha must be 4-byte aligned"
                                                         : "d_beta must be 4-byte aligned");
    const size_t ws_need = kda_prefill_backward_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, flags);
    if (workspace_bytes < ws_need)
        return fail(KDA_ERR_INVALID_ARG, "workspace smaller than kda_prefill_backward_workspace_size");
    if (!workspace) return fail(KDA_ERR_INVALID_ARG, "workspace must not be NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(KDA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    kda::BackwardArgs a{q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, N, T_tot, H, d_k, d_v,
                        dtype == KDA_DTYPE_BF16, d_q, d_k_out, d_v_out, d_log_alpha, d_beta, d_S0,
                        workspace, stream, scalar_gate};
    (void)hipGetLastError();  // report only this launch's status
    const hipError_t e = (flags & KDA_PREFILL_ANY_DECAY) ? kda::launch_prefill_bwd(a) : kda::launch_prefill_bwd_chunk(a);
    if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                                int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                const void* d_o, const float* d_S_T, float* d_q, float* d_k_out,
                                float* d_v_out, float* d_log_alpha, float* d_beta, float* d_S0,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o, d_S_T, d_q,
                         d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace, workspace_bytes, stream, 0u);
}

kda_status kda_prefill_backward_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                                   const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                                   int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                   const void* d_o, const float* d_S_T, float* d_q, float* d_k_out,
                                   float* d_v_out, float* d_log_alpha, float* d_beta, float* d_S0,
                                   void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    return backward_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o, d_S_T, d_q,
                         d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace, workspace_bytes, stream, flags);
}

kda_status gdn_prefill_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                                const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                                int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                const void* d_o, const float* d_S_T, float* d_q, float* d_k_out,
                                float* d_v_out, float* d_log_alpha, float* d_beta, float* d_S0,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o, d_S_T, d_q,
                         d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace, workspace_bytes, stream,
                         KDA_PREFILL_SCALAR_GATE);
}

}  // extern "C"

namespace {

// Shared by every prefill entry point.  KDA_PREFILL_SCALAR_GATE changes only
// the shape of log_alpha ([T_tot, H], 4-byte aligned); KDA_PREFILL_ANY_DECAY
// selects the chunked kernel over chunk lists when the workspace holds them,
// the token-recurrent kernel otherwise; KDA_PREFILL_WIDE_DECAY selects the
// wide-decay kernel variant.
kda_status prefill_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                        int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                        float* S_T, void* workspace, size_t workspace_bytes, int32_t v_split,
                        uint32_t flags, void* stream) {
    g_last_error.clear();
    if ((flags & ~static_cast<uint32_t>(KDA_PREFILL_SCALAR_GATE | KDA_PREFILL_WIDE_DECAY | KDA_PREFILL_ANY_DECAY)) != 0)
        return fail(KDA_ERR_INVALID_ARG, "unknown bits in flags");
    if ((flags & KDA_PREFILL_WIDE_DECAY) && (flags & KDA_PREFILL_ANY_DECAY))
        return fail(KDA_ERR_INVALID_ARG, "KDA_PREFILL_WIDE_DECAY and KDA_PREFILL_ANY_DECAY exclude each other");
    const bool scalar_gate = (flags & KDA_PREFILL_SCALAR_GATE) != 0;
    if (N < 1 || H < 1 || T_tot < 0)
        return fail(KDA_ERR_INVALID_ARG, "need N >= 1, H >= 1 and T_tot >= 0");
    const kda_status ds = check_dims(d_k, d_v, dtype);
    if (ds != KDA_OK) return ds;
    if (!cu_seqlens || !S_T) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens and S_T must not be NULL");
    if (T_tot > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, log_alpha, beta and o must not be NULL when T_tot > 0");
    if (T_tot > INT32_MAX) return fail(KDA_ERR_INVALID_ARG, "T_tot must fit in int32 (cu_seqlens is int32)");
    if (T_tot * H * static_cast<int64_t>(d_k > d_v ? d_k : d_v) > INT32_MAX)
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, o and log_alpha must each hold fewer than 2^31 elements");
    if (static_cast<int64_t>(H) * (d_k > d_v ? d_k : d_v) > (int64_t{1} << 20))
        return fail(KDA_ERR_INVALID_ARG, "H * max(d_k, d_v) must not exceed 2^20");
    const void* ptrs[] = {q, k, v, scalar_gate ? nullptr : log_alpha, o, S0, S_T};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (scalar_gate && log_alpha && (reinterpret_cast<uintptr_t>(log_alpha) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARG, "log_alpha must be 4-byte aligned");
    const bool bf16 = dtype == KDA_DTYPE_BF16;
    const int cus = kda::device_cus_or_default();
    const bool any_decay = (flags & KDA_PREFILL_ANY_DECAY) != 0;
    // any decay: the chunk lists when the workspace holds them (else the
    // token-recurrent kernel, which needs none)
    const bool mapped = any_decay && workspace && workspace_bytes >= kda::any_map_bytes(N, T_tot, H);
    const size_t ws_need = any_decay ? 0 : kda::prefill_workspace_bytes(N, T_tot, H, d_k, d_v, bf16, cus);
    if (workspace_bytes < ws_need)
        return fail(KDA_ERR_INVALID_ARG, "workspace smaller than kda_prefill_workspace_size");
    if (ws_need > 0 && !workspace) return fail(KDA_ERR_INVALID_ARG, "workspace must not be NULL");
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(KDA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (v_split == 0) v_split = kda::default_v_split(N, T_tot, H, d_k, d_v, bf16, cus);
    if (!(v_split == 1 || v_split == 2 || v_split == 4 || v_split == 8) || d_v / v_split < 16)
        return fail(KDA_ERR_INVALID_ARG, "v_split must be 1, 2, 4 or 8 with d_v / v_split >= 16");
    // Workgroups of the prefill kernel: (sequence or segment, head, value
    // slice[, identity run]); each has at most 1024 work-items.
    const bool segmented = kda::prefill_segmented(N, T_tot, H, d_k, d_v, cus);
    const int64_t units = segmented ? kda::seg_units_max(N, T_tot) : N;
    const int64_t grid = units * H * v_split * (segmented ? 2 : 1);
    if (grid > (int64_t{1} << 22)) return fail(KDA_ERR_INVALID_ARG, "N * H * v_split too large");

    kda::PrefillArgs a{q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                       bf16, o, S_T, v_split, stream, workspace, cus, scalar_gate,
                       (flags & KDA_PREFILL_WIDE_DECAY) != 0, any_decay};
    (void)hipGetLastError();  // report only this launch's status
    const hipError_t e = mapped ? kda::launch_prefill_mapped(a)
                                : (any_decay ? kda::launch_prefill_recurrent(a) : kda::launch_prefill(a));
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return KDA_OK;
}

kda_status decode_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, float* S, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                       kda_dtype dtype, void* o, void* stream, bool scalar_gate) {
    g_last_error.clear();
    if (N < 1 || H < 1) return fail(KDA_ERR_INVALID_ARG, "need N >= 1 and H >= 1");
    const kda_status ds = check_dims(d_k, d_v, dtype);
    if (ds != KDA_OK) return ds;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o)
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, log_alpha, beta, S and o must not be NULL");
    const void* ptrs[] = {q, k, v, scalar_gate ? nullptr : log_alpha, S, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (scalar_gate && (reinterpret_cast<uintptr_t>(log_alpha) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARG, "log_alpha must be 4-byte aligned");
    if (static_cast<int64_t>(N) * H > INT32_MAX) return fail(KDA_ERR_INVALID_ARG, "N * H too large");
    kda::DecodeArgs a{q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype == KDA_DTYPE_BF16, o, stream,
                      scalar_gate};
    (void)hipGetLastError();  // report only this launch's status
    const hipError_t e = kda::launch_decode(a);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_split(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, const int32_t* cu_seqlens,
                             int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                             kda_dtype dtype, void* o, float* S_T, void* workspace,
                             size_t workspace_bytes, int32_t v_split, void* stream) {
    return prefill_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        workspace, workspace_bytes, v_split, 0, stream);
}

kda_status kda_prefill_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                          int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                          float* S_T, void* workspace, size_t workspace_bytes, int32_t v_split,
                          uint32_t flags, void* stream) {
    return prefill_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        workspace, workspace_bytes, v_split, flags, stream);
}

kda_status kda_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                       int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                       float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        workspace, workspace_bytes, 0, 0, stream);
}

kda_status gdn_prefill_split(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, const int32_t* cu_seqlens,
                             int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                             kda_dtype dtype, void* o, float* S_T, void* workspace,
                             size_t workspace_bytes, int32_t v_split, void* stream) {
    return prefill_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        workspace, workspace_bytes, v_split, KDA_PREFILL_SCALAR_GATE, stream);
}

kda_status gdn_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, const float* S0, const int32_t* cu_seqlens, int32_t N,
                       int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                       float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        workspace, workspace_bytes, 0, KDA_PREFILL_SCALAR_GATE, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, float* S, int32_t N, int32_t H, int32_t d_k,
                           int32_t d_v, kda_dtype dtype, void* o, void* stream) {
    return decode_impl(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream, false);
}

kda_status gdn_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, float* S, int32_t N, int32_t H, int32_t d_k,
                           int32_t d_v, kda_dtype dtype, void* o, void* stream) {
    return decode_impl(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream, true);
}

}  // extern "C"
