// kda_decode.hip -- fused single-token KDA step for gfx950.
//
// One workgroup per (sequence, head).  For one token the update rule of
// "Kimi Linear：让长上下文大模型真正实用的线性注意力架构", section 三.5, with
// per-channel decay (section 三.1), is evaluated as
//
//     S' = Diag(alpha) S          u = S'^T k        w = S'^T q
//     e  = beta (v - u)           S_new = S' + k e^T
//     o  = S_new^T q = w + (k . q) e
//
// so the state is read from HBM once, kept in registers, and written once.
// The kernel is bound by HBM bandwidth: 8 d_k d_v bytes of state traffic
// against about 7 d_k d_v flops.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <bool BF16, int DK, int DV>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const typename Elem<BF16>::G* __restrict__ q, const typename Elem<BF16>::G* __restrict__ k,
    const typename Elem<BF16>::G* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, float* __restrict__ S, int H,
    typename Elem<BF16>::G* __restrict__ o) {
    using T = Elem<BF16>;
    constexpr int NT = 256;
    constexpr int CQ = DV / 4;     // float4 column groups per state row
    constexpr int NRG = NT / CQ;   // row groups
    constexpr int RPT = DK / NRG;  // rows per thread: row = rg + NRG * r
    static_assert(NT % CQ == 0 && DK % NRG == 0, "decode thread map");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_u[NRG][DV], s_w[NRG][DV], s_kq[NRG];
    __shared__ float s_e[DV];

    const int pair = blockIdx.x;  // n * H + h
    const int tid = threadIdx.x;
    const int cq = tid % CQ;
    const int rg = tid / CQ;
    float* Sp = S + static_cast<size_t>(pair) * DK * DV;

    // Issue the state loads first; they dominate the traffic.
    float4 st[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        st[r] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(rg + NRG * r) * DV + 4 * cq);

    const size_t tk = static_cast<size_t>(pair) * DK;
    for (int i = tid; i < DK; i += NT) {
        s_k[i] = T::to_f32(k[tk + i]);
        s_q[i] = T::to_f32(q[tk + i]);
        s_a[i] = exp_e(log_alpha[tk + i]);
    }
    __syncthreads();

    float u[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = rg + NRG * r;
        const float a = s_a[row], kk = s_k[row], qq = s_q[row];
        st[r].x *= a;
        st[r].y *= a;
        st[r].z *= a;
        st[r].w *= a;
        u[0] += kk * st[r].x;
        u[1] += kk * st[r].y;
        u[2] += kk * st[r].z;
        u[3] += kk * st[r].w;
        w[0] += qq * st[r].x;
        w[1] += qq * st[r].y;
        w[2] += qq * st[r].z;
        w[3] += qq * st[r].w;
        kq += kk * qq;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        s_u[rg][4 * cq + c] = u[c];
        s_w[rg][4 * cq + c] = w[c];
    }
    if (cq == 0) s_kq[rg] = kq;
    __syncthreads();

    if (tid < DV) {
        float ut = 0.f, wt = 0.f, kqt = 0.f;
#pragma unroll
        for (int p = 0; p < NRG; ++p) {
            ut += s_u[p][tid];
            wt += s_w[p][tid];
            kqt += s_kq[p];
        }
        const size_t tv = static_cast<size_t>(pair) * DV + tid;
        const float e = beta[pair] * (T::to_f32(v[tv]) - ut);
        s_e[tid] = e;
        const float ov = wt + kqt * e;
        if constexpr (BF16) {
            o[tv] = f32_to_bf16(ov);
        } else {
            o[tv] = ov;
        }
    }
    __syncthreads();

    const float e0 = s_e[4 * cq], e1 = s_e[4 * cq + 1], e2 = s_e[4 * cq + 2], e3 = s_e[4 * cq + 3];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = rg + NRG * r;
        const float kk = s_k[row];
        float4 x = st[r];
        x.x += kk * e0;
        x.y += kk * e1;
        x.z += kk * e2;
        x.w += kk * e3;
        *reinterpret_cast<float4*>(Sp + static_cast<size_t>(row) * DV + 4 * cq) = x;
    }
}

template <bool BF16, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    using G = typename Elem<BF16>::G;
    hipLaunchKernelGGL((decode_step_kernel<BF16, DK, DV>), dim3(static_cast<unsigned>(a.N) * a.H),
                       dim3(256), 0, static_cast<hipStream_t>(a.stream),
                       static_cast<const G*>(a.q), static_cast<const G*>(a.k),
                       static_cast<const G*>(a.v), a.log_alpha, a.beta, a.S, a.H,
                       static_cast<G*>(a.o));
    return hipGetLastError();
}

template <bool BF16, int DK>
static hipError_t launch_decode_dk(const DecodeArgs& a) {
    switch (a.d_v) {
        case 32: return launch_decode_t<BF16, DK, 32>(a);
        case 64: return launch_decode_t<BF16, DK, 64>(a);
        case 128: return launch_decode_t<BF16, DK, 128>(a);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
    switch (a.d_k) {
        case 32: return launch_decode_dk<BF16, 32>(a);
        case 64: return launch_decode_dk<BF16, 64>(a);
        case 128: return launch_decode_dk<BF16, 128>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs& a) {
    return a.bf16 ? launch_decode_dt<true>(a) : launch_decode_dt<false>(a);
}

}  // namespace kda
