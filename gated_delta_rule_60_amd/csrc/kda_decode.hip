// kda_decode.hip -- fused single-token KDA step for gfx950.
//
// For one token the update rule of "Kimi Linear：让长上下文大模型真正实用的线性
// 注意力架构", section 三.5, with per-channel decay (section 三.1), is evaluated
// per (sequence, head) as
//
//     S' = Diag(alpha) S          u = S'^T k        w = S'^T q
//     e  = beta (v - u)           S_new = S' + k e^T
//     o  = S_new^T q = w + (k . q) e
//
// so the state is read from HBM once, kept in registers, and written once.
// The kernel is bound by HBM bandwidth (8 d_k d_v bytes of state traffic
// against about 7 d_k d_v flops), so it streams: a grid of a few workgroups
// per CU walks the (sequence, head) pairs, and each workgroup loads the
// next pair's state while it reduces and updates the current one.  State
// accesses are non-temporal (each byte is touched once per step).
//
// A scalar gate (Gated DeltaNet, one alpha per head: the same page, section
// 三.1) reads one log alpha per pair and uses it for every channel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kDecodeThreads = 1024;
constexpr int kDecodeBlocksPerCU = 2;

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NT = DK * (DV / 4) >= 4 * kDecodeThreads ? kDecodeThreads : 256;
    static constexpr int CQ = DV / 4;     // float4 column groups per state row
    static constexpr int NRG = NT / CQ;   // row groups
    static constexpr int RPT = DK / NRG;  // rows per thread: row = rg + NRG * r
    static_assert(NT % CQ == 0 && DK % NRG == 0 && RPT >= 1, "decode thread map");
};

}  // namespace

template <bool BF16, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_step_kernel(
    const typename Elem<BF16>::G* __restrict__ q, const typename Elem<BF16>::G* __restrict__ k,
    const typename Elem<BF16>::G* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, float* __restrict__ S, int npairs,
    typename Elem<BF16>::G* __restrict__ o, int la_pair, int la_chan) {
    using T = Elem<BF16>;
    using Sh = DecodeShape<DK, DV>;
    constexpr int NT = Sh::NT, CQ = Sh::CQ, NRG = Sh::NRG, RPT = Sh::RPT;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_u[NRG][DV], s_w[NRG][DV], s_kq[NRG];
    __shared__ float s_e[DV];

    const int tid = threadIdx.x;
    const int cq = tid % CQ;
    const int rg = tid / CQ;
    const int stride = gridDim.x;

    // state of pair p, rows rg + NRG r, columns 4 cq .. 4 cq + 3
    auto state_at = [&](int p, int r) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4_t*>(S + static_cast<size_t>(p) * DK * DV +
                                          static_cast<size_t>(rg + NRG * r) * DV + 4 * cq);
    };
    f32x4_t st[2][RPT];
    auto load_state = [&](auto X, int p) __attribute__((always_inline)) {
        constexpr int x = decltype(X)::value;
        const bool live = p < npairs;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            st[x][r] = __builtin_nontemporal_load(live ? state_at(p, r) : reinterpret_cast<f32x4_t*>(S + static_cast<size_t>(blockIdx.x) * DK * DV));
    };

    // One pair with its state in set X.  The next pair's loads (set 1 - X)
    // were issued before this call and stay in flight throughout.
    auto step = [&](auto X, int pair) __attribute__((always_inline)) {
        constexpr int x = decltype(X)::value;
        const size_t tk = static_cast<size_t>(pair) * DK;
        for (int i = tid; i < DK; i += NT) {
            s_k[i] = T::to_f32(k[tk + i]);
            s_q[i] = T::to_f32(q[tk + i]);
            s_a[i] = exp_e(log_alpha[static_cast<size_t>(la_pair) * pair + la_chan * i]);
        }
        __syncthreads();

        f32x4_t u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = rg + NRG * r;
            const float a = s_a[row], kk = s_k[row], qq = s_q[row];
            kq += kk * qq;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                st[x][r][c] *= a;
                u[c] += kk * st[x][r][c];
                w[c] += qq * st[x][r][c];
            }
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

        const f32x4_t e4 = *reinterpret_cast<const f32x4_t*>(s_e + 4 * cq);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float kk = s_k[rg + NRG * r];
            f32x4_t xs = st[x][r];
#pragma unroll
            for (int c = 0; c < 4; ++c) xs[c] += kk * e4[c];
            __builtin_nontemporal_store(xs, state_at(pair, r));
        }
        // the next step rewrites s_k, s_q, s_a and s_e
        __syncthreads();
    };

    // Pairs blockIdx.x, + stride, ...: even ones in set 0, odd ones in set 1.
    // Every load is unconditional, so the compiler's wait counts stay exact
    // (a wait for one set never covers the other): a load for a pair past
    // the last one reads a single 16-byte quad of this workgroup's first
    // pair, whose values are never used.
    const int p0 = blockIdx.x;
    if (p0 >= npairs) return;
    load_state(std::integral_constant<int, 0>{}, p0);
    asm volatile("" ::: "memory");
    load_state(std::integral_constant<int, 1>{}, p0 + stride);
    for (int p = p0; p < npairs; p += 2 * stride) {
        step(std::integral_constant<int, 0>{}, p);
        load_state(std::integral_constant<int, 0>{}, p + 2 * stride);
        if (p + stride >= npairs) break;
        step(std::integral_constant<int, 1>{}, p + stride);
        load_state(std::integral_constant<int, 1>{}, p + 3 * stride);
    }
}

template <bool BF16, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    using G = typename Elem<BF16>::G;
    int cus = 0;
    const hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const int64_t npairs = static_cast<int64_t>(a.N) * a.H;
    const int64_t grid = npairs < int64_t{kDecodeBlocksPerCU} * cus ? npairs : int64_t{kDecodeBlocksPerCU} * cus;
    hipLaunchKernelGGL((decode_step_kernel<BF16, DK, DV>), dim3(static_cast<unsigned>(grid)),
                       dim3(DecodeShape<DK, DV>::NT), 0, static_cast<hipStream_t>(a.stream),
                       static_cast<const G*>(a.q), static_cast<const G*>(a.k),
                       static_cast<const G*>(a.v), a.log_alpha, a.beta, a.S, static_cast<int>(npairs),
                       static_cast<G*>(a.o), a.scalar_gate ? 1 : DK, a.scalar_gate ? 0 : 1);
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
