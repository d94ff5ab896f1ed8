// kda_backward.hip -- backward pass of the KDA prefill on gfx950.
//
// Gradients of a scalar loss with respect to q, k, v, log alpha, beta and the
// initial state, given dL/do for every token and dL/dS_T for the final states.
// The forward recurrence (the update rule of "Kimi Linear：让长上下文大模型真正实用
// 的线性注意力架构", section 三.5, with per-channel gates from section 三.1 and
// the read-out o_t = S_t^T q_t after the update) is, per token,
//
//     S' = Diag(a) S_{t-1},  u = S'^T k,  w = v - u,  e = beta w,
//     S_t = S' + k e^T,      o_t = S_t^T q.
//
// Its reverse-mode derivative, with G = dL/dS_t carried from the last token:
//
//     dq = S_t do,  G += q do^T,  de = G^T k,  dv = beta de,  dbeta = de . w,
//     du = -beta de,  dk = G e + S' du,  dS' = G + k du^T,
//     dlog_alpha_i = a_i sum_j dS'_ij S_{t-1,ij},  G <- Diag(a) dS'.
//
// The columns of the state evolve independently of one another (column j
// sees only v_j), so one wave owns 8 value columns of one (sequence, head)
// for the whole sequence: every column sum of the recurrence (u and de) is a
// reduction across the lanes of one wave, with no barrier on the token chain.
// Row sums over the value columns (dq, dk, dlog_alpha) and dbeta are not on
// that chain; they are staged in LDS and summed over the workgroup's waves
// once per 8 tokens.
//
// Pass 1 (bwd_forward_kernel) runs the forward recurrence and stores the
// state entering every 16-token block (fp32 checkpoints) and w_t = v_t - u_t
// for every token.  Pass 2 (bwd_kernel) walks the blocks from the last: it
// stages a block's inputs in LDS, recomputes the states of 8 tokens at a time
// from the block's checkpoint into registers (steps that need no column sum,
// since w is stored), and applies the reverse step token by token.  A
// compile-time flag (SG) serves one gate per token and head (Gated DeltaNet).
//
// In this token-by-token form every step is rank-1 updates and
// matrix-vector products, done in fp32 on the vector ALU.  (The chunk form of
// the adjoint would turn the state-sized products into MFMA contractions.)
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kBwdBlock = 16;  // tokens per checkpoint block
constexpr int kBwdHalf = 8;    // tokens whose entering states are held in registers at once
constexpr int kBwdCols = 8;    // value columns per wave

// Lane layout of one wave's share (kBwdCols columns, all d_k rows) of a state.
//   d_k >= 64: lane l holds rows R l .. R l + R - 1 (R = d_k / 64) and all 8 columns.
//   d_k == 32: lane l holds row l & 31 and columns 4 (l >> 5) .. 4 (l >> 5) + 3.
template <int DK>
struct BwdLanes {
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k in {32, 64, 128}");
    static constexpr int R = DK >= 64 ? DK / 64 : 1;
    static constexpr int CPL = DK >= 64 ? kBwdCols : kBwdCols / 2;
    __device__ static int row(int lane, int rr) { return DK >= 64 ? R * lane + rr : (lane & 31); }
    __device__ static int col(int lane) { return DK >= 64 ? 0 : 4 * (lane >> 5); }
};

template <bool BF16>
__device__ __forceinline__ float ld(const typename Elem<BF16>::G* p) {
    if constexpr (BF16) {
        return bf16_to_f32(*p);
    } else {
        return *p;
    }
}

// DPP lane permutations inside a row of 16 lanes, each an xor pairing:
// row_mirror (lane i <- 15 - i: xor 15), row_half_mirror (xor 7), and
// quad_perm [1,0,3,2] (xor 1) and [2,3,0,1] (xor 2).
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppXor1 = 0xB1, kDppXor2 = 0x4E;

// value of v in lane src (wave-uniform result)
__device__ __forceinline__ float read_lane(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the rows of each of the lane's columns (the wave holds every row
// of its 8 columns), returned in every lane.  A butterfly halves the values a
// lane carries at each exchange (partners l ^ 32 and l ^ 16 across rows of
// lanes, then l ^ 15 inside a row), the three remaining exchanges (xor 1, 2
// and 7) finish each column's total, and the totals are broadcast to every
// lane through scalar registers.
template <int DK>
__device__ __forceinline__ void column_sums(const float (&p)[BwdLanes<DK>::CPL], float (&out)[BwdLanes<DK>::CPL],
                                            int lane) {
    float s;
    if constexpr (DK >= 64) {
        const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
        float h4[4], h2[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float send = b5 ? p[i] : p[i + 4];
            h4[i] = (b5 ? p[i + 4] : p[i]) + __shfl_xor(send, 32);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = b4 ? h4[i] : h4[i + 2];
            h2[i] = (b4 ? h4[i + 2] : h4[i]) + __shfl_xor(send, 16);
        }
        s = (b3 ? h2[1] : h2[0]) + dpp<kDppRowMirror>(b3 ? h2[0] : h2[1]);
    } else {
        const bool b4 = lane & 16, b3 = lane & 8;
        float h2[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = b4 ? p[i] : p[i + 2];
            h2[i] = (b4 ? p[i + 2] : p[i]) + __shfl_xor(send, 16);
        }
        s = (b3 ? h2[1] : h2[0]) + dpp<kDppRowMirror>(b3 ? h2[0] : h2[1]);
    }
    s += dpp<kDppXor1>(s);
    s += dpp<kDppXor2>(s);
    s += dpp<kDppRowHalfMirror>(s);
    // lane l holds the total of column 4 b5 + 2 b4 + b3 (d_k = 32: 2 b4 + b3 of
    // its half); the totals are read out of lanes 8 c into scalar registers
    if constexpr (DK >= 64) {
#pragma unroll
        for (int c = 0; c < 8; ++c) out[c] = read_lane(s, c << 3);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float lo = read_lane(s, c << 3), hi = read_lane(s, 32 | (c << 3));
            out[c] = (lane & 32) ? hi : lo;
        }
    }
}

// Sum of x over the 64 lanes of the wave, in every lane (partners xor 32, 16,
// then 15, 1, 2 and 7 inside rows of 16 lanes: together every lane bit).
__device__ __forceinline__ float wave_sum(float x) {
    x += __shfl_xor(x, 32);
    x += __shfl_xor(x, 16);
    x += dpp<kDppRowMirror>(x);
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    return x;
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// accesses, not for its outstanding global stores.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct BwdArgs {
    const void *q, *k, *v, *dO;
    const float *la, *beta, *S0, *dST;
    const int32_t* cu;
    int32_t N, H, DV;
    float *ckpt, *w;
    float *dq, *dk, *dv, *dla, *dbeta, *dS0;
};

__device__ __forceinline__ int64_t ckpt_slot(const int32_t* cu, int n, int b) {
    return static_cast<int64_t>(cu[n] / kBwdBlock) + n + b;
}

// The sequence of rank r when sequences are taken longest first (ties by
// index): workgroups go out in that order, so the longest chains start
// first even when not every workgroup fits on the GPU at once. Each wave
// computes it on its own, at kernel entry with all lanes active; batches of
// more than 64 sequences keep their order.
__device__ __forceinline__ int seq_longest_first(const int32_t* cu, int N, int r) {
    if (N > 64) return r;
    const int j = threadIdx.x & 63;
    const int len = j < N ? cu[j + 1] - cu[j] : -1;
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int lm = __shfl(len, m);
        rank += (lm > len || (lm == len && m < j)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(j < N && rank == r);
    return __ffsll(static_cast<unsigned long long>(hit)) - 1;
}

// ---------------------------------------------------------------------------
// Pass 1: forward recurrence; checkpoints and w.  SG: one gate per token and
// head (log_alpha [T_tot, H], Gated DeltaNet), used for every key channel.  Grid: N * H * slices
// workgroups of NW waves; wave wv of slice s owns columns
// (s NW + wv) 8 .. + 7.
// ---------------------------------------------------------------------------
template <bool BF16, int DK, int NW, bool SG>
__global__ void __launch_bounds__(64 * NW) bwd_forward_kernel(BwdArgs a) {
    using L = BwdLanes<DK>;
    using G = typename Elem<BF16>::G;
    constexpr int R = L::R, CPL = L::CPL;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slices = a.DV / (kBwdCols * NW);
    const int s = blockIdx.x % slices, pair = blockIdx.x / slices;
    const int n = seq_longest_first(a.cu, a.N, pair / a.H), h = pair % a.H;
    const int H = a.H, DV = a.DV;
    const int c0 = (s * NW + wv) * kBwdCols + L::col(lane);
    const int64_t t0 = a.cu[n], t1 = a.cu[n + 1];

    float S[R][CPL];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            S[rr][c] = a.S0 ? a.S0[((static_cast<int64_t>(n) * H + h) * DK + L::row(lane, rr)) * DV + c0 + c] : 0.f;

    const G* gk = static_cast<const G*>(a.k);
    const G* gv = static_cast<const G*>(a.v);
    // Tokens run in groups of 4; the inputs of the next group are
    // loaded while the current group is computed.
    constexpr int GT = 4;
    float cla[GT][R], ckk[GT][R], cvv[GT][CPL], cb[GT];
    float nla[GT][R], nkk[GT][R], nvv[GT][CPL], nb[GT];
    auto fetch = [&](int64_t g0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            if (g0 + j < t1) {
                const int64_t t = g0 + j, tk = (t * H + h) * DK, tv = (t * H + h) * DV;
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    nla[j][rr] = SG ? a.la[t * H + h] : a.la[tk + L::row(lane, rr)];
                    nkk[j][rr] = ld<BF16>(gk + tk + L::row(lane, rr));
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) nvv[j][c] = ld<BF16>(gv + tv + c0 + c);
                nb[j] = a.beta[t * H + h];
            }
        }
    };
    if (t0 < t1) fetch(t0);
    for (int64_t g0 = t0; g0 < t1; g0 += GT) {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                cla[j][rr] = nla[j][rr];
                ckk[j][rr] = nkk[j][rr];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) cvv[j][c] = nvv[j][c];
            cb[j] = nb[j];
        }
        if (g0 + GT < t1) fetch(g0 + GT);
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            const int64_t t = g0 + j;
            if (t >= t1) break;
            if ((t - t0) % kBwdBlock == 0) {
                float* ck = a.ckpt + (ckpt_slot(a.cu, n, static_cast<int>((t - t0) / kBwdBlock)) * H + h) * DK * DV;
#pragma unroll
                for (int rr = 0; rr < R; ++rr)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) ck[static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c] = S[rr][c];
            }
            float up[CPL], u[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    S[rr][c] *= exp_e(cla[j][rr]);
                    acc = __builtin_fmaf(ckk[j][rr], S[rr][c], acc);
                }
                up[c] = acc;
            }
            column_sums<DK>(up, u, lane);
            float wv_[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                wv_[c] = cvv[j][c] - u[c];
                const float e = cb[j] * wv_[c];
#pragma unroll
                for (int rr = 0; rr < R; ++rr) S[rr][c] = __builtin_fmaf(ckk[j][rr], e, S[rr][c]);
            }
            if ((lane & 31) == 0 && (DK == 32 || lane == 0)) {
                const int64_t tv = (t * H + h) * DV;
#pragma unroll
                for (int c = 0; c < CPL; ++c) a.w[tv + c0 + c] = wv_[c];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 2: reverse walk.  Grid: N * H * SL workgroups of NW waves; wave wv
// of slice s owns columns (s NW + wv) 8 .. + 7, as in pass 1.
// With SL = 2 slices (d_v = 128) the two workgroups of one (sequence, head)
// meet in their row sums (dq, dk, dlog_alpha, dbeta) by atomic addition
// into outputs zeroed beforehand: with exactly two addends on zero the
// result does not depend on their order.
// ---------------------------------------------------------------------------
template <bool BF16, int DK, int NW>
struct BwdStage {
    static constexpr int BV = kBwdCols * NW;  // value columns of the workgroup
    // row sums: [quantity dq, dk, dlog_alpha][token of the half][wave][row], then dbeta [token][wave]
    static constexpr int kRowFloats = 3 * kBwdHalf * NW * DK;
    static constexpr int kBetaFloats = kBwdHalf * NW;  // also the per-head gate's [token][wave] sums
    // inputs of one block, fp32: alpha = exp(log_alpha), k, q [token][row]; w, do [token][column]; beta
    static constexpr int kInFloats = 3 * kBwdBlock * DK + 2 * kBwdBlock * BV + kBwdBlock;
    static constexpr int kFloats = kRowFloats + 2 * kBetaFloats + kInFloats;
};

template <bool BF16, int DK, int NW, int SL, bool SG>
__global__ void __launch_bounds__(64 * NW) bwd_kernel(BwdArgs a) {
    using L = BwdLanes<DK>;
    using G = typename Elem<BF16>::G;
    using St = BwdStage<BF16, DK, NW>;
    constexpr int R = L::R, CPL = L::CPL;
    constexpr int BV = St::BV;
    __shared__ float stage[St::kFloats];
    float* sRow = stage;
    float* sBeta = sRow + St::kRowFloats;
    float* sGate = sBeta + St::kBetaFloats;
    float* sA = sGate + St::kBetaFloats;
    float* sK = sA + kBwdBlock * DK;
    float* sQ = sK + kBwdBlock * DK;
    float* sW = sQ + kBwdBlock * DK;
    float* sDO = sW + kBwdBlock * BV;
    float* sB = sDO + kBwdBlock * BV;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    static_assert(SL == 1 || SL == 2, "one or two slices");
    const int s = blockIdx.x % SL, pair = blockIdx.x / SL;
    const int n = seq_longest_first(a.cu, a.N, pair / a.H), h = pair % a.H;
    const int H = a.H, DV = a.DV;
    const int c0 = (s * NW + wv) * kBwdCols + L::col(lane);
    const int cs = c0 - s * BV;  // the lane's first column inside the workgroup's slice
    const int64_t t0 = a.cu[n], t1 = a.cu[n + 1];
    const int nblk = static_cast<int>((t1 - t0 + kBwdBlock - 1) / kBwdBlock);
    const G* gq = static_cast<const G*>(a.q);
    const G* gk = static_cast<const G*>(a.k);
    const G* gdo = static_cast<const G*>(a.dO);
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;

    float Gr[R][CPL];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            Gr[rr][c] = a.dST ? a.dST[sbase + static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c] : 0.f;

    // one forward step of row r of the staged block without a column sum (w is stored)
    auto step = [&](float (&S)[R][CPL], int r) __attribute__((always_inline)) {
        const float bt = sB[r];
        float al[R], kk[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            al[rr] = sA[r * DK + L::row(lane, rr)];
            kk[rr] = sK[r * DK + L::row(lane, rr)];
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float e = bt * sW[r * BV + cs + c];
#pragma unroll
            for (int rr = 0; rr < R; ++rr) S[rr][c] = __builtin_fmaf(kk[rr], e, al[rr] * S[rr][c]);
        }
    };

    for (int b = nblk - 1; b >= 0; --b) {
        const int64_t tb = t0 + static_cast<int64_t>(b) * kBwdBlock;
        const int64_t te = tb + kBwdBlock < t1 ? tb + kBwdBlock : t1;
        const float* ck = a.ckpt + (ckpt_slot(a.cu, n, b) * H + h) * DK * DV;
        // stage the block's inputs (every reader of the previous block has
        // passed the barrier that ends its last half)
        const int ntok = static_cast<int>(te - tb);
        for (int i = threadIdx.x; i < ntok * DK; i += 64 * NW) {
            const int64_t tk = ((tb + i / DK) * H + h) * DK + i % DK;
            sA[i] = exp_e(SG ? a.la[(tb + i / DK) * H + h] : a.la[tk]);
            sK[i] = ld<BF16>(gk + tk);
            sQ[i] = ld<BF16>(gq + tk);
        }
        for (int i = threadIdx.x; i < ntok * BV; i += 64 * NW) {
            const int64_t tv = ((tb + i / BV) * H + h) * DV + s * BV + i % BV;
            sW[i] = a.w[tv];
            sDO[i] = ld<BF16>(gdo + tv);
        }
        if (threadIdx.x < ntok) sB[threadIdx.x] = a.beta[(tb + threadIdx.x) * H + h];
        lds_barrier();
        for (int half = 1; half >= 0; --half) {
            const int64_t th = tb + half * kBwdHalf;
            if (th >= te) continue;  // uniform over the workgroup
            float S[R][CPL];
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int c = 0; c < CPL; ++c) S[rr][c] = ck[static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c];
            for (int r = 0; r < half * kBwdHalf; ++r) step(S, r);
            float Sp[kBwdHalf][R][CPL];
#pragma unroll
            for (int r = 0; r < kBwdHalf; ++r) {
#pragma unroll
                for (int rr = 0; rr < R; ++rr)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) Sp[r][rr][c] = S[rr][c];
                if (th + r < te) step(S, half * kBwdHalf + r);
            }
#pragma unroll
            for (int r = kBwdHalf - 1; r >= 0; --r) {
                const int64_t t = th + r;
                if (t >= te) continue;
                const int64_t tv = (t * H + h) * DV;
                const int rb = half * kBwdHalf + r;  // row of the staged block
                const float bt = sB[rb];
                float al[R], kk[R], qq[R], dqp[R], dkp[R], dap[R];
                float wv_[CPL], dov[CPL], dep[CPL], de[CPL];
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const int row = L::row(lane, rr);
                    al[rr] = sA[rb * DK + row];
                    kk[rr] = sK[rb * DK + row];
                    qq[rr] = sQ[rb * DK + row];
                    dqp[rr] = 0.f;
                    dkp[rr] = 0.f;
                    dap[rr] = 0.f;
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    wv_[c] = sW[rb * BV + cs + c];
                    dov[c] = sDO[rb * BV + cs + c];
                    dep[c] = 0.f;
                }
                // read-out and the rank-1 correction: dq = S_t do, G += q do^T, de = G^T k
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const float e = bt * wv_[c];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) {
                        const float st = __builtin_fmaf(kk[rr], e, al[rr] * Sp[r][rr][c]);
                        dqp[rr] = __builtin_fmaf(st, dov[c], dqp[rr]);
                        Gr[rr][c] = __builtin_fmaf(qq[rr], dov[c], Gr[rr][c]);
                        dep[c] = __builtin_fmaf(Gr[rr][c], kk[rr], dep[c]);
                    }
                }
                column_sums<DK>(dep, de, lane);
                // error, prediction and decay
                float dbp = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    dbp = __builtin_fmaf(de[c], wv_[c], dbp);
                    const float e = bt * wv_[c];
                    const float du = -bt * de[c];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) {
                        const float sd = al[rr] * Sp[r][rr][c];
                        dkp[rr] = __builtin_fmaf(Gr[rr][c], e, __builtin_fmaf(sd, du, dkp[rr]));
                        const float g = __builtin_fmaf(kk[rr], du, Gr[rr][c]);
                        dap[rr] = __builtin_fmaf(g, Sp[r][rr][c], dap[rr]);
                        Gr[rr][c] = al[rr] * g;
                    }
                }
                if (DK >= 64 ? lane == 0 : (lane & 31) == 0) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) a.dv[tv + c0 + c] = bt * de[c];
                }
                if constexpr (SG) {
                    // the per-head gate: dlog_alpha summed over the key channels too
                    float gp = 0.f;
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) gp = __builtin_fmaf(al[rr], dap[rr], gp);
                    gp = wave_sum(gp);
                    if (lane == 0) sGate[r * NW + wv] = gp;
                }
                if constexpr (DK == 32) {
                    // the two column halves of a row meet
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) {
                        dqp[rr] += __shfl_xor(dqp[rr], 32);
                        dkp[rr] += __shfl_xor(dkp[rr], 32);
                        dap[rr] += __shfl_xor(dap[rr], 32);
                    }
                    dbp += __shfl_xor(dbp, 32);
                }
                if (DK >= 64 || lane < 32) {
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) {
                        const int row = L::row(lane, rr);
                        sRow[((0 * kBwdHalf + r) * NW + wv) * DK + row] = dqp[rr];
                        sRow[((1 * kBwdHalf + r) * NW + wv) * DK + row] = dkp[rr];
                        if constexpr (!SG) sRow[((2 * kBwdHalf + r) * NW + wv) * DK + row] = al[rr] * dap[rr];
                    }
                }
                if (lane == 0) sBeta[r * NW + wv] = dbp;
            }
            lds_barrier();
            // sums over the waves, one output element per thread and item: row sums
            // of NQ quantities, then dbeta, then (SG) the per-head gate
            constexpr int NQ = SG ? 2 : 3;
            for (int it = threadIdx.x; it < NQ * kBwdHalf * DK + (SG ? 2 : 1) * kBwdHalf; it += 64 * NW) {
                if (it < NQ * kBwdHalf * DK) {
                    const int qn = it / (kBwdHalf * DK), r = (it / DK) % kBwdHalf, row = it % DK;
                    const int64_t t = th + r;
                    if (t < te) {
                        float acc = 0.f;
                        for (int w2 = 0; w2 < NW; ++w2) acc += sRow[((qn * kBwdHalf + r) * NW + w2) * DK + row];
                        float* out = qn == 0 ? a.dq : (qn == 1 ? a.dk : a.dla);
                        float* dst = out + (t * H + h) * DK + row;
                        if constexpr (SL > 1) {
                            atomicAdd(dst, acc);
                        } else {
                            *dst = acc;
                        }
                    }
                } else {
                    const int r2 = it - NQ * kBwdHalf * DK, r = r2 % kBwdHalf;
                    const bool gate = r2 >= kBwdHalf;  // SG only
                    const int64_t t = th + r;
                    if (t < te) {
                        float acc = 0.f;
                        for (int w2 = 0; w2 < NW; ++w2) acc += (gate ? sGate : sBeta)[r * NW + w2];
                        float* dst = (gate ? a.dla : a.dbeta) + t * H + h;
                        if constexpr (SL > 1) {
                            atomicAdd(dst, acc);
                        } else {
                            *dst = acc;
                        }
                    }
                }
            }
            lds_barrier();
        }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int c = 0; c < CPL; ++c) a.dS0[sbase + static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c] = Gr[rr][c];
}

// ---------------------------------------------------------------------------
// Token-recurrent prefill (KDA_PREFILL_ANY_DECAY): the forward recurrence of
// pass 1 plus the read-out o_t = S_t^T q_t and the final state.  It forms no
// decay products across tokens, so any finite log alpha <= 0 works (a token
// with alpha underflowing to 0 resets the state exactly).  Same grid and
// column ownership as pass 1.  S_T may alias S0: each lane reads and writes
// only its own elements.
// ---------------------------------------------------------------------------
struct RecArgs {
    const void *q, *k, *v;
    const float *la, *beta, *S0;
    const int32_t* cu;
    int32_t H, DV;
    void* o;
    float* S_T;
};

template <bool BF16, int DK, int NW, bool SG>
__global__ void __launch_bounds__(64 * NW) rec_prefill_kernel(RecArgs a) {
    using L = BwdLanes<DK>;
    using G = typename Elem<BF16>::G;
    constexpr int R = L::R, CPL = L::CPL;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slices = a.DV / (kBwdCols * NW);
    const int s = blockIdx.x % slices, pair = blockIdx.x / slices;
    const int n = pair / a.H, h = pair % a.H;
    const int H = a.H, DV = a.DV;
    const int c0 = (s * NW + wv) * kBwdCols + L::col(lane);
    const int64_t t0 = a.cu[n], t1 = a.cu[n + 1];
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;
    const G* gq = static_cast<const G*>(a.q);
    const G* gk = static_cast<const G*>(a.k);
    const G* gv = static_cast<const G*>(a.v);
    G* go = static_cast<G*>(a.o);

    float S[R][CPL];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            S[rr][c] = a.S0 ? a.S0[sbase + static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c] : 0.f;

    // inputs of the next token are loaded while the current one is computed
    float nla[R], nk[R], nq[R], nv[CPL], nb = 0.f;
    auto fetch = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t tk = (t * H + h) * DK, tv = (t * H + h) * DV;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            nla[rr] = SG ? a.la[t * H + h] : a.la[tk + L::row(lane, rr)];
            nk[rr] = ld<BF16>(gk + tk + L::row(lane, rr));
            nq[rr] = ld<BF16>(gq + tk + L::row(lane, rr));
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) nv[c] = ld<BF16>(gv + tv + c0 + c);
        nb = a.beta[t * H + h];
    };
    if (t0 < t1) fetch(t0);
    for (int64_t t = t0; t < t1; ++t) {
        float al[R], kk[R], qq[R], vv[CPL];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            al[rr] = exp_e(nla[rr]);
            kk[rr] = nk[rr];
            qq[rr] = nq[rr];
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) vv[c] = nv[c];
        const float bt = nb;
        if (t + 1 < t1) fetch(t + 1);
        float up[CPL], u[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                S[rr][c] *= al[rr];
                acc = __builtin_fmaf(kk[rr], S[rr][c], acc);
            }
            up[c] = acc;
        }
        column_sums<DK>(up, u, lane);
        float op[CPL], ov[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float e = bt * (vv[c] - u[c]);
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                S[rr][c] = __builtin_fmaf(kk[rr], e, S[rr][c]);
                acc = __builtin_fmaf(qq[rr], S[rr][c], acc);
            }
            op[c] = acc;
        }
        column_sums<DK>(op, ov, lane);
        if ((lane & 31) == 0 && (DK == 32 || lane == 0)) {
            const int64_t tv = (t * H + h) * DV;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if constexpr (BF16) {
                    go[tv + c0 + c] = f32_to_bf16(ov[c]);
                } else {
                    go[tv + c0 + c] = ov[c];
                }
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int c = 0; c < CPL; ++c) a.S_T[sbase + static_cast<int64_t>(L::row(lane, rr)) * DV + c0 + c] = S[rr][c];
}

__global__ void __launch_bounds__(256) bwd_zero_kernel(float* __restrict__ p, int64_t count) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = 0.f;
}

// waves per workgroup (8 columns each): 8, or 4 at d_v = 32; a workgroup
// covers at most 64 columns, so d_v = 128 runs two slices per (sequence, head)
inline int bwd_waves(int d_v) { return d_v >= 64 ? 8 : 4; }

inline unsigned grid_1d(int64_t count) {
    const int64_t blocks = (count + 255) / 256;
    return static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
}

template <bool BF16, int DK, int NW, bool SG>
hipError_t launch_bwd_nw(const BwdArgs& a, int64_t T_tot, hipStream_t st) {
    const int slices = a.DV / (kBwdCols * NW);
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.N) * a.H * slices);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_forward_kernel<BF16, DK, NW, SG>), dim3(grid), dim3(64 * NW), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (slices == 2) {
        // zero the outputs the slices add into: dq, dk, dlog_alpha [T_tot, H, d_k] ([T_tot, H]
        // with SG), dbeta [T_tot, H]
        const int64_t rowN = T_tot * a.H * DK;
        float* bufs[4] = {a.dq, a.dk, a.dla, a.dbeta};
        const int64_t counts[4] = {rowN, rowN, SG ? T_tot * a.H : rowN, T_tot * a.H};
        for (int i = 0; i < 4; ++i)
            if (counts[i] > 0)
                hipLaunchKernelGGL(bwd_zero_kernel, dim3(grid_1d(counts[i])), dim3(256), 0, st, bufs[i], counts[i]);
        hipLaunchKernelGGL((bwd_kernel<BF16, DK, NW, 2, SG>), dim3(grid), dim3(64 * NW), 0, st, a);
    } else if (slices == 1) {
        hipLaunchKernelGGL((bwd_kernel<BF16, DK, NW, 1, SG>), dim3(grid), dim3(64 * NW), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16, int DK, bool SG>
hipError_t launch_bwd_sg(const BwdArgs& a, int64_t T_tot, hipStream_t st) {
    switch (bwd_waves(a.DV)) {
        case 4: return launch_bwd_nw<BF16, DK, 4, SG>(a, T_tot, st);
        case 8: return launch_bwd_nw<BF16, DK, 8, SG>(a, T_tot, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, int DK>
hipError_t launch_bwd_dk(const BwdArgs& a, bool scalar_gate, int64_t T_tot, hipStream_t st) {
    return scalar_gate ? launch_bwd_sg<BF16, DK, true>(a, T_tot, st) : launch_bwd_sg<BF16, DK, false>(a, T_tot, st);
}

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// workspace: checkpoints | w
inline size_t bwd_ckpt_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v) {
    const int64_t slots = T_tot / kBwdBlock + N + 1;
    return round256(static_cast<size_t>(slots) * H * d_k * d_v * sizeof(float));
}

}  // namespace

size_t prefill_bwd_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v) {
    return bwd_ckpt_bytes(N, T_tot, H, d_k, d_v) + static_cast<size_t>(T_tot) * H * d_v * sizeof(float);
}

hipError_t launch_prefill_bwd(const BackwardArgs& b) {
    BwdArgs a;
    a.q = b.q;
    a.k = b.k;
    a.v = b.v;
    a.dO = b.dO;
    a.la = b.log_alpha;
    a.beta = b.beta;
    a.S0 = b.S0;
    a.dST = b.dS_T;
    a.cu = b.cu_seqlens;
    a.N = b.N;
    a.H = b.H;
    a.DV = b.d_v;
    unsigned char* ws = static_cast<unsigned char*>(b.workspace);
    a.ckpt = reinterpret_cast<float*>(ws);
    a.w = reinterpret_cast<float*>(ws + bwd_ckpt_bytes(b.N, b.T_tot, b.H, b.d_k, b.d_v));
    a.dq = b.dq;
    a.dk = b.dk;
    a.dv = b.dv;
    a.dla = b.dlog_alpha;
    a.dbeta = b.dbeta;
    a.dS0 = b.dS0;
    hipStream_t st = static_cast<hipStream_t>(b.stream);
    if (b.bf16) {
        switch (b.d_k) {
            case 32: return launch_bwd_dk<true, 32>(a, b.scalar_gate, b.T_tot, st);
            case 64: return launch_bwd_dk<true, 64>(a, b.scalar_gate, b.T_tot, st);
            case 128: return launch_bwd_dk<true, 128>(a, b.scalar_gate, b.T_tot, st);
        }
    } else {
        switch (b.d_k) {
            case 32: return launch_bwd_dk<false, 32>(a, b.scalar_gate, b.T_tot, st);
            case 64: return launch_bwd_dk<false, 64>(a, b.scalar_gate, b.T_tot, st);
            case 128: return launch_bwd_dk<false, 128>(a, b.scalar_gate, b.T_tot, st);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_recurrent(const PrefillArgs& p) {
    RecArgs a{p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, p.cu_seqlens, p.H, p.d_v, p.o, p.S_T};
    const int nw = bwd_waves(p.d_v);
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(p.N) * p.H * (p.d_v / (kBwdCols * nw)));
    if (grid == 0) return hipSuccess;
    hipStream_t st = static_cast<hipStream_t>(p.stream);
#define KDA_REC_LAUNCH(BF, DKV, NWV, SGV) \
    hipLaunchKernelGGL((rec_prefill_kernel<BF, DKV, NWV, SGV>), dim3(grid), dim3(64 * NWV), 0, st, a)
#define KDA_REC_DK(BF, DKV)                                                   \
    do {                                                                      \
        if (nw == 8) {                                                        \
            if (p.scalar_gate) KDA_REC_LAUNCH(BF, DKV, 8, true);              \
            else KDA_REC_LAUNCH(BF, DKV, 8, false);                           \
        } else {                                                              \
            if (p.scalar_gate) KDA_REC_LAUNCH(BF, DKV, 4, true);              \
            else KDA_REC_LAUNCH(BF, DKV, 4, false);                           \
        }                                                                     \
    } while (0)
    if (p.bf16) {
        switch (p.d_k) {
            case 32: KDA_REC_DK(true, 32); break;
            case 64: KDA_REC_DK(true, 64); break;
            case 128: KDA_REC_DK(true, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.d_k) {
            case 32: KDA_REC_DK(false, 32); break;
            case 64: KDA_REC_DK(false, 64); break;
            case 128: KDA_REC_DK(false, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef KDA_REC_DK
#undef KDA_REC_LAUNCH
    return hipGetLastError();
}

}  // namespace kda
