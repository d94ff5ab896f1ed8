// kda_bwd_chunk.hip -- chunked backward pass of the KDA prefill on gfx950.
//
// Gradients of a scalar loss with respect to q, k, v, log alpha, beta and the
// initial state, given dL/do for every token and dL/dS_T for the final
// states, for the recurrence of "Kimi Linear：让长上下文大模型真正实用的线性注意
// 力架构" (juejin.cn), section 三.5 (per-channel gates, section 三.1; read-out
// o_t = S_t^T q_t after the update).  It is the reverse-mode derivative of
// the chunk algebra the forward kernel evaluates (exact, so it equals the
// derivative of the token recurrence up to rounding).  For one chunk of C
// tokens with entering state S, g_r the cumulative log decay, Gamma = e^g:
//
//   forward:  K~ = K Gamma, K^ = K / Gamma, Q~ = Q Gamma, Kbar = K^ Gamma_C
//             G = K~ K^T, L = strictly_lower(beta G), A = lower_incl(Q~ K^T)
//             W0 = V - K~ S, U = (I + L)^-1 beta W0
//             O = Q~ S + A U,  S_next = Gamma_C S + Kbar^T U
//   reverse, with D = dL/dS_next carried from the chunk after this one and
//   Dg = Gamma_C D:
//             dU  = K^ Dg + A^T dO                (Kbar D = K^ Dg)
//             dR  = (I + L)^-T dU
//             dS  = Dg + Q~^T dO - K~^T (beta dR)        (carried to the chunk before)
//             dA  = lower_incl(dO U^T),   dL = -strictly_lower(dR U^T)
//             dQ~ = dO S^T + dA K^
//             dK~ = beta (dL K^ - dR S^T)
//             dK^ = dA^T Q~ + (beta dL)^T K~
//             dKbar' = U Dg^T               (= dKbar Gamma_C)
//             dbeta_r = dR_r . W0_r + sum_s dL_rs G_rs
//             dq = dQ~ Gamma,  dk = dK~ Gamma + (dK^ + dKbar') / Gamma
//             dg = k (dK~ Gamma - (dK^ + dKbar') / Gamma) + q dQ~ Gamma
//             dlog alpha_r = sum_{r' >= r} dg_r' + sum_j S_ij Dg_ij + sum_r dKbar'_r k_r / Gamma_r
//   (the last two terms: Gamma_C, through S_next and Kbar, depends on every
//   gate of the chunk).
//
// Pass 1 is the forward kernel in its checkpointing variant (kda_prefill.hip):
// per chunk it stores the entering state S and W0 (storage type).  This pass
// walks each sequence's chunks from the last, one workgroup per (sequence,
// head), all d_v columns, in barrier-separated stages per chunk:
//   P  every wave: the chunk's decayed operand tiles in LDS (leaf waves hold
//      the k, q, log alpha strips; chain waves copy dO), then the loads of the
//      chunk before are issued;
//   J  chain waves: the C x C products G, L, A and the inverses of the 16 x 16
//      diagonal blocks of I + L (nilpotent products, as in the forward);
//   CH chain waves (32 value columns each; D in fp32 registers): dU, dR,
//      dv = beta dR, the carried gradient's update, and dR, Dg published to
//      LDS in row order (each 16 x 16 tile transposed by an MFMA with the
//      identity); beside it the leaf waves solve U = (I + L)^-1 beta W0,
//      which only the later stages use;
//   LA every wave: the C x C products dA and dL;
//   LB every wave, one 16-channel tile at a time (S of those rows in
//      registers, loaded at the chunk's start): the products reduced over the
//      value columns and over the chunk's tokens, then dq, dk, dlog alpha and
//      dbeta.
// Every product of two operands is an MFMA (bf16 operands for bf16 inputs,
// fp32 for fp32 inputs) with fp32 accumulation; the carried gradient is fp32.
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

// No implicit contraction: the scalar-gate instances then perform the same
// roundings as the per-channel ones (identical bits for a repeated gate).
#pragma clang fp contract(off)

namespace kda {

namespace {

constexpr int kBcSortMax = 64;  // sequences ordered by length in-kernel up to this many

constexpr size_t bc_align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// Chunk length of the forward's checkpoints: the prefill kernel's choice
// (32 tokens, 16 for fp32 inputs with d_k >= 64); checked on the host.
template <bool BF16, int DK>
constexpr int kBcChunk = (BF16 || DK == 32) ? 32 : 16;

template <bool BF16, int DK, int DV, int C>
struct BcLayout {
    using E = typename Elem<BF16>::E;
    static constexpr int ES = static_cast<int>(sizeof(E));
    static constexpr int NB = C / 16;
    static constexpr int NC = DV / 32;  // chain waves: 32 value columns each
    static constexpr int NL = DK / 32;  // leaf waves: 32 key channels each
    static constexpr int NW = NC + NL;
    static constexpr int NT = 64 * NW;
    static constexpr int PADE = 16 / ES;  // 16 bytes of row padding
    static constexpr int DM = DK > DV ? DK : DV;
    static constexpr int LK = DM + PADE;  // [C][d] tiles: K~ (later U), K^, Q~ (later dR)
    static constexpr int LT = C + PADE;   // [d_k][C] tiles and C x C tiles
    static constexpr int LO = DV + PADE;  // dO
    static constexpr int LS = DV + PADE;  // Dg
    static constexpr int LB = 16 + PADE;  // diagonal 16 x 16 blocks
    static constexpr int NJOB = NB * (NB + 1) / 2;
    // producer geometry of the k, q, log alpha strips: lane = rg * QW + cq
    // holds rows 4 rg .. 4 rg + 3 and channels 4 cq .. 4 cq + 3 of its strip
    static constexpr int NRG = C / 4;
    static constexpr int QW = 64 / NRG;
    static constexpr int NQ = DK / 4;
    static constexpr int NPS = NQ > QW ? NQ / QW : 1;
    static_assert(NPS <= NL, "one leaf wave per channel strip");
    // dO copy: 4 x 4 blocks over the chain waves
    static constexpr int DITEMS = (C / 4) * (DV / 4);
    static constexpr int DPT = (DITEMS + 64 * NC - 1) / (64 * NC);

    static constexpr size_t SZ_CK = bc_align16(static_cast<size_t>(C) * LK * ES);
    static constexpr size_t SZ_TK = bc_align16(static_cast<size_t>(DK) * LT * ES);
    static constexpr size_t SZ_DO = bc_align16(static_cast<size_t>(C) * LO * ES);
    static constexpr size_t SZ_DS = bc_align16(static_cast<size_t>(DK) * LS * ES);
    static constexpr size_t SZ_CC = bc_align16(static_cast<size_t>(C) * LT * ES);
    static constexpr size_t SZ_TB = bc_align16(static_cast<size_t>(NB) * 16 * LB * ES);
    static constexpr size_t O_KT = 0;  // K~ rows; U rows from stage CH on
    static constexpr size_t O_KH = O_KT + SZ_CK;
    static constexpr size_t O_QT = O_KH + SZ_CK;  // Q~ rows; -dR rows from stage CH on
    static constexpr size_t O_KTT = O_QT + SZ_CK;  // K~^T
    static constexpr size_t O_QTT = O_KTT + SZ_TK;  // Q~^T
    static constexpr size_t O_KHT = O_QTT + SZ_TK;  // K^^T
    static constexpr size_t O_DO = O_KHT + SZ_TK;
    static constexpr size_t O_DS = O_DO + SZ_DO;
    static constexpr size_t O_L = O_DS + SZ_DS;     // L            [r][s]
    static constexpr size_t O_LT = O_L + SZ_CC;     // -L^T         [s][r]
    static constexpr size_t O_AT = O_LT + SZ_CC;    // A^T          [s][r]
    static constexpr size_t O_GT = O_AT + SZ_CC;    // G^T          [s][r]
    static constexpr size_t O_DA = O_GT + SZ_CC;    // dA           [r][s]
    static constexpr size_t O_DAT = O_DA + SZ_CC;   // dA^T         [s][r]
    static constexpr size_t O_DL = O_DAT + SZ_CC;   // dL           [r][s]
    static constexpr size_t O_BDLT = O_DL + SZ_CC;  // (beta dL)^T  [s][r]
    static constexpr size_t O_TN = O_BDLT + SZ_CC;  // -T_bb        [r][c] per block
    static constexpr size_t O_TT = O_TN + SZ_TB;    // T_bb^T       [r][c] per block
    static constexpr size_t O_G = O_TT + SZ_TB;  // cumulative log2 decay [C][DK] fp32
    static constexpr size_t O_BETA = O_G + bc_align16(static_cast<size_t>(4) * C * DK);
    static constexpr size_t O_GC = O_BETA + bc_align16(4 * C);
    static constexpr size_t O_DB = O_GC + bc_align16(4 * DK);
    static constexpr size_t O_DBL = O_DB + bc_align16(4 * NC * C);
    static constexpr size_t O_SG = O_DBL + bc_align16(4 * NJOB * C);
    static constexpr size_t O_SCAN = O_SG + bc_align16(4 * (DK / 16) * C);
    static constexpr size_t O_SEQ = O_SCAN + static_cast<size_t>(NPS) * 64 * 16;
    static constexpr size_t BYTES = O_SEQ + bc_align16(4 * (kBcSortMax + 1));
    static_assert(BYTES <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

struct BcArgs {
    const void* q;
    const void* k;
    const float* la;
    const float* beta;
    const void* dO;
    const float* dST;  // may be null
    const int32_t* cu;
    const void* cks;  // state checkpoints (storage type)
    const void* ckw;  // W0 checkpoints (storage type)
    float *dq, *dk, *dv, *dla, *dbeta, *dS0;
    int N, H;
};

// LDS barrier: waits for this wave's LDS operations only (global loads in
// flight stay in flight across it).
__device__ __forceinline__ void bc_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int CTRL>
__device__ __forceinline__ float bc_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Inclusive suffix sum over the 16 lanes of each row (row_shl 1, 2, 4, 8).
__device__ __forceinline__ float row_suffix(float x) {
    x += bc_dpp<0x101>(x);
    x += bc_dpp<0x102>(x);
    x += bc_dpp<0x104>(x);
    x += bc_dpp<0x108>(x);
    return x;
}
// Sum over the 16 lanes of each row, the same bits in every lane of the row:
// DPP butterflies within the row (quad permutations [1,0,3,2] and [2,3,0,1],
// then the half-row and the row mirror), no trip through LDS.
__device__ __forceinline__ float row_sum(float x) {
    x += bc_dpp<0xB1>(x);
    x += bc_dpp<0x4E>(x);
    x += bc_dpp<0x141>(x);
    x += bc_dpp<0x140>(x);
    return x;
}

// four consecutive storage elements, raw
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::R4 bc_load_raw4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (BF16) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return make_uint2(x[0], x[1]);
    } else {
        return buf_load_f4(r, voff, soff);
    }
}

// four fp32 values as four consecutive operand elements (bf16: round to nearest even)
template <bool BF16>
__device__ __forceinline__ void bc_put4(typename Elem<BF16>::E* p, float a, float b, float c, float d) {
    if constexpr (BF16) {
        bf16x4_t r;
        r[0] = static_cast<__bf16>(a);
        r[1] = static_cast<__bf16>(b);
        r[2] = static_cast<__bf16>(c);
        r[3] = static_cast<__bf16>(d);
        *reinterpret_cast<bf16x4_t*>(p) = r;
    } else {
        *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
    }
}

template <bool BF16>
__device__ __forceinline__ f32x4_t bc_widen(const typename Elem<BF16>::F4& x) {
    return f32x4_t{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                   static_cast<float>(x[3])};
}

// acc += A B over the C tokens of a chunk, A and B given as row-major LDS
// tiles (rows: the MFMA's m and n indices, k along the row).
template <bool BF16, int C>
__device__ __forceinline__ f32x4_t mma_rows(f32x4_t acc, const typename Elem<BF16>::E* a, int lda,
                                            const typename Elem<BF16>::E* b, int ldb, int lane) {
    if constexpr (C == 32) {
        return mma8<BF16>(acc, lds_frag8<BF16>(a, lda, lane), lds_frag8<BF16>(b, ldb, lane));
    } else {
        return mma4<BF16>(acc, lds_frag4<BF16>(a, lda, lane), lds_frag4<BF16>(b, ldb, lane));
    }
}

template <bool BF16, int DK, int DV, int C, bool SG>
__global__ __launch_bounds__((BcLayout<BF16, DK, DV, C>::NT)) void bwd_chunk_kernel(BcArgs a) {
    using Ly = BcLayout<BF16, DK, DV, C>;
    using T = Elem<BF16>;
    using E = typename T::E;
    using G = typename T::G;
    using R4 = typename T::R4;
    using F8 = typename T::F8;
    using F4 = typename T::F4;
    constexpr int NB = Ly::NB, NC = Ly::NC, NL = Ly::NL, NT = Ly::NT, NJOB = Ly::NJOB;
    constexpr int LK = Ly::LK, LT = Ly::LT, LO = Ly::LO, LS = Ly::LS, LB = Ly::LB;
    constexpr int NRG = Ly::NRG, QW = Ly::QW, NQ = Ly::NQ, NPS = Ly::NPS, DPT = Ly::DPT;
    constexpr int KBK = DK / 32, KBV = DV / 32;
    constexpr int NW = Ly::NW;
    constexpr int NCT = DK / 16;                    // 16-channel tiles of stage LB
    constexpr int TPW = (NCT + NW - 1) / NW;        // stage LB tiles per wave

    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::BYTES];
    E* const tKt = reinterpret_cast<E*>(smem + Ly::O_KT);
    E* const tU = tKt;
    E* const tKh = reinterpret_cast<E*>(smem + Ly::O_KH);
    E* const tQt = reinterpret_cast<E*>(smem + Ly::O_QT);
    E* const tDR = tQt;
    E* const tKtT = reinterpret_cast<E*>(smem + Ly::O_KTT);
    E* const tQtT = reinterpret_cast<E*>(smem + Ly::O_QTT);
    E* const tKhT = reinterpret_cast<E*>(smem + Ly::O_KHT);
    E* const tDO = reinterpret_cast<E*>(smem + Ly::O_DO);
    E* const tDS = reinterpret_cast<E*>(smem + Ly::O_DS);
    E* const tL = reinterpret_cast<E*>(smem + Ly::O_L);
    E* const tLt = reinterpret_cast<E*>(smem + Ly::O_LT);
    E* const tAt = reinterpret_cast<E*>(smem + Ly::O_AT);
    E* const tGt = reinterpret_cast<E*>(smem + Ly::O_GT);
    E* const tdA = reinterpret_cast<E*>(smem + Ly::O_DA);
    E* const tdAt = reinterpret_cast<E*>(smem + Ly::O_DAT);
    E* const tdL = reinterpret_cast<E*>(smem + Ly::O_DL);
    E* const tbdLt = reinterpret_cast<E*>(smem + Ly::O_BDLT);
    E* const tTn = reinterpret_cast<E*>(smem + Ly::O_TN);
    E* const tTt = reinterpret_cast<E*>(smem + Ly::O_TT);
    float* const sG = reinterpret_cast<float*>(smem + Ly::O_G);
    float* const sBeta = reinterpret_cast<float*>(smem + Ly::O_BETA);
    float* const sGC = reinterpret_cast<float*>(smem + Ly::O_GC);
    float* const sDb = reinterpret_cast<float*>(smem + Ly::O_DB);
    float* const sDbL = reinterpret_cast<float*>(smem + Ly::O_DBL);
    float* const sSG = reinterpret_cast<float*>(smem + Ly::O_SG);
    int* const sSeq = reinterpret_cast<int*>(smem + Ly::O_SEQ);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int H = a.H, N = a.N;

    // ---- work assignment: one workgroup per (sequence, head), longest first
    const int h = static_cast<int>(blockIdx.x) % H;
    const int rank = static_cast<int>(blockIdx.x) / H;
    int n = rank;
    if (N > 1 && N <= kBcSortMax) {
        for (int i = tid; i < N; i += NT) sSeq[i] = a.cu[i + 1] - a.cu[i];
        __syncthreads();
        for (int i = tid; i < N; i += NT) {
            const int li = sSeq[i];
            int r = 0;
            for (int j = 0; j < N; ++j) {
                const int lj = sSeq[j];
                r += (lj > li) || (lj == li && j < i);
            }
            if (r == rank) sSeq[kBcSortMax] = i;
        }
        __syncthreads();
        n = sSeq[kBcSortMax];
    }
    const int t_beg = a.cu[n];
    const int len = a.cu[n + 1] - t_beg;
    const int nch = (len + C - 1) / C;
    const size_t slot0 = static_cast<size_t>(t_beg / C + n);
    const size_t pair = static_cast<size_t>(n) * H + h;
    auto rows_of = [&](int m) __attribute__((always_inline)) { return min(C, len - m * C); };

    // The C x C tiles' blocks above the diagonal are never written: zero once.
    {
        uint4* z = reinterpret_cast<uint4*>(smem + Ly::O_L);
        constexpr int NZ = static_cast<int>((Ly::O_G - Ly::O_L) / 16);
        for (int i = tid; i < NZ; i += NT) z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    const bool is_chain = wave < NC;
    const int w = wave;       // chain wave: value columns 32 w .. 32 w + 31
    const int v = wave - NC;  // leaf wave: key channels 32 v .. 32 v + 31

    // ---- registers ------------------------------------------------------
    f32x4_t dS[2][DK / 16];  // chain: dL/dS entering the chunk after the current one (C layout)
    F4 w0c[2][NB];              // W0 of the current chunk, one 32-column block (C layout)
    R4 rdo[DPT][4];             // chain: raw dO rows of the next chunk
    R4 rk[4], rq[4];              // strip waves: raw k, q of the next chunk
    float4 rla[4];
    float rbeta = 0.f;

    const int strip = v;
    const int rg = lane / QW, cq = lane % QW;
    const int gq = strip * QW + cq;
    const bool qok = NQ >= QW || gq < NQ;
    const int i0 = 4 * min(gq, NQ - 1);
    constexpr int GS = static_cast<int>(sizeof(G));
    const int rowK = H * DK * GS;
    const int strideLA = SG ? H : H * DK;
    const int rowLA = strideLA * 4;
    const int rowB = H * 4;
    const int rowV = H * DV * GS;
    const G* const qh = static_cast<const G*>(a.q) + static_cast<size_t>(h) * DK;
    const G* const kh = static_cast<const G*>(a.k) + static_cast<size_t>(h) * DK;
    const float* const lah = a.la + static_cast<size_t>(h) * (SG ? 1 : DK);
    const float* const bh = a.beta + h;
    const G* const doh = static_cast<const G*>(a.dO) + static_cast<size_t>(h) * DV;
    const bool strip_wave = !is_chain && strip < NPS;
    const bool loads_beta = strip_wave && strip == 0 && lane < C;

    // Loads of chunk inputs.  Every load is unconditional: a chunk index below
    // 0, and waves or lanes without the data, read through empty buffer
    // ranges (zero, no memory touched).  The compiler's vmcnt waits then count
    // exactly, and a use of one chunk's data never waits for a later prefetch.
    auto rows_or0 = [&](int m) __attribute__((always_inline)) { return m >= 0 ? rows_of(m) : 0; };
    // chain: raw dO rows of chunk m (issued at the end of the chunk after it)
    auto issue_dO = [&](int m) __attribute__((always_inline)) {
        const int t0 = t_beg + max(m, 0) * C;
        const int rows = __builtin_amdgcn_readfirstlane(rows_or0(m));
        const auto rdo_r = buffer_rsrc(doh + static_cast<size_t>(t0) * H * DV, rows * rowV);
#pragma unroll
        for (int t = 0; t < DPT; ++t) {
            const int idx = lane + 64 * w + 64 * NC * t;
            const bool ok = Ly::DITEMS % (64 * NC) == 0 || idx < Ly::DITEMS;
            const int c4 = 4 * (idx % (DV / 4)), r0 = 4 * (idx / (DV / 4));
            const int off = ok ? r0 * rowV + c4 * GS : kNoAccess;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) rdo[t][rr] = bc_load_raw4<BF16>(rdo_r, off, rr * rowV);
        }
    };
    // W0 of chunk m, 32-column block cb (chain: block w for dbeta in stage CH;
    // leaf: the blocks of stage U)
    auto load_w0_block = [&](int m, int cb) __attribute__((always_inline)) {
        const E* wb = static_cast<const E*>(a.ckw) + ((slot0 + m) * H + h) * C * DV;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
                w0c[ct][rt] = *reinterpret_cast<const F4*>(wb + (static_cast<size_t>((2 * cb + ct) * NB + rt) * 64 + lane) * 4);
        }
    };
    auto load_w0 = [&](int m) __attribute__((always_inline)) { load_w0_block(m, is_chain ? w : min(v, DV / 32 - 1)); };
    // leaf strip waves: k, q, log alpha and beta rows of chunk m (one chunk ahead)
    auto issue_strip = [&](int m) __attribute__((always_inline)) {
        const int t0 = t_beg + max(m, 0) * C;
        const int rows = __builtin_amdgcn_readfirstlane(strip_wave ? rows_or0(m) : 0);
        const size_t tok = static_cast<size_t>(t0) * H * DK;
        const auto rk_r = buffer_rsrc(kh + tok, rows * rowK);
        const auto rq_r = buffer_rsrc(qh + tok, rows * rowK);
        const auto rl_r = buffer_rsrc(lah + static_cast<size_t>(t0) * strideLA, rows * rowLA);
        const auto rb_r = buffer_rsrc(bh + static_cast<size_t>(t0) * H, rows * rowB);
        const int offK = 4 * rg * rowK + i0 * GS;
        const int offLA = 4 * rg * rowLA + (SG ? 0 : i0 * 4);
        rbeta = buf_load_f1(rb_r, loads_beta ? lane * rowB : kNoAccess, 0);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            if constexpr (SG) {
                const float x = buf_load_f1(rl_r, offLA, rr * rowLA);
                rla[rr] = make_float4(x, x, x, x);
            } else {
                rla[rr] = buf_load_f4(rl_r, offLA, rr * rowLA);
            }
            rk[rr] = bc_load_raw4<BF16>(rk_r, offK, rr * rowK);
            rq[rr] = bc_load_raw4<BF16>(rq_r, offK, rr * rowK);
        }
    };

    __syncthreads();  // zeroed tiles visible

    // identity, as the B operand of a 16-deep product
    F4 eye;
#pragma unroll
    for (int j = 0; j < 4; ++j) eye[j] = T::to_e(4 * lg + j == ln ? 1.f : 0.f);
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};

    // scalar gate: dlog alpha of one head, the sum of the channel tiles'
    // partials (sSG), stored for chunk m by the first leaf wave
    auto flush_sg = [&](int m) __attribute__((always_inline)) {
        if constexpr (SG) {
            if (wave == NC && lane < rows_of(m)) {
                float s = 0.f;
#pragma unroll
                for (int u = 0; u < NCT; ++u) s += sSG[u * C + lane];
                a.dla[static_cast<size_t>(t_beg + m * C + lane) * H + h] = s;
            }
        }
    };

    // ---- stages that every wave shares -----------------------------------
    // S rows of channel tile cti (channels 16 cti .. + 15) of chunk m, as
    // A-operand fragments over the value columns
    auto load_stile = [&](int m, int cti, F8 (&sf)[KBV]) __attribute__((always_inline)) {
        const E* sb = static_cast<const E*>(a.cks) + ((slot0 + m) * H + h) * DK * DV;
#pragma unroll
        for (int kb = 0; kb < KBV; ++kb)
            sf[kb] = *reinterpret_cast<const F8*>(sb + (static_cast<size_t>(cti * KBV + kb) * 64 + lane) * 8);
    };
    // Stage LA: the C x C products dA = lower_incl(dO U^T) and
    // dL = -strictly_lower(dR U^T) (from tDR = -dR), 16 x 16 blocks dealt
    // round-robin to the waves.
    auto stage_LA = [&]() __attribute__((always_inline)) {
        for (int jb = wave; jb < 2 * NJOB; jb += NW) {
            const bool isA = jb < NJOB;
            const int jc = isA ? jb : jb - NJOB;
            const int sb = jc == 2 ? 0 : jc, rb = jc == 2 ? 1 : jc;
            const E* xa = isA ? tDO : tDR;
            const int lda = isA ? LO : LK;
            f32x4_t acc = z4;
#pragma unroll
            for (int kb = 0; kb < KBV; ++kb)
                acc = mma8<BF16>(acc, lds_frag8<BF16>(xa + 16 * rb * lda + 32 * kb, lda, lane),
                                 lds_frag8<BF16>(tU + 16 * sb * LK + 32 * kb, LK, lane));
            // lane (ln = s): rows r = 16 rb + 4 lg + j of column s = 16 sb + ln
            const int s = 16 * sb + ln;
            const float4 b4 = *reinterpret_cast<const float4*>(sBeta + 16 * rb + 4 * lg);
            const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
            f32x4_t x;
            if (isA) {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = (s <= 16 * rb + 4 * lg + j) ? acc[j] : 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) tdA[(16 * rb + 4 * lg + j) * LT + s] = T::to_e(x[j]);
                bc_put4<BF16>(tdAt + s * LT + 16 * rb + 4 * lg, x[0], x[1], x[2], x[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = (s < 16 * rb + 4 * lg + j) ? acc[j] : 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) tdL[(16 * rb + 4 * lg + j) * LT + s] = T::to_e(x[j]);
                bc_put4<BF16>(tbdLt + s * LT + 16 * rb + 4 * lg, bj[0] * x[0], bj[1] * x[1], bj[2] * x[2],
                              bj[3] * x[3]);
                // second term of dbeta: sum over s of dL[r][s] G[r][s]
                const f32x4_t gv = bc_widen<BF16>(*reinterpret_cast<const F4*>(tGt + s * LT + 16 * rb + 4 * lg));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = row_sum(x[j] * gv[j]);
                    if (ln == 0) sDbL[jc * C + 16 * rb + 4 * lg + j] = t;
                }
            }
        }
    };

    // Stage LB for channel tile cti: the products over the value columns and
    // over the chunk's tokens, then dq, dk and dlog alpha of those 16 channels
    // for every token of the chunk.
    auto lb_tile = [&](int cti, const F8 (&sf)[KBV], int t0, int rows) __attribute__((always_inline)) {
        const int crow = 16 * cti;
        // value-column products, one 32-column block at a time:
        //   aq = S dO^T,  akk = -S dR^T (tDR holds -dR),  akb = Dg U^T
        // and c = sum_j S_ij Dg_ij
        f32x4_t aq[NB], akk[NB], akh[NB], akb[NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            aq[rt] = z4;
            akk[rt] = z4;
            akb[rt] = z4;
        }
        float cpart = 0.f;
#pragma unroll
        for (int kb = 0; kb < KBV; ++kb) {
            const F8 dga = lds_frag8<BF16>(tDS + crow * LS + 32 * kb, LS, lane);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                cpart = __builtin_fmaf(static_cast<float>(sf[kb][e]), static_cast<float>(dga[e]), cpart);
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
                aq[rt] = mma8<BF16>(aq[rt], sf[kb], lds_frag8<BF16>(tDO + 16 * rt * LO + 32 * kb, LO, lane));
                akk[rt] = mma8<BF16>(akk[rt], sf[kb], lds_frag8<BF16>(tDR + 16 * rt * LK + 32 * kb, LK, lane));
                akb[rt] = mma8<BF16>(akb[rt], dga, lds_frag8<BF16>(tU + 16 * rt * LK + 32 * kb, LK, lane));
            }
        }
        // c for channel crow + ln, in every lane of that column
        cpart += __shfl_xor(cpart, 16);
        cpart += __shfl_xor(cpart, 32);
        // token products: dQ~ += dA K^, dK~ / beta = dL K^ - dR S^T, dK^ = dA^T Q~ + (beta dL)^T K~
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            aq[rt] = mma_rows<BF16, C>(aq[rt], tKhT + crow * LT, LT, tdA + 16 * rt * LT, LT, lane);
            akk[rt] = mma_rows<BF16, C>(akk[rt], tKhT + crow * LT, LT, tdL + 16 * rt * LT, LT, lane);
            akh[rt] = mma_rows<BF16, C>(z4, tQtT + crow * LT, LT, tdAt + 16 * rt * LT, LT, lane);
            akh[rt] = mma_rows<BF16, C>(akh[rt], tKtT + crow * LT, LT, tbdLt + 16 * rt * LT, LT, lane);
        }
        // epilogue: lane (ln, lg) holds channels ch0 .. ch0 + 3 of token 16 rt + ln.
        // k and q enter dlog alpha only through the decayed tiles of the chunk,
        // k Gamma, k / Gamma and q Gamma (the operands of the chunk's products):
        // K^ from its rows, K~ and Q~ from their transposes.
        const int ch0 = crow + 4 * lg;
        float dg[NB][4], ex[4] = {0.f, 0.f, 0.f, 0.f};
        float dqv[NB][4], dkv[NB][4];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            const int r = 16 * rt + ln;
            const f32x4_t khv = bc_widen<BF16>(*reinterpret_cast<const F4*>(tKh + r * LK + ch0));
            float ktv[4], qtv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ktv[j] = static_cast<float>(tKtT[(ch0 + j) * LT + r]);
                qtv[j] = static_cast<float>(tQtT[(ch0 + j) * LT + r]);
            }
            // cumulative decay (log2 units) of these channels up to token r
            const float4 g4 = *reinterpret_cast<const float4*>(sG + r * DK + ch0);
            const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
            const float br = sBeta[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p = gv[j];
                const float gm = __builtin_amdgcn_exp2f(p), ig = __builtin_amdgcn_exp2f(-p);
                const float dqt = aq[rt][j];
                const float dkt = br * akk[rt][j];
                const float dkh = akh[rt][j] + akb[rt][j];
                const float a1 = dkt * gm, a2 = dkh * ig, a3 = dqt * gm;
                dqv[rt][j] = a3;
                dkv[rt][j] = a1 + a2;
                dg[rt][j] = (dkt * ktv[j] - dkh * khv[j]) + dqt * qtv[j];
                ex[j] = __builtin_fmaf(akb[rt][j], khv[j], ex[j]);
            }
        }
        // extra term of every row: c (moved to the epilogue layout) plus the
        // sum over the chunk's tokens of dKbar' k / Gamma
#pragma unroll
        for (int j = 0; j < 4; ++j) ex[j] = row_sum(ex[j]) + __shfl(cpart, 4 * lg + j);
        // suffix sums of dg over the tokens, from the last block
        const int rowDK = H * DK * 4;
        const size_t gbase = (static_cast<size_t>(t0) * H + h) * DK;
        const auto dq_r = buffer_rsrc(a.dq + gbase, rows * rowDK);
        const auto dk_r = buffer_rsrc(a.dk + gbase, rows * rowDK);
        const auto dla_r = buffer_rsrc(a.dla + (SG ? 0 : gbase), SG ? 0 : rows * rowDK);
        const int eo = ln * rowDK + 4 * ch0;
        float sfx[4] = {0.f, 0.f, 0.f, 0.f};
        float sg_row[NB];
#pragma unroll
        for (int rt = NB - 1; rt >= 0; --rt) {
            float out[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sv = row_suffix(dg[rt][j]) + sfx[j];
                sfx[j] += row_sum(dg[rt][j]);
                out[j] = sv + ex[j];
            }
            // rows past the sequence fall outside the buffer ranges
            buf_store_f4(dq_r, eo, 16 * rt * rowDK, dqv[rt][0], dqv[rt][1], dqv[rt][2], dqv[rt][3]);
            buf_store_f4(dk_r, eo, 16 * rt * rowDK, dkv[rt][0], dkv[rt][1], dkv[rt][2], dkv[rt][3]);
            if constexpr (!SG) buf_store_f4(dla_r, eo, 16 * rt * rowDK, out[0], out[1], out[2], out[3]);
            sg_row[rt] = (out[0] + out[1]) + (out[2] + out[3]);
        }
        if constexpr (SG) {
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
                float sv = sg_row[rt];
                sv += __shfl_xor(sv, 16);
                sv += __shfl_xor(sv, 32);
                if (lg == 0) sSG[cti * C + 16 * rt + ln] = sv;
            }
        }
    };
    // Stage LB of this wave: channel tiles wave, wave + NW, ...; the first
    // tile's S rows were loaded at the chunk's start.
    auto stage_LB = [&](int m, const F8 (&sf0)[KBV]) __attribute__((always_inline)) {
        const int t0 = t_beg + m * C;
        const int rows = rows_of(m);
        if (wave < NCT) lb_tile(wave, sf0, t0, rows);
#pragma unroll
        for (int k2 = 1; k2 < TPW; ++k2) {
            const int cti = wave + k2 * NW;
            if (cti < NCT) {
                F8 sf[KBV];
                load_stile(m, cti, sf);
                lb_tile(cti, sf, t0, rows);
            }
        }
        // dbeta of the chunk's tokens: the chain waves' partials plus the C x C term
        if (wave == NW - 1 && lane < rows) {
            float sv = 0.f;
#pragma unroll
            for (int u = 0; u < NC; ++u) sv += sDb[u * C + lane];
            const int rb = lane >> 4;
#pragma unroll
            for (int jc = 0; jc < NJOB; ++jc) {
                const int rbj = jc == 2 ? 1 : jc;
                if (rbj == rb) sv += sDbL[jc * C + lane];
            }
            a.dbeta[static_cast<size_t>(t0 + lane) * H + h] = sv;
        }
    };
    // the first LB tile's operands for chunk m, loaded at the chunk's start
    auto load_lb0 = [&](int m, F8 (&sf0)[KBV]) __attribute__((always_inline)) {
        load_stile(m, min(wave, NCT - 1), sf0);
    };

    if (is_chain) {
        // ---- initial carried gradient: dL/dS_T ----------------------------
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const size_t col = static_cast<size_t>(32 * w + 16 * ct + ln);
#pragma unroll
            for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dS[ct][it][j] = a.dST ? a.dST[pair * DK * DV + static_cast<size_t>(16 * it + 4 * lg + j) * DV + col] : 0.f;
            }
        }
        issue_dO(nch - 1);
        for (int m = nch - 1; m >= 0; --m) {
            // =============================== P: dO rows; this chunk's loads
            load_w0(m);
            const int t0 = t_beg + m * C;
            const int rows = rows_of(m);
#pragma unroll
            for (int t = 0; t < DPT; ++t) {
                const int idx = lane + 64 * w + 64 * NC * t;
                if (Ly::DITEMS % (64 * NC) == 0 || idx < Ly::DITEMS) {
                    const int c4 = 4 * (idx % (DV / 4)), r0 = 4 * (idx / (DV / 4));
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) T::lds_put_raw4(tDO + (r0 + rr) * LO + c4, rdo[t][rr]);
                }
            }
            bc_barrier();

            // =============================== J: C x C products and block inverses
            for (int jc = w; jc < NJOB; jc += NC) {
                // jobs: 0 -> (0,0), 1 -> (1,1), 2 -> (st 0, rt 1)
                const int st = jc == 2 ? 0 : jc, rt = jc == 2 ? 1 : jc;
                f32x4_t accG = z4, accN = z4, accA = z4;
#pragma unroll
                for (int kb = 0; kb < KBK; ++kb) {
                    const F8 ks = lds_frag8<BF16>(tKh + 16 * st * LK + 32 * kb, LK, lane);
                    const F8 kr = lds_frag8<BF16>(tKt + 16 * rt * LK + 32 * kb, LK, lane);
                    const F8 qr = lds_frag8<BF16>(tQt + 16 * rt * LK + 32 * kb, LK, lane);
                    accG = mma8<BF16>(accG, ks, kr);  // [s][r] = K^_s . K~_r = G[r][s]: lane (ln = r)
                    accN = mma8<BF16>(accN, kr, ks);  // [r][s] = G[r][s]: lane (ln = s)
                    accA = mma8<BF16>(accA, qr, ks);  // [r][s] = A[r][s] before the mask: lane (ln = s)
                }
                const int r_l = 16 * rt + ln;  // row of lane (ln = r) values
                const float br = sBeta[r_l];
                const float4 b4 = *reinterpret_cast<const float4*>(sBeta + 16 * rt + 4 * lg);
                const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
                f32x4_t Lr, Lc, At, Gc;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s_ = 16 * st + 4 * lg + j;  // column of lane (ln = r) values
                    const int r_ = 16 * rt + 4 * lg + j;  // row of lane (ln = s) values
                    const int s_l = 16 * st + ln;
                    Lr[j] = s_ < r_l ? br * accG[j] : 0.f;          // L[r_l][s_]
                    Lc[j] = s_l < r_ ? bj[j] * accN[j] : 0.f;       // L[r_][s_l]
                    At[j] = s_l <= r_ ? accA[j] : 0.f;              // A[r_][s_l]
                    Gc[j] = accN[j];                                // G[r_][s_l]
                }
                bc_put4<BF16>(tL + r_l * LT + 16 * st + 4 * lg, Lr[0], Lr[1], Lr[2], Lr[3]);
                const int srow = (16 * st + ln) * LT + 16 * rt + 4 * lg;
                bc_put4<BF16>(tLt + srow, -Lc[0], -Lc[1], -Lc[2], -Lc[3]);
                bc_put4<BF16>(tAt + srow, At[0], At[1], At[2], At[3]);
                bc_put4<BF16>(tGt + srow, Gc[0], Gc[1], Gc[2], Gc[3]);
                if (st == rt) {
                    // T = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for the
                    // strictly lower N = L_bb, from the C layouts of N^T (Lr) and N (Lc)
                    auto f4 = [&](const f32x4_t& x) __attribute__((always_inline)) { return acc_frag4<BF16>(x); };
                    auto eye_plus = [&](f32x4_t x, float sgn) __attribute__((always_inline)) {
                        f32x4_t y;
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[j] = sgn * x[j] + ((4 * lg + j == ln) ? 1.f : 0.f);
                        return y;
                    };
                    const f32x4_t N2c = mma4<BF16>(z4, f4(Lr), f4(Lc));
                    const f32x4_t N2t = mma4<BF16>(z4, f4(Lc), f4(Lr));
                    const f32x4_t P1c = mma4<BF16>(z4, f4(eye_plus(Lr, -1.f)), f4(eye_plus(N2c, 1.f)));
                    const f32x4_t N4c = mma4<BF16>(z4, f4(N2t), f4(N2c));
                    const f32x4_t N4t = mma4<BF16>(z4, f4(N2c), f4(N2t));
                    const f32x4_t P2c = mma4<BF16>(z4, f4(eye_plus(N4t, 1.f)), f4(P1c));
                    const f32x4_t N8t = mma4<BF16>(z4, f4(N4c), f4(N4t));
                    const f32x4_t Tc = mma4<BF16>(z4, f4(eye_plus(N8t, 1.f)), f4(P2c));  // C layout of T
                    const f32x4_t Tt = mma4<BF16>(z4, f4(P2c), f4(eye_plus(N8t, 1.f)));  // C layout of T^T
                    // lane (ln, lg): Tt -> T[ln][4 lg + j]; Tc -> T^T[ln][4 lg + j]
                    bc_put4<BF16>(tTn + (16 * st + ln) * LB + 4 * lg, -Tt[0], -Tt[1], -Tt[2], -Tt[3]);
                    bc_put4<BF16>(tTt + (16 * st + ln) * LB + 4 * lg, Tc[0], Tc[1], Tc[2], Tc[3]);
                }
            }
            bc_barrier();

            // =============================== CH: the carried gradient's chain
            float bt[NB][4];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
                const float4 b4 = *reinterpret_cast<const float4*>(sBeta + 16 * rt + 4 * lg);
                bt[rt][0] = b4.x;
                bt[rt][1] = b4.y;
                bt[rt][2] = b4.z;
                bt[rt][3] = b4.w;
            }
            // dO as the B operand over the chunk's tokens (C layout of each 16-row block)
            F8 dof8[2];
            F4 dof4[2][NB];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = 32 * w + 16 * ct + ln;
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) dof4[ct][rt][j] = tDO[(16 * rt + 4 * lg + j) * LO + col];
                }
                if constexpr (NB == 2)
                    dof8[ct] = __builtin_shufflevector(dof4[ct][0], dof4[ct][1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
            auto mma_tok = [&](f32x4_t acc, const E* arow, int ld, int ct) __attribute__((always_inline)) {
                if constexpr (NB == 2) return mma8<BF16>(acc, lds_frag8<BF16>(arow, ld, lane), dof8[ct]);
                else return mma4<BF16>(acc, lds_frag4<BF16>(arow, ld, lane), dof4[ct][0]);
            };
            f32x4_t w0f[2][NB];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) w0f[ct][rt] = bc_widen<BF16>(w0c[ct][rt]);
            }
            // Dg = Gamma_C D (rows scaled), as B-operand fragments over the key channels
            F8 dgf[2][KBK];
#pragma unroll
            for (int kb = 0; kb < KBK; ++kb) {
                const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(sGC + 32 * kb + 4 * lg);
                const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(sGC + 32 * kb + 16 + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) dgf[ct][kb] = acc_frag8<BF16>(dS[ct][2 * kb] * g0, dS[ct][2 * kb + 1] * g1);
            }
            // dU = K^ Dg + A^T dO
            f32x4_t dU[2][NB];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) dU[ct][rt] = z4;
#pragma unroll
                for (int kb = 0; kb < KBK; ++kb) {
                    const F8 ka = lds_frag8<BF16>(tKh + 16 * rt * LK + 32 * kb, LK, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) dU[ct][rt] = mma8<BF16>(dU[ct][rt], ka, dgf[ct][kb]);
                }
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) dU[ct][rt] = mma_tok(dU[ct][rt], tAt + 16 * rt * LT, LT, ct);
            }
            // dR = (I + L)^-T dU from the last block: dR_b = T_bb^T (dU_b - sum_{c>b} L_cb^T dR_c)
            f32x4_t dR[2][NB];
            F4 drf[2][NB];
#pragma unroll
            for (int b = NB - 1; b >= 0; --b) {
                const F4 tb = lds_frag4<BF16>(tTt + 16 * b * LB, LB, lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f32x4_t zb = dU[ct][b];
#pragma unroll
                    for (int c = b + 1; c < NB; ++c)
                        zb = mma4<BF16>(zb, lds_frag4<BF16>(tLt + 16 * b * LT + 16 * c, LT, lane), drf[ct][c]);
                    dR[ct][b] = mma4<BF16>(z4, tb, acc_frag4<BF16>(zb));
                    drf[ct][b] = acc_frag4<BF16>(dR[ct][b]);
                }
            }
            // dv = beta dR (fp32, from the C layout: lane holds 4 tokens of one column;
            // rows past the sequence fall outside the buffer range), and the first
            // term of dbeta, sum over this wave's columns of dR * W0
            const int rowDV = H * DV * 4;
            const auto dv_r = buffer_rsrc(a.dv + (static_cast<size_t>(t0) * H + h) * DV, rows * rowDV);
            const int dvo = 4 * lg * rowDV + 4 * (32 * w + ln);
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
                float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        buf_store_f1(dv_r, dvo + 64 * ct, (16 * rt + j) * rowDV, bt[rt][j] * dR[ct][rt][j]);
                        part[j] = __builtin_fmaf(dR[ct][rt][j], w0f[ct][rt][j], part[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float s = row_sum(part[j]);
                    if (ln == 0) sDb[w * C + 16 * rt + 4 * lg + j] = s;
                }
            }
            // publish -dR rows (transposed by the identity product) and Dg rows
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) {
                    const int off = (16 * rt + ln) * LK + 32 * w + 16 * ct + 4 * lg;
                    const f32x4_t tr = mma4<BF16>(z4, drf[ct][rt], eye);
                    bc_put4<BF16>(tDR + off, -tr[0], -tr[1], -tr[2], -tr[3]);
                }
#pragma unroll
                for (int it = 0; it < DK / 16; ++it) {
                    const F4 dg4 = (it & 1) ? F4(__builtin_shufflevector(dgf[ct][it >> 1], dgf[ct][it >> 1], 4, 5, 6, 7))
                                            : F4(__builtin_shufflevector(dgf[ct][it >> 1], dgf[ct][it >> 1], 0, 1, 2, 3));
                    const f32x4_t td = mma4<BF16>(z4, dg4, eye);
                    bc_put4<BF16>(tDS + (16 * it + ln) * LS + 32 * w + 16 * ct + 4 * lg, td[0], td[1], td[2], td[3]);
                }
            }
            // D <- Dg + Q~^T dO - K~^T (beta dR)
            F8 nb8[2];
            F4 nb4[2][NB];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) {
                    f32x4_t x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = -(bt[rt][j] * dR[ct][rt][j]);
                    nb4[ct][rt] = acc_frag4<BF16>(x);
                }
                if constexpr (NB == 2)
                    nb8[ct] = __builtin_shufflevector(nb4[ct][0], nb4[ct][1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int it = 0; it < DK / 16; ++it) {
                const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(sGC + 16 * it + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f32x4_t acc = dS[ct][it] * g4;
                    acc = mma_tok(acc, tQtT + 16 * it * LT, LT, ct);
                    if constexpr (NB == 2)
                        acc = mma8<BF16>(acc, lds_frag8<BF16>(tKtT + 16 * it * LT, LT, lane), nb8[ct]);
                    else
                        acc = mma4<BF16>(acc, lds_frag4<BF16>(tKtT + 16 * it * LT, LT, lane), nb4[ct][0]);
                    dS[ct][it] = acc;
                }
            }
            // stage LB's operands, in flight during stage LA (the registers of
            // stage CH are free again)
            F8 sf0[KBV];
            load_lb0(m, sf0);
            bc_barrier();
            stage_LA();
            bc_barrier();
            stage_LB(m, sf0);
            // the next chunk's dO rows (in flight over the leaf waves' stage P)
            issue_dO(m - 1);
            bc_barrier();
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const size_t col = static_cast<size_t>(32 * w + 16 * ct + ln);
#pragma unroll
            for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a.dS0[pair * DK * DV + static_cast<size_t>(16 * it + 4 * lg + j) * DV + col] = dS[ct][it][j];
            }
        }
    } else {
        issue_strip(nch - 1);
        for (int m = nch - 1; m >= 0; --m) {
            if (m + 1 < nch) flush_sg(m + 1);
            // =============================== P: operand tiles; this chunk's loads
            load_w0(m);  // the first 32-column block of stage U
            F8 sf0[KBV];
            load_lb0(m, sf0);
            if (strip_wave) {
                if (loads_beta) sBeta[lane] = rbeta;
                if (qok) {
                    // log alpha in log2 units: row-group sums, then the exclusive
                    // prefix over the NRG row groups through this wave's scratch
                    float la[4][4], tot[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        la[rr][0] = rla[rr].x;
                        la[rr][1] = rla[rr].y;
                        la[rr][2] = rla[rr].z;
                        la[rr][3] = rla[rr].w;
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) tot[c] = ((la[0][c] + la[1][c]) + (la[2][c] + la[3][c])) * kLog2e;
                    float4* const scan = reinterpret_cast<float4*>(smem + Ly::O_SCAN) + 64 * strip;
                    scan[lane] = make_float4(tot[0], tot[1], tot[2], tot[3]);
                    float g[4] = {0.f, 0.f, 0.f, 0.f}, sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < NRG; ++r) {
                        const float4 t4 = scan[QW * r + cq];
                        const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            g[c] = r < rg ? g[c] + tv[c] : g[c];
                            sum[c] += tv[c];
                        }
                    }
                    if (rg == 0)
                        *reinterpret_cast<float4*>(sGC + i0) =
                            make_float4(__builtin_amdgcn_exp2f(sum[0]), __builtin_amdgcn_exp2f(sum[1]),
                                        __builtin_amdgcn_exp2f(sum[2]), __builtin_amdgcn_exp2f(sum[3]));
                    float kt[4][4], kh4[4][4], qt[4][4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = 4 * rg + rr;
                        float kk[4], qq[4];
                        T::unpack4(rk[rr], kk);
                        T::unpack4(rq[rr], qq);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            g[c] = __builtin_fmaf(la[rr][c], kLog2e, g[c]);
                            const float gm = __builtin_amdgcn_exp2f(g[c]);
                            kt[rr][c] = kk[c] * gm;
                            kh4[rr][c] = kk[c] * __builtin_amdgcn_exp2f(-g[c]);
                            qt[rr][c] = qq[c] * gm;
                        }
                        *reinterpret_cast<float4*>(sG + r * DK + i0) = make_float4(g[0], g[1], g[2], g[3]);
                        bc_put4<BF16>(tKt + r * LK + i0, kt[rr][0], kt[rr][1], kt[rr][2], kt[rr][3]);
                        bc_put4<BF16>(tKh + r * LK + i0, kh4[rr][0], kh4[rr][1], kh4[rr][2], kh4[rr][3]);
                        bc_put4<BF16>(tQt + r * LK + i0, qt[rr][0], qt[rr][1], qt[rr][2], qt[rr][3]);
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int off = (i0 + c) * LT + 4 * rg;
                        bc_put4<BF16>(tKtT + off, kt[0][c], kt[1][c], kt[2][c], kt[3][c]);
                        bc_put4<BF16>(tQtT + off, qt[0][c], qt[1][c], qt[2][c], qt[3][c]);
                        bc_put4<BF16>(tKhT + off, kh4[0][c], kh4[1][c], kh4[2][c], kh4[3][c]);
                    }
                }
            }
            issue_strip(m - 1);
            bc_barrier();
            bc_barrier();  // J (chain waves)

            // =============================== U: (I + L) U = beta W0 (32-column blocks v, v + NL, ...)
            // Only stages LA and LB use U, so it is solved beside stage CH,
            // off the carried gradient's chain.
            for (int cb = v; cb < DV / 32; cb += NL) {
                if (cb != v) load_w0_block(m, cb);
                float bt[NB][4];
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) {
                    const float4 b4 = *reinterpret_cast<const float4*>(sBeta + 16 * rt + 4 * lg);
                    bt[rt][0] = b4.x;
                    bt[rt][1] = b4.y;
                    bt[rt][2] = b4.z;
                    bt[rt][3] = b4.w;
                }
                // U_b = (-T_bb)(-beta W0_b + sum_{c<b} L_bc U_c); each 16 x 16 tile of U
                // goes to LDS as rows (transposed by the identity product)
                F4 uf[2][NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const F4 tb = lds_frag4<BF16>(tTn + 16 * b * LB, LB, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const f32x4_t w0f = bc_widen<BF16>(w0c[ct][b]);
                        f32x4_t y;
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[j] = -(bt[b][j] * w0f[j]);
#pragma unroll
                        for (int c = 0; c < b; ++c)
                            y = mma4<BF16>(y, lds_frag4<BF16>(tL + 16 * b * LT + 16 * c, LT, lane), uf[ct][c]);
                        uf[ct][b] = acc_frag4<BF16>(mma4<BF16>(z4, tb, acc_frag4<BF16>(y)));
                        const f32x4_t tu = mma4<BF16>(z4, uf[ct][b], eye);
                        bc_put4<BF16>(tU + (16 * b + ln) * LK + 32 * cb + 16 * ct + 4 * lg, tu[0], tu[1], tu[2], tu[3]);
                    }
                }
            }
            bc_barrier();
            stage_LA();
            bc_barrier();
            stage_LB(m, sf0);
            bc_barrier();
        }
        if (nch > 0) flush_sg(0);
    }
}

template <bool BF16, int DK, int DV, bool SG>
hipError_t launch_bc_t(const BackwardArgs& b, const void* cks, const void* ckw) {
    constexpr int C = kBcChunk<BF16, DK>;
    using Ly = BcLayout<BF16, DK, DV, C>;
    BcArgs a{b.q, b.k, b.log_alpha, b.beta, b.dO, b.dS_T, b.cu_seqlens, cks, ckw,
             b.dq, b.dk, b.dv, b.dlog_alpha, b.dbeta, b.dS0, b.N, b.H};
    const unsigned grid = static_cast<unsigned>(b.N) * static_cast<unsigned>(b.H);
    hipLaunchKernelGGL((bwd_chunk_kernel<BF16, DK, DV, C, SG>), dim3(grid), dim3(Ly::NT), 0,
                       static_cast<hipStream_t>(b.stream), a);
    return hipGetLastError();
}

template <bool BF16, int DK>
hipError_t launch_bc_dk(const BackwardArgs& b, const void* cks, const void* ckw) {
    switch (b.d_v) {
        case 32: return b.scalar_gate ? launch_bc_t<BF16, DK, 32, true>(b, cks, ckw) : launch_bc_t<BF16, DK, 32, false>(b, cks, ckw);
        case 64: return b.scalar_gate ? launch_bc_t<BF16, DK, 64, true>(b, cks, ckw) : launch_bc_t<BF16, DK, 64, false>(b, cks, ckw);
        case 128: return b.scalar_gate ? launch_bc_t<BF16, DK, 128, true>(b, cks, ckw) : launch_bc_t<BF16, DK, 128, false>(b, cks, ckw);
        default: return hipErrorInvalidValue;
    }
}

int bc_chunk(int32_t d_k, bool bf16) {
    switch (d_k) {
        case 32: return bf16 ? kBcChunk<true, 32> : kBcChunk<false, 32>;
        case 64: return bf16 ? kBcChunk<true, 64> : kBcChunk<false, 64>;
        case 128: return bf16 ? kBcChunk<true, 128> : kBcChunk<false, 128>;
        default: return 0;
    }
}

// checkpoint slots per head: t_beg / C + n + i over every chunk i of every sequence n
size_t bc_slots(int32_t N, int64_t T_tot, int C) { return static_cast<size_t>(T_tot / C + N + 1); }

}  // namespace

size_t prefill_bwd_chunk_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16) {
    const int C = bc_chunk(d_k, bf16);
    if (C == 0) return 0;
    const size_t es = bf16 ? 2 : 4;
    const size_t per = bc_slots(N, T_tot, C) * static_cast<size_t>(H);
    const size_t s_bytes = (per * d_k * d_v * es + 255) / 256 * 256;
    return s_bytes + per * C * d_v * es;
}

hipError_t launch_prefill_bwd_chunk(const BackwardArgs& b) {
    const int C = bc_chunk(b.d_k, b.bf16);
    if (C == 0 || C != prefill_chunk_len(b.d_k, b.bf16)) return hipErrorInvalidValue;
    const size_t es = b.bf16 ? 2 : 4;
    const size_t per = bc_slots(b.N, b.T_tot, C) * static_cast<size_t>(b.H);
    unsigned char* ws = static_cast<unsigned char*>(b.workspace);
    void* cks = ws;
    void* ckw = ws + (per * b.d_k * b.d_v * es + 255) / 256 * 256;
    // pass 1: the forward with checkpoints (no outputs)
    PrefillArgs p{b.q, b.k, b.v, b.log_alpha, b.beta, b.S0, b.cu_seqlens, b.N, b.T_tot, b.H, b.d_k, b.d_v,
                  b.bf16, nullptr, nullptr, 1, b.stream, nullptr, device_cus_or_default(), b.scalar_gate, false, false};
    hipError_t e = launch_prefill_ckpt(p, CkptView{cks, ckw});
    if (e != hipSuccess) return e;
    // pass 2: the reverse walk over the chunks
    switch (b.d_k) {
        case 32: return b.bf16 ? launch_bc_dk<true, 32>(b, cks, ckw) : launch_bc_dk<false, 32>(b, cks, ckw);
        case 64: return b.bf16 ? launch_bc_dk<true, 64>(b, cks, ckw) : launch_bc_dk<false, 64>(b, cks, ckw);
        case 128: return b.bf16 ? launch_bc_dk<true, 128>(b, cks, ckw) : launch_bc_dk<false, 128>(b, cks, ckw);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
