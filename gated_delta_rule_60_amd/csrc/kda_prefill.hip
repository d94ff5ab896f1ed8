// kda_prefill.hip -- chunk-parallel KDA prefill for gfx950.
//
// Recurrence: the update rule of "Kimi Linear：让长上下文大模型真正实用的线性
// 注意力架构" (juejin.cn), section 三.5, with per-channel decay alpha_t
// (section 三.1) and read-out o_t = S_t^T q_t.  Section 三.2 of that page
// states that the specialised diagonal-plus-low-rank transition
// (I - b k k^T) Diag(alpha) admits chunk-parallel evaluation without the
// matrix inverse of general DPLR; the chunk algebra below is derived from
// the recurrence itself and is exact (not an approximation).
//
// Chunk algebra.  Inside a chunk of C tokens (rows r), with S the state
// entering the chunk, g_r = sum_{j<=r} log alpha_j (per key channel),
// Gamma_r = exp(g_r):
//     K~ = K * Gamma,  K^ = K / Gamma,  Q~ = Q * Gamma,  Kbar = K * Gamma_C / Gamma
//     L    = strictly_lower(beta K~ K^T)           (C x C)
//     A_qk = lower_incl(Q~ K^T)                    (C x C)
//     (I + L) U = beta (V - K~ S)                  (U: C x d_v)
//     O      = Q~ S + A_qk U
//     S_next = Diag(Gamma_C) S + Kbar^T U
// (I + L) is unit lower triangular.  Its 16x16 diagonal blocks are inverted
// with MFMA products, T_bb = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8)
// for the nilpotent N = L_bb; U is obtained block by block,
// U_b = T_bb (R_b - sum_{c<b} L_bc U_c), with MFMA products.
// Padded tail rows (past the end of a sequence) carry k = q = v = beta =
// log alpha = 0 and therefore contribute nothing.
//
// Parallel decomposition.  One workgroup per (sequence, head, value slice)
// walks its sequence chunk by chunk.  Each wave owns CT 16-column tiles of
// the state for the whole sequence, in fp32 registers (MFMA C layout); the
// columns of S evolve independently, so the per-column work never leaves the
// wave, and one LDS read of a shared operand feeds CT MFMAs.
//
// Software pipeline.  The S-independent terms of a chunk ("prep") are built
// one chunk ahead of the S-dependent recurrence ("chain"), in the same
// barrier stages, from double-buffered LDS tiles, so that prep's VALU and
// LDS work overlaps the chain's MFMA work.  For chunk i:
//     stage X: prep 1 of i+1: beta, V^T, sums of log alpha | chain of i: R'
//     stage Y: prep 2 of i+1: cumulative decay, decayed tiles; loads of i+2
//                                                          | chain of i: U, O
//     stage Z: prep 3 of i+1: Gram products, block inverse | chain of i: S update,
//                                                            O store
// All MFMA operands are bf16 (or fp32 for f32 inputs); accumulation and the
// carried state are fp32.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr size_t align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// Sequence-length ordering (longest first) is computed in-kernel for up to
// this many sequences; larger batches run in natural order.
constexpr int kSortMax = 64;
constexpr size_t kLdsBudget = 160 * 1024;

template <bool BF16, int DK, int NW, int CT, int C_>
struct Layout {
    using E = typename Elem<BF16>::E;
    static constexpr int C = C_;
    static constexpr int NB = C / 16;
    static constexpr int NT = 64 * NW;
    static constexpr int BV = 16 * CT * NW;
    static constexpr int PAD = 16 / static_cast<int>(sizeof(E));  // 16 bytes of row padding
    static constexpr int LDK = DK + PAD;
    static constexpr int LDC = C + PAD;
    static constexpr int LDV = BV + PAD;
    static constexpr int LDT = 16 + PAD;
    static constexpr size_t ES = sizeof(E);
    // double-buffered tiles
    static constexpr size_t SZ_KB = align16(C * LDK * ES);      // beta K~, Q~  [C][LDK]
    static constexpr size_t SZ_KBT = align16(DK * LDC * ES);    // Kbar^T       [DK][LDC]
    static constexpr size_t SZ_L = align16(C * LDC * ES);       // L, A_qk      [C][LDC]
    static constexpr size_t SZ_T = align16(NB * 16 * LDT * ES);  // -T_bb       [NB][16][LDT]
    static constexpr size_t SZ_VT = align16(BV * LDC * ES);     // V^T          [BV][LDC]
    static constexpr size_t SZ_GC = align16(DK * 4);            // Gamma_C      [DK]
    static constexpr size_t SZ_BETA = align16(C * 4);           // beta         [C]
    static constexpr size_t OFF_KB = 0;
    static constexpr size_t OFF_Q = OFF_KB + 2 * SZ_KB;
    static constexpr size_t OFF_KBT = OFF_Q + 2 * SZ_KB;
    static constexpr size_t OFF_L = OFF_KBT + 2 * SZ_KBT;
    static constexpr size_t OFF_A = OFF_L + 2 * SZ_L;
    static constexpr size_t OFF_T = OFF_A + 2 * SZ_L;
    static constexpr size_t OFF_VT = OFF_T + 2 * SZ_T;
    static constexpr size_t OFF_GC = OFF_VT + 2 * SZ_VT;
    static constexpr size_t OFF_BETA = OFF_GC + 2 * SZ_GC;
    // single-buffered
    static constexpr size_t OFF_KH = OFF_BETA + 2 * SZ_BETA;                 // K^ [C][LDK]
    static constexpr size_t OFF_O = OFF_KH + align16(C * LDK * ES);          // O  [C][LDV]
    static constexpr size_t OFF_TOT = OFF_O + align16(C * LDV * ES);         // group sums [C/4][DK]
    static constexpr size_t OFF_SEQ = OFF_TOT + align16((C / 4) * DK * 4);
    static constexpr size_t BYTES = align16(OFF_SEQ + (kSortMax + 1) * 4);
};

template <bool BF16, int DK, int NW, int CT>
using ChosenLayout =
    Layout<BF16, DK, NW, CT, (Layout<BF16, DK, NW, CT, 32>::BYTES <= kLdsBudget ? 32 : 16)>;

template <bool BF16, int DK, int NW, int CT>
struct PrefillShape : ChosenLayout<BF16, DK, NW, CT> {
    using Base = ChosenLayout<BF16, DK, NW, CT>;
    static_assert(Base::BYTES <= kLdsBudget, "LDS budget of one gfx950 workgroup");
    static constexpr int RG = 4;                // rows per prefix-sum group (fixed)
    static constexpr int NG = Base::C / RG;     // prefix-sum groups per chunk
    static constexpr int QPR = DK / 4;          // channel quads per row
    static constexpr int NITEMS = NG * QPR;     // (group, channel quad) items
    static constexpr int IPT = (NITEMS + Base::NT - 1) / Base::NT;
    static constexpr int VITEMS = (Base::C / 4) * (Base::BV / 4);  // 4x4 blocks of V
    static constexpr int VPT = (VITEMS + Base::NT - 1) / Base::NT;
};

template <bool BF16>
__device__ __forceinline__ void lds_store4(typename Elem<BF16>::E* p, float a, float b, float c, float d) {
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

// 4 consecutive operand elements from LDS, widened to fp32
template <bool BF16>
__device__ __forceinline__ f32x4_t lds_load4(const typename Elem<BF16>::E* p) {
    if constexpr (BF16) {
        const bf16x4_t r = *reinterpret_cast<const bf16x4_t*>(p);
        return f32x4_t{static_cast<float>(r[0]), static_cast<float>(r[1]), static_cast<float>(r[2]),
                       static_cast<float>(r[3])};
    } else {
        return *reinterpret_cast<const f32x4_t*>(p);
    }
}

// Transposes a 4x4 block given as four raw row quads into four column quads.
template <bool BF16>
__device__ __forceinline__ void transpose4(const typename Elem<BF16>::R4 (&rows)[4],
                                           typename Elem<BF16>::R4 (&cols)[4]) {
    if constexpr (BF16) {
        // rows[r] = {x: c0 | c1 << 16, y: c2 | c3 << 16}
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int sh = (c & 1) ? 16 : 0;
            uint32_t e[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) e[r] = (((c < 2) ? rows[r].x : rows[r].y) >> sh) & 0xFFFFu;
            cols[c].x = e[0] | (e[1] << 16);
            cols[c].y = e[2] | (e[3] << 16);
        }
    } else {
        cols[0] = make_float4(rows[0].x, rows[1].x, rows[2].x, rows[3].x);
        cols[1] = make_float4(rows[0].y, rows[1].y, rows[2].y, rows[3].y);
        cols[2] = make_float4(rows[0].z, rows[1].z, rows[2].z, rows[3].z);
        cols[3] = make_float4(rows[0].w, rows[1].w, rows[2].w, rows[3].w);
    }
}

}  // namespace

template <bool BF16, int DK, int NW, int CT>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(
    const typename Elem<BF16>::G* __restrict__ q, const typename Elem<BF16>::G* __restrict__ k,
    const typename Elem<BF16>::G* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, const float* __restrict__ S0, const int32_t* __restrict__ cu,
    int N, int H, int dv, int v_split, typename Elem<BF16>::G* __restrict__ o,
    float* __restrict__ S_T) {
    using Sh = PrefillShape<BF16, DK, NW, CT>;
    using T = Elem<BF16>;
    using E = typename T::E;
    using G = typename T::G;
    using R4 = typename T::R4;
    using F8 = typename T::F8;
    using F4 = typename T::F4;
    constexpr int C = Sh::C, NB = Sh::NB, NT = Sh::NT, BV = Sh::BV;
    constexpr int LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV, LDT = Sh::LDT;
    constexpr int KB = DK / 32;  // 32-deep k blocks over key channels
    constexpr int RG = Sh::RG, NG = Sh::NG, QPR = Sh::QPR, IPT = Sh::IPT, NITEMS = Sh::NITEMS;
    constexpr int VPT = Sh::VPT, VITEMS = Sh::VITEMS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::BYTES];
#define KDA_TILE(name, type, off, sz) \
    auto name = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<type*>(smem + (off) + b * (sz)); }
    KDA_TILE(tKb, E, Sh::OFF_KB, Sh::SZ_KB);
    KDA_TILE(tQ, E, Sh::OFF_Q, Sh::SZ_KB);
    KDA_TILE(tKbT, E, Sh::OFF_KBT, Sh::SZ_KBT);
    KDA_TILE(tL, E, Sh::OFF_L, Sh::SZ_L);
    KDA_TILE(tA, E, Sh::OFF_A, Sh::SZ_L);
    KDA_TILE(tT, E, Sh::OFF_T, Sh::SZ_T);
    KDA_TILE(tVt, E, Sh::OFF_VT, Sh::SZ_VT);
    KDA_TILE(sGC, float, Sh::OFF_GC, Sh::SZ_GC);
    KDA_TILE(sBeta, float, Sh::OFF_BETA, Sh::SZ_BETA);
#undef KDA_TILE
    E* const tKh = reinterpret_cast<E*>(smem + Sh::OFF_KH);
    E* const tO = reinterpret_cast<E*>(smem + Sh::OFF_O);
    float* const sTot = reinterpret_cast<float*>(smem + Sh::OFF_TOT);
    int* const sSeq = reinterpret_cast<int*>(smem + Sh::OFF_SEQ);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lg = lane >> 4;

    // ---- work assignment -------------------------------------------------
    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs.
    // Units (sequence, head) are laid out so the value slices of one unit run
    // back to back on the same XCD (shared q/k/log alpha lines in its L2),
    // and lower unit ids (dispatched first) are the longer sequences.
    int unit, slice;
    {
        const int b = blockIdx.x;
        const int units = N * H;
        if ((units & 7) == 0) {
            const int x = b & 7, qq = b >> 3;
            unit = 8 * (qq / v_split) + x;
            slice = qq % v_split;
        } else {
            unit = b / v_split;
            slice = b % v_split;
        }
    }
    const int h = unit % H;
    const int rank = unit / H;
    int n = rank;
    if (N > 1 && N <= kSortMax) {
        for (int i = tid; i < N; i += NT) sSeq[i] = cu[i + 1] - cu[i];
        __syncthreads();
        for (int i = tid; i < N; i += NT) {
            const int li = sSeq[i];
            int r = 0;
            for (int j = 0; j < N; ++j) {
                const int lj = sSeq[j];
                r += (lj > li) || (lj == li && j < i);
            }
            if (r == rank) sSeq[kSortMax] = i;
        }
        __syncthreads();
        n = sSeq[kSortMax];
    }
    const int t_beg = cu[n];
    const int t_end = cu[n + 1];
    const int nchunks = (t_end - t_beg + C - 1) / C;
    const int j0 = slice * BV;  // first value column of this workgroup
    const size_t pair = static_cast<size_t>(n) * H + h;

    // Per-head base pointers; per-token offsets below fit in 32 bits (the
    // host rejects tensors of 2^31 elements or more).
    const int strideK = H * DK;
    const int strideV = H * dv;
    const G* const qh = q + static_cast<size_t>(h) * DK;
    const G* const kh = k + static_cast<size_t>(h) * DK;
    const float* const lah = log_alpha + static_cast<size_t>(h) * DK;
    const float* const bh = beta + h;
    const G* const vh = v + static_cast<size_t>(h) * dv + j0;
    G* const oh = o + static_cast<size_t>(h) * dv + j0;

    // Upper block-triangles of L and A_qk stay zero for the whole kernel.
    for (int idx = tid; idx < C * LDC; idx += NT) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            tL(b)[idx] = T::to_e(0.f);
            tA(b)[idx] = T::to_e(0.f);
        }
    }

    // ---- state slice in registers: Sr[ct][it][j] = S[16 it + 4 lg + j][col]
    auto col0 = [&](int ct) __attribute__((always_inline)) { return 16 * (CT * wave + ct); };
    f32x4_t Sr[CT][DK / 16];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const size_t col = static_cast<size_t>(j0 + col0(ct) + ln);
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sr[ct][it][j] = S0 ? S0[(pair * DK + 16 * it + 4 * lg + j) * dv + col] : 0.f;
        }
    }

    // ---- raw inputs of one chunk, in registers -----------------------------
    // Every load is unconditional: rows past the end of the sequence read the
    // last valid row (always in bounds) and are zeroed where they are used.
    float4 rla[IPT][RG];
    R4 rk[IPT][RG], rq[IPT][RG], rv[VPT][4];
    float rb = 0.f;
    auto load_chunk = [&](int c0, int len) __attribute__((always_inline)) {
        const int last = len - 1;
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int it = tid + NT * ii;
            if (NITEMS % NT == 0 || it < NITEMS) {
                const int grp = it / QPR;
                const int i0 = 4 * (it % QPR);
#pragma unroll
                for (int rr = 0; rr < RG; ++rr) {
                    const int off = (c0 + min(grp * RG + rr, last)) * strideK + i0;
                    rla[ii][rr] = *reinterpret_cast<const float4*>(lah + off);
                    rk[ii][rr] = T::raw4(kh + off);
                    rq[ii][rr] = T::raw4(qh + off);
                }
            }
        }
#pragma unroll
        for (int vv = 0; vv < VPT; ++vv) {
            const int idx = tid + NT * vv;
            if (VITEMS % NT == 0 || idx < VITEMS) {
                const int r0 = 4 * (idx / (BV / 4));
                const int c4 = 4 * (idx % (BV / 4));
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    rv[vv][rr] = T::raw4(vh + (c0 + min(r0 + rr, last)) * strideV + c4);
            }
        }
        if (tid < C) rb = bh[(c0 + min(tid, last)) * H];
    };

    // ---- prep 1: beta, V^T, group sums of log alpha ------------------------
    auto prep1 = [&](int B, int len) __attribute__((always_inline)) {
        if (tid < C) sBeta(B)[tid] = (tid < len) ? rb : 0.f;
#pragma unroll
        for (int vv = 0; vv < VPT; ++vv) {
            const int idx = tid + NT * vv;
            if (VITEMS % NT == 0 || idx < VITEMS) {
                const int r0 = 4 * (idx / (BV / 4));
                const int c4 = 4 * (idx % (BV / 4));
                R4 rows[4], cols[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rows[rr] = (r0 + rr < len) ? rv[vv][rr] : R4{};
                transpose4<BF16>(rows, cols);
#pragma unroll
                for (int c = 0; c < 4; ++c) T::lds_put_raw4(tVt(B) + (c4 + c) * LDC + r0, cols[c]);
            }
        }
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int it = tid + NT * ii;
            if (NITEMS % NT == 0 || it < NITEMS) {
                const int grp = it / QPR;
                const int i0 = 4 * (it % QPR);
                float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int rr = 0; rr < RG; ++rr) {
                    const bool ok = grp * RG + rr < len;
                    tot.x += ok ? rla[ii][rr].x : 0.f;
                    tot.y += ok ? rla[ii][rr].y : 0.f;
                    tot.z += ok ? rla[ii][rr].z : 0.f;
                    tot.w += ok ? rla[ii][rr].w : 0.f;
                }
                *reinterpret_cast<float4*>(sTot + grp * DK + i0) = tot;
            }
        }
    };

    // ---- prep 2: cumulative decay and decayed operand tiles ----------------
    auto prep2_item = [&](auto full, int ii, int B, int len) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        const int it = tid + NT * ii;
        const int grp = it / QPR;
        const int i0 = 4 * (it % QPR);
        // g = sum of the group sums before this group; g_C = sum of all of
        // them; both in the same fixed order for every launch shape.
        float g[4] = {0.f, 0.f, 0.f, 0.f}, gcs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NG; ++p) {
            const float4 sm = *reinterpret_cast<const float4*>(sTot + p * DK + i0);
            const bool before = p < grp;
            g[0] += before ? sm.x : 0.f;
            g[1] += before ? sm.y : 0.f;
            g[2] += before ? sm.z : 0.f;
            g[3] += before ? sm.w : 0.f;
            gcs[0] += sm.x;
            gcs[1] += sm.y;
            gcs[2] += sm.z;
            gcs[3] += sm.w;
        }
        float Gc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) Gc[c] = __builtin_amdgcn_exp2f(gcs[c] * kLog2e);
        if (grp == 0) *reinterpret_cast<float4*>(sGC(B) + i0) = make_float4(Gc[0], Gc[1], Gc[2], Gc[3]);
        float kbar[RG][4];
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
            const int r = grp * RG + rr;
            const bool ok = FULL || r < len;
            float kk[4], qq[4];
            T::unpack4(rk[ii][rr], kk);
            T::unpack4(rq[ii][rr], qq);
            const float4 a = rla[ii][rr];
            g[0] += ok ? a.x : 0.f;
            g[1] += ok ? a.y : 0.f;
            g[2] += ok ? a.z : 0.f;
            g[3] += ok ? a.w : 0.f;
            const float b = sBeta(B)[r];
            float gam[4], inv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (!FULL && !ok) {
                    kk[c] = 0.f;
                    qq[c] = 0.f;
                }
                // exp(+-g) as 2^(+-g log2 e): one v_exp_f32 each; |g| stays
                // within the numerical contract, where results are normal.
                const float gl = g[c] * kLog2e;
                gam[c] = __builtin_amdgcn_exp2f(gl);
                inv[c] = __builtin_amdgcn_exp2f(-gl);
                kbar[rr][c] = kk[c] * (Gc[c] * inv[c]);
            }
            const float bk0 = b * kk[0], bk1 = b * kk[1], bk2 = b * kk[2], bk3 = b * kk[3];
            lds_store4<BF16>(tKb(B) + r * LDK + i0, bk0 * gam[0], bk1 * gam[1], bk2 * gam[2], bk3 * gam[3]);
            lds_store4<BF16>(tKh + r * LDK + i0, kk[0] * inv[0], kk[1] * inv[1], kk[2] * inv[2],
                             kk[3] * inv[3]);
            lds_store4<BF16>(tQ(B) + r * LDK + i0, qq[0] * gam[0], qq[1] * gam[1], qq[2] * gam[2],
                             qq[3] * gam[3]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            lds_store4<BF16>(tKbT(B) + (i0 + c) * LDC + grp * RG, kbar[0][c], kbar[1][c], kbar[2][c],
                             kbar[3][c]);
    };
    auto prep2 = [&](int B, int len) __attribute__((always_inline)) {
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            if (NITEMS % NT == 0 || tid + NT * ii < NITEMS) {
                if (len == C) {
                    prep2_item(std::true_type{}, ii, B, len);
                } else {
                    prep2_item(std::false_type{}, ii, B, len);
                }
            }
        }
    };

    // ---- prep 3: Gram products and block inverse ---------------------------
    // Job (st, rt), st <= rt, computes the tiles at block (rt, st) of
    // L = strictly_lower(beta K~ K^T) and A_qk = lower_incl(Q~ K^T), sharing
    // the K^ operand.  They are computed transposed, P[s][r] = K^_s . X_r, so
    // that each lane's four C-layout values are four consecutive columns of
    // row r.
    //
    // A diagonal job also forms -T_bb = -(I + N)^-1, N = L_bb (strictly lower,
    // nilpotent: N^16 = 0), as the product (I - N)(I + N^2)(I + N^4)(I + N^8),
    // with MFMA.  The factors are polynomials in N and commute, so every
    // product can take its A operand from a C-layout tile already held:
    // the A operand of X is the C layout of X^T, the B operand of X is the C
    // layout of X.  Both layouts of N come from the Gram MFMAs (P and P^T).
    auto prep3 = [&](int B) __attribute__((always_inline)) {
        constexpr int NJOB = NB * (NB + 1) / 2;
        for (int job = NW - 1 - wave; job < NJOB; job += NW) {
            int st, rt;
            if (job < NB) {
                st = rt = job;
            } else {
                int tix = job - NB;  // enumerate st < rt
                rt = 1;
                while (tix >= rt) {
                    tix -= rt;
                    ++rt;
                }
                st = tix;
            }
            const bool diag = st == rt;
            const E* Ab = tKh + 16 * st * LDK;
            const E* Bk = tKb(B) + 16 * rt * LDK;
            const E* Bq = tQ(B) + 16 * rt * LDK;
            f32x4_t accL = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f}, accN = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const F8 a = lds_frag8<BF16>(Ab + 32 * kb, LDK, lane);
                const F8 bk = lds_frag8<BF16>(Bk + 32 * kb, LDK, lane);
                accL = mma8<BF16>(accL, a, bk);
                accA = mma8<BF16>(accA, a, lds_frag8<BF16>(Bq + 32 * kb, LDK, lane));
                if (diag) accN = mma8<BF16>(accN, bk, a);  // P^T: C layout of N
            }
            const int r = 16 * rt + ln;
            float vl[4], va[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s2 = 16 * st + 4 * lg + j;
                vl[j] = (s2 < r) ? accL[j] : 0.f;
                va[j] = (s2 <= r) ? accA[j] : 0.f;
            }
            lds_store4<BF16>(tL(B) + r * LDC + 16 * st + 4 * lg, vl[0], vl[1], vl[2], vl[3]);
            lds_store4<BF16>(tA(B) + r * LDC + 16 * st + 4 * lg, va[0], va[1], va[2], va[3]);
            if (diag) {
                // C layout: lane (ln, lg), value j is element (row 4 lg + j, col ln).
                f32x4_t Nt, Nc;  // C layouts of N^T and N (strictly lower N)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Nt[j] = vl[j];
                    Nc[j] = (ln < 4 * lg + j) ? accN[j] : 0.f;
                }
                auto eye = [&](f32x4_t x, float sgn) __attribute__((always_inline)) {
                    f32x4_t y;
#pragma unroll
                    for (int j = 0; j < 4; ++j) y[j] = sgn * x[j] + ((4 * lg + j == ln) ? 1.f : 0.f);
                    return y;
                };
                const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
                const f32x4_t N2 = mma4<BF16>(z, acc_frag4<BF16>(Nt), acc_frag4<BF16>(Nc));
                const f32x4_t N2t = mma4<BF16>(z, acc_frag4<BF16>(Nc), acc_frag4<BF16>(Nt));
                const f32x4_t N4 = mma4<BF16>(z, acc_frag4<BF16>(N2t), acc_frag4<BF16>(N2));
                const f32x4_t N4t = mma4<BF16>(z, acc_frag4<BF16>(N2), acc_frag4<BF16>(N2t));
                const f32x4_t N8 = mma4<BF16>(z, acc_frag4<BF16>(N4t), acc_frag4<BF16>(N4));
                // Q1 = (I + N8^T)(I + N4^T), Q2 = (I + N2^T) Q1, Q3 = (I - N^T) Q2 = T^T
                const f32x4_t Q1 = mma4<BF16>(z, acc_frag4<BF16>(eye(N8, 1.f)), acc_frag4<BF16>(eye(N4t, 1.f)));
                const f32x4_t Q2 = mma4<BF16>(z, acc_frag4<BF16>(eye(N2, 1.f)), acc_frag4<BF16>(Q1));
                const f32x4_t Q3 = mma4<BF16>(z, acc_frag4<BF16>(eye(Nc, -1.f)), acc_frag4<BF16>(Q2));
                // lane (ln, lg) holds T[ln][4 lg + j]: store -T row-major
                lds_store4<BF16>(tT(B) + (rt * 16 + ln) * LDT + 4 * lg, -Q3[0], -Q3[1], -Q3[2], -Q3[3]);
            }
        }
    };

    // ---- chain: per-wave column recurrence of the chunk in buffer B ---------
    F8 sf[CT][KB];
    f32x4_t Rp[CT][NB], U[CT][NB];
    F4 uf[CT][NB];

    // R' = beta K~ S - beta V  (= -R)
    auto chain_R = [&](int B) __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sf[ct][kb] = acc_frag8<BF16>(Sr[ct][2 * kb], Sr[ct][2 * kb + 1]);
        }
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            const float4 b4 = *reinterpret_cast<const float4*>(sBeta(B) + 16 * rt + 4 * lg);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const f32x4_t v4 = lds_load4<BF16>(tVt(B) + (col0(ct) + ln) * LDC + 16 * rt + 4 * lg);
                Rp[ct][rt] = f32x4_t{-b4.x * v4[0], -b4.y * v4[1], -b4.z * v4[2], -b4.w * v4[3]};
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const F8 a = lds_frag8<BF16>(tKb(B) + 16 * rt * LDK + 32 * kb, LDK, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Rp[ct][rt] = mma8<BF16>(Rp[ct][rt], a, sf[ct][kb]);
            }
        }
    };
    auto u_frag8 = [&](int ct, int b) __attribute__((always_inline)) {
        return F8(__builtin_shufflevector(uf[ct][b], uf[ct][b + 1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // U_b = (-T_bb) (R'_b + sum_{c<b} L_bc U_c);  then O^T = S^T Q~^T + U^T A_qk^T
    auto chain_UO = [&](int B) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4_t Y[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Y[ct] = Rp[ct][b];
#pragma unroll
            for (int kp = 0; kp + 1 < b; kp += 2) {
                const F8 a = lds_frag8<BF16>(tL(B) + 16 * b * LDC + 16 * kp, LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Y[ct] = mma8<BF16>(Y[ct], a, u_frag8(ct, kp));
            }
            if (b & 1) {
                const F4 a = lds_frag4<BF16>(tL(B) + 16 * b * LDC + 16 * (b - 1), LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Y[ct] = mma4<BF16>(Y[ct], a, uf[ct][b - 1]);
            }
            const F4 tb = lds_frag4<BF16>(tT(B) + 16 * b * LDT, LDT, lane);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                U[ct][b] = mma4<BF16>(z, tb, acc_frag4<BF16>(Y[ct]));
                uf[ct][b] = acc_frag4<BF16>(U[ct][b]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            f32x4_t acc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const F8 bq = lds_frag8<BF16>(tQ(B) + 16 * rt * LDK + 32 * kb, LDK, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mma8<BF16>(acc[ct], sf[ct][kb], bq);
            }
#pragma unroll
            for (int sp = 0; sp + 1 <= rt; sp += 2) {
                const F8 ba = lds_frag8<BF16>(tA(B) + 16 * rt * LDC + 16 * sp, LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mma8<BF16>(acc[ct], u_frag8(ct, sp), ba);
            }
            if (!(rt & 1)) {
                const F4 ba = lds_frag4<BF16>(tA(B) + 16 * rt * LDC + 16 * rt, LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mma4<BF16>(acc[ct], uf[ct][rt], ba);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                lds_store4<BF16>(tO + (16 * rt + ln) * LDV + col0(ct) + 4 * lg, acc[ct][0], acc[ct][1],
                                 acc[ct][2], acc[ct][3]);
        }
    };
    // S <- Diag(Gamma_C) S + Kbar^T U
    auto chain_S = [&](int B) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
            const float4 g4 = *reinterpret_cast<const float4*>(sGC(B) + 16 * it + 4 * lg);
            f32x4_t acc[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                acc[ct] = f32x4_t{Sr[ct][it][0] * g4.x, Sr[ct][it][1] * g4.y, Sr[ct][it][2] * g4.z,
                                  Sr[ct][it][3] * g4.w};
#pragma unroll
            for (int kb = 0; kb < NB / 2; ++kb) {
                const F8 a = lds_frag8<BF16>(tKbT(B) + 16 * it * LDC + 32 * kb, LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mma8<BF16>(acc[ct], a, u_frag8(ct, 2 * kb));
            }
            if constexpr (NB & 1) {
                const F4 a = lds_frag4<BF16>(tKbT(B) + 16 * it * LDC + 16 * (NB - 1), LDC, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = mma4<BF16>(acc[ct], a, uf[ct][NB - 1]);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Sr[ct][it] = acc[ct];
        }
    };
    // coalesced store of the chunk's outputs
    auto store_O = [&](int c0, int len) __attribute__((always_inline)) {
        for (int idx = tid; idx < len * (BV / 4); idx += NT) {
            const int r = idx / (BV / 4);
            const int cq = idx % (BV / 4);
            G* dst = oh + (c0 + r) * strideV + 4 * cq;
            if constexpr (BF16) {
                *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(tO + r * LDV + 4 * cq);
            } else {
                *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(tO + r * LDV + 4 * cq);
            }
        }
    };
    auto chunk_len = [&](int i) __attribute__((always_inline)) { return min(C, t_end - (t_beg + i * C)); };

    // ---- prologue: prep 1-3 of chunk 0 ---------------------------------------
    __syncthreads();  // zeroed L / A_qk tiles
    if (nchunks > 0) {
        load_chunk(t_beg, chunk_len(0));
        prep1(0, chunk_len(0));
        __syncthreads();
        prep2(0, chunk_len(0));
        if (nchunks > 1) load_chunk(t_beg + C, chunk_len(1));
        __syncthreads();
        prep3(0);
        __syncthreads();
    }

    // ---- steady state: chunk i in buffer i & 1, prep of chunk i+1 in the other
    for (int i = 0; i < nchunks; ++i) {
        const int B = i & 1;
        const bool has_next = i + 1 < nchunks;
        const int len1 = has_next ? chunk_len(i + 1) : 0;
        // stage X
        if (has_next) prep1(1 - B, len1);
        chain_R(B);
        __syncthreads();
        // stage Y
        if (has_next) {
            prep2(1 - B, len1);
            if (i + 2 < nchunks) load_chunk(t_beg + (i + 2) * C, chunk_len(i + 2));
        }
        chain_UO(B);
        __syncthreads();
        // stage Z
        if (has_next) prep3(1 - B);
        chain_S(B);
        store_O(t_beg + i * C, chunk_len(i));
        __syncthreads();
    }

    // ---- final state --------------------------------------------------------
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const size_t col = static_cast<size_t>(j0 + col0(ct) + ln);
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) S_T[(pair * DK + 16 * it + 4 * lg + j) * dv + col] = Sr[ct][it][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Host launchers.  The workgroup shape follows the value slice width
// BV = d_v / v_split: 4 waves x 2 tiles (128), 4 x 1 (64), 2 x 1 (32), 1 x 1 (16).
// ---------------------------------------------------------------------------
template <bool BF16, int DK, int NW, int CT>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
    using G = typename Elem<BF16>::G;
    const unsigned grid = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H) *
                          static_cast<unsigned>(a.v_split);
    hipLaunchKernelGGL((prefill_kernel<BF16, DK, NW, CT>), dim3(grid), dim3(64 * NW), 0,
                       static_cast<hipStream_t>(a.stream), static_cast<const G*>(a.q),
                       static_cast<const G*>(a.k), static_cast<const G*>(a.v), a.log_alpha, a.beta,
                       a.S0, a.cu_seqlens, a.N, a.H, a.d_v, a.v_split, static_cast<G*>(a.o), a.S_T);
    return hipGetLastError();
}

template <bool BF16, int DK>
static hipError_t launch_prefill_dk(const PrefillArgs& a) {
    switch (a.d_v / a.v_split) {
        case 128: return launch_prefill_t<BF16, DK, 4, 2>(a);
        case 64: return launch_prefill_t<BF16, DK, 4, 1>(a);
        case 32: return launch_prefill_t<BF16, DK, 2, 1>(a);
        case 16: return launch_prefill_t<BF16, DK, 1, 1>(a);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
static hipError_t launch_prefill_dt(const PrefillArgs& a) {
    switch (a.d_k) {
        case 32: return launch_prefill_dk<BF16, 32>(a);
        case 64: return launch_prefill_dk<BF16, 64>(a);
        case 128: return launch_prefill_dk<BF16, 128>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs& a) {
    return a.bf16 ? launch_prefill_dt<true>(a) : launch_prefill_dt<false>(a);
}

int32_t default_v_split(int32_t N, int32_t H, int32_t d_k, int32_t d_v, bool bf16) {
    (void)d_k;
    (void)bf16;
    const int64_t units = static_cast<int64_t>(N) * H;
    int32_t split = 1;
    // Aim for at least ~192 workgroups on the 256 CUs; every split shares the
    // same per-column arithmetic, so this only changes the launch shape.
    while (units * split < 192 && split < 8 && d_v / (split * 2) >= 16) split *= 2;
    return split;
}

}  // namespace kda
