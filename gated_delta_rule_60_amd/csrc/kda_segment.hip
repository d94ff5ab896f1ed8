// kda_segment.hip -- segmented prefill for long sequences: the plan of
// segments and the fix-up passes that chain them.
//
// The recurrence of "Kimi Linear：让长上下文大模型真正实用的线性注意力架构",
// section 三.5, is affine in the entering state: over a segment of tokens,
// S_out = M S_in + D and o_t = o_t^0 + S_in^T q^_t, where D and o^0 are the
// segment's final state and outputs from S_in = 0, M is the product of the
// segment's transitions and q^_t = M_t^T q_t with M_t the product up to token
// t.  Running the same recurrence with V = 0 and S_in = I (the identity run)
// gives M as its final state and q^_t as its outputs.  The prefill kernel
// runs every segment of every head (and the identity runs) in parallel; the
// fix-up here chains the segments of each long sequence:
//
//     S_in(1) = final state of segment 0,
//     S_in(s+1) = M(s) S_in(s) + D(s),   S_T = S_in(P)     (state chain, in order)
//     O(s) += q^(s) S_in(s)                                  (output correction)
//
// The state chain is sequential over segments and splits the independent
// columns of S over workgroups; the output correction is parallel over
// segments, heads and token tiles.
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanSortMax = 64;  // sequences ordered by length (longest first) up to this many
constexpr int kFixCols = 32;      // value columns per state-chain workgroup
constexpr int kFixThreads = 256;  // threads per output-correction workgroup
constexpr int kOutTokens = 512;  // tokens per output fix-up workgroup
constexpr int kOutGroups = 8;    // output workgroups per (segment, head)
static_assert(kSegTokens % kOutTokens == 0, "output tiles cover a segment");

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct SegLayout {
    int umax, lmax;
    size_t off_units, off_longs, off_qhat, off_m, off_d, bytes;
};

// Workspace: {count, nlong} | units [umax] | longs [lmax] | q^ | M | D
SegLayout seg_layout(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16) {
    SegLayout L{};
    const int64_t full = seg_units_max(N, T_tot) - N;  // segments beyond one per sequence, at most
    L.umax = static_cast<int>(N + full);
    L.lmax = static_cast<int>(full < N ? (full > 0 ? full : 1) : N);
    const size_t es = bf16 ? 2 : 4;
    L.off_units = 256;
    L.off_longs = L.off_units + align256(static_cast<size_t>(L.umax) * 16);
    L.off_qhat = L.off_longs + align256(static_cast<size_t>(L.lmax) * 16);
    L.off_m = L.off_qhat + align256(static_cast<size_t>(T_tot) * H * d_k * es);
    L.off_d = L.off_m + align256(static_cast<size_t>(L.umax) * H * d_k * d_k * 4);
    L.bytes = L.off_d + align256(static_cast<size_t>(L.umax) * H * d_k * d_v * 4);
    return L;
}

// Segment length of a sequence of len tokens: a quarter of it, rounded up to
// a multiple of the output tile (512), within [kSegMinTokens, kSegTokens].
// It depends on len alone, so a sequence is cut the same way in any batch
// that runs segmented.
__device__ __forceinline__ int seg_len_for(int len) {
    const int q = ((len + 3) / 4 + kOutTokens - 1) / kOutTokens * kOutTokens;
    return q < kSegMinTokens ? kSegMinTokens : (q > kSegTokens ? kSegTokens : q);
}
static_assert(kSegMinTokens % kOutTokens == 0 && kSegTokens % kOutTokens == 0, "segments of whole output tiles");

// ---------------------------------------------------------------------------
// Plan: one workgroup.  Sequences are taken longest first (up to
// kPlanSortMax of them; natural order beyond), each split into
// ceil(len / seg_len_for(len)) segments (one for an empty sequence); units
// list the segments in that order, longs the sequences with two or more.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void seg_plan_kernel(const int32_t* __restrict__ cu, int N,
                                                              int4* __restrict__ units,
                                                              int* __restrict__ counts,
                                                              int4* __restrict__ longs, int umax,
                                                              int lmax) {
    __shared__ int sLen[kPlanSortMax], sOrder[kPlanSortMax];
    __shared__ int sScanA[kPlanThreads], sScanB[kPlanThreads];
    __shared__ int sCarry[2];
    const int tid = threadIdx.x;
    const bool sorted = N > 1 && N <= kPlanSortMax;
    if (sorted) {
        for (int i = tid; i < N; i += kPlanThreads) sLen[i] = cu[i + 1] - cu[i];
        __syncthreads();
        for (int i = tid; i < N; i += kPlanThreads) {
            const int li = sLen[i];
            int r = 0;
            for (int j = 0; j < N; ++j) {
                const int lj = sLen[j];
                r += (lj > li) || (lj == li && j < i);
            }
            sOrder[r] = i;
        }
    }
    if (tid == 0) {
        sCarry[0] = 0;
        sCarry[1] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += kPlanThreads) {
        const int r = base + tid;
        int n = 0, len = 0, P = 0, seg = kSegTokens;
        if (r < N) {
            n = sorted ? sOrder[r] : r;
            len = cu[n + 1] - cu[n];
            seg = seg_len_for(len);
            P = len > seg ? (len + seg - 1) / seg : 1;
        }
        // inclusive scans of the segment counts and of the long-sequence flags
        sScanA[tid] = P;
        sScanB[tid] = P >= 2 ? 1 : 0;
        __syncthreads();
        for (int d = 1; d < kPlanThreads; d *= 2) {
            const int a = tid >= d ? sScanA[tid - d] : 0;
            const int b = tid >= d ? sScanB[tid - d] : 0;
            __syncthreads();
            sScanA[tid] += a;
            sScanB[tid] += b;
            __syncthreads();
        }
        const int u0 = sCarry[0] + sScanA[tid] - P;
        const int l0 = sCarry[1] + sScanB[tid] - (P >= 2 ? 1 : 0);
        if (r < N) {
            const int t0 = cu[n], t1 = cu[n + 1];
            // (bounds hold for valid offsets; the guards keep malformed ones in the workspace)
            for (int s = 0; s < P && u0 + s < umax; ++s) {
                const int a = t0 + s * seg;
                units[u0 + s] = make_int4(n, s, a, min(t1, a + seg));
            }
            if (P >= 2 && l0 < lmax && u0 + P <= umax) longs[l0] = make_int4(n, u0, P, 0);
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) {
            sCarry[0] += sScanA[tid];
            sCarry[1] += sScanB[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        counts[0] = min(sCarry[0], umax);
        counts[1] = min(sCarry[1], lmax);
    }
}

// ---------------------------------------------------------------------------
// State chain: one workgroup per (long sequence, head, 32 value columns).
// The entering state of segment 1 is the final state of segment 0 (written
// to S_T by the prefill kernel); for s = 1 .. P-1
//     S_in(s+1) = M(s) S_in(s) + D(s)            (fp32 MFMA, fp32 state)
// and S_in(s) replaces D(s) in the workspace for the output pass.  The last
// state is the sequence's final state.  One wave per 16x16 tile of the
// [DK][32] state slice; M(s+1) and D(s+1) are fetched into registers while
// step s computes.
// ---------------------------------------------------------------------------
template <int DK>
struct ChainShape {
    static constexpr int NT = 64 * (DK / 16) * (kFixCols / 16);  // one wave per tile
    static constexpr int MQ = DK * DK / 4 / NT;                 // float4 of M per thread
    static constexpr int SQ = DK * kFixCols / 4 / NT;           // float4 of the state slice per thread
};

template <int DK>
__global__ __launch_bounds__(ChainShape<DK>::NT) void seg_chain_kernel(const int* __restrict__ counts,
                                                                      const int4* __restrict__ longs,
                                                                      const float* __restrict__ mstate,
                                                                      float* __restrict__ dstate, int H,
                                                                      int dv, float* __restrict__ S_T) {
    constexpr int CS = kFixCols;
    constexpr int LDM = DK + 4;  // padded rows of M
    constexpr int NT = ChainShape<DK>::NT, MQ = ChainShape<DK>::MQ, SQ = ChainShape<DK>::SQ;
    static_assert(DK % 32 == 0 && DK <= 128 && MQ >= 1 && SQ == 1, "chain tiling");
    __shared__ __attribute__((aligned(16))) float sM[DK * LDM];
    __shared__ __attribute__((aligned(16))) float sS[DK * CS];

    const int nsl = dv / CS;
    const int w = blockIdx.x;
    const int l = w / (H * nsl);
    const int h = (w / nsl) % H;
    const int c0 = (w % nsl) * CS;
    if (l >= counts[1]) return;  // whole workgroup: before any barrier
    const int4 lg4 = longs[l];
    const int n = lg4.x, u0 = lg4.y, P = lg4.z;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lgp = lane >> 4;
    const int r0 = 16 * (wave >> 1);  // this wave's tile: rows r0.., columns cc..
    const int cc = 16 * (wave & 1);
    float* const Sblk = S_T + (static_cast<size_t>(n) * H + h) * DK * dv + c0;
    const size_t mstride = static_cast<size_t>(H) * DK * DK;  // next segment, same head
    const size_t dstride = static_cast<size_t>(H) * DK * dv;
    const float4* Mg = reinterpret_cast<const float4*>(mstate + (static_cast<size_t>(u0 + 1) * H + h) * DK * DK);
    float* Dg = dstate + (static_cast<size_t>(u0 + 1) * H + h) * DK * dv + c0;

    // M prefetch in four named registers (an indexed array of them would be
    // placed in LDS by the compiler's alloca promotion)
    static_assert(MQ == 1 || MQ == 2 || MQ == 4, "M prefetch registers");
    float4 m0, m1, m2, m3;
#define KDA_LOAD_M()                                   \
    {                                                  \
        m0 = Mg[tid];                                  \
        if constexpr (MQ > 1) m1 = Mg[tid + NT];       \
        if constexpr (MQ > 2) m2 = Mg[tid + 2 * NT];   \
        if constexpr (MQ > 2) m3 = Mg[tid + 3 * NT];   \
    }
#define KDA_STORE_M(k, reg)                                                          \
    if constexpr (MQ > k) {                                                          \
        const int i = 4 * (tid + k * NT);                                            \
        *reinterpret_cast<float4*>(sM + (i / DK) * LDM + i % DK) = reg;              \
    }
    float dreg[4];
    KDA_LOAD_M()
#pragma unroll
    for (int j = 0; j < 4; ++j) dreg[j] = Dg[static_cast<size_t>(r0 + 4 * lgp + j) * dv + cc + ln];
    {
        const int i = 4 * tid;
        *reinterpret_cast<float4*>(sS + i) = *reinterpret_cast<const float4*>(Sblk + (i / CS) * dv + i % CS);
    }

    for (int s = 1; s < P; ++s) {
        __syncthreads();  // sS complete; every wave is done reading the last sM
        KDA_STORE_M(0, m0)
        KDA_STORE_M(1, m1)
        KDA_STORE_M(2, m2)
        KDA_STORE_M(3, m3)
        f32x4_t acc = {dreg[0], dreg[1], dreg[2], dreg[3]};
        __syncthreads();
        if (s + 1 < P) {  // M(s+1), D(s+1): in flight during the products
            Mg += mstride / 4;
            KDA_LOAD_M()
#pragma unroll
            for (int j = 0; j < 4; ++j) dreg[j] = Dg[dstride + static_cast<size_t>(r0 + 4 * lgp + j) * dv + cc + ln];
        }
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[(r0 + ln) * LDM + k0 + lgp], sS[(k0 + lgp) * CS + cc + ln],
                                                       acc, 0, 0, 0);
        // this thread read D(s) at these addresses before the products used
        // it: S_in(s) takes its place
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Dg[static_cast<size_t>(r0 + 4 * lgp + j) * dv + cc + ln] = sS[(r0 + 4 * lgp + j) * CS + cc + ln];
        Dg += dstride;
        __syncthreads();  // every wave has read S_in(s)
#pragma unroll
        for (int j = 0; j < 4; ++j) sS[(r0 + 4 * lgp + j) * CS + cc + ln] = acc[j];
    }
    __syncthreads();
    {
        const int i = 4 * tid;
        *reinterpret_cast<float4*>(Sblk + (i / CS) * dv + i % CS) = *reinterpret_cast<const float4*>(sS + i);
    }
#undef KDA_LOAD_M
#undef KDA_STORE_M
}

// ---------------------------------------------------------------------------
// Outputs of later segments: o_t += S_in^T q^_t for every token t of the
// segment.  kOutGroups workgroups per (unit, head), each taking every
// kOutGroups-th tile of kOutTokens tokens; S_in^T is staged once per
// workgroup in LDS in the operand type.  Each wave takes 16-token tiles:
//   1. q^ and o rows are loaded 16 bytes per lane along each row (every
//      instruction reads whole row segments), one tile ahead;
//   2. the q^ rows pass through the wave's LDS staging area into MFMA
//      operand layout (lane: token, k slots);
//   3. the products give o^T in the C layout; they pass through the same
//      staging area back to row order, are added to o and stored 16 bytes
//      per lane along each row.
// Buffer ranges end at the segment's last token (loads past it return zero,
// stores are dropped), so every load and store is unconditional.
// ---------------------------------------------------------------------------

template <bool BF16, int DK>
struct OutShape {
    static constexpr int ES = BF16 ? 2 : 4;
    static constexpr int RB = DK * ES;           // bytes of one token's head slice (q^ and o)
    static constexpr int LPR = RB / 16;          // lanes per row at 16 bytes
    static constexpr int RPI = 64 / LPR;         // rows per load instruction
    static constexpr int NI = 16 / RPI;          // instructions per 16-row tile
    static constexpr int OE = 16 / ES;           // elements per 16-byte access
    static constexpr int LDQ = RB + 16;          // staging row stride (bytes), q^ rows
    static constexpr int LDA = DK * 4 + 16;      // staging row stride (bytes), fp32 products
    static constexpr int STAGE = 16 * (LDQ > LDA ? LDQ : LDA);  // bytes per wave
    static constexpr int LDB = DK + 4;           // rows of S_in^T (elements)
    static_assert(RB % 64 == 0 && NI >= 1, "row tiling");
};

template <bool BF16, int DK>
__global__ __launch_bounds__(kFixThreads) void seg_out_kernel(const int4* __restrict__ units,
                                                            const int* __restrict__ counts,
                                                            const typename Elem<BF16>::G* __restrict__ qhat,
                                                            const float* __restrict__ sin_state, int H,
                                                            typename Elem<BF16>::G* __restrict__ o) {
    using T = Elem<BF16>;
    using E = typename T::E;
    using G = typename T::G;
    using F8 = typename T::F8;
    using Sh = OutShape<BF16, DK>;
    constexpr int DV = DK;  // segmented runs have d_v = d_k
    constexpr int KB = DK / 32;
    constexpr int NCT = DV / 16;
    constexpr int LDB = Sh::LDB, NI = Sh::NI, LPR = Sh::LPR, RPI = Sh::RPI, OE = Sh::OE;
    constexpr int TILES = kOutGroups;  // workgroups per (unit, head); each takes every TILES-th tile
    constexpr int SQ = DK * DV / 4 / kFixThreads;  // float4 of S_in per thread
    static_assert(SQ >= 1, "state staging");
    __shared__ __attribute__((aligned(16))) E sBt[DV * LDB];
    __shared__ __attribute__((aligned(16))) unsigned char sStage[kFixThreads / 64][Sh::STAGE];

    const int w = blockIdx.x;
    // Heads vary fastest: consecutive workgroups go round-robin over the 8
    // XCDs, so the few working tiles of short segments use every XCD.
    const int u = w / (H * TILES);
    const int tile = (w / H) % TILES;
    const int h = w % H;
    if (u >= counts[0]) return;  // whole workgroup: before any barrier
    const int4 it = units[u];
    if (it.y == 0) return;  // a first segment starts from the true state
    if (it.z + tile * kOutTokens >= it.w) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lgp = lane >> 4;
    unsigned char* const stage = sStage[wave];

    {
        const float4* Sg = reinterpret_cast<const float4*>(sin_state + (static_cast<size_t>(u) * H + h) * DK * DV);
        float4 x[SQ];
#pragma unroll
        for (int r = 0; r < SQ; ++r) x[r] = Sg[tid + r * kFixThreads];
#pragma unroll
        for (int r = 0; r < SQ; ++r) {
            const int i = 4 * (tid + r * kFixThreads);
            const int row = i / DV, col = i % DV;
            sBt[(col + 0) * LDB + row] = T::to_e(x[r].x);
            sBt[(col + 1) * LDB + row] = T::to_e(x[r].y);
            sBt[(col + 2) * LDB + row] = T::to_e(x[r].z);
            sBt[(col + 3) * LDB + row] = T::to_e(x[r].w);
        }
    }
    __syncthreads();

    // the tiles of this workgroup: tile, tile + TILES, ... while inside the segment
    for (int tl = tile; it.z + tl * kOutTokens < it.w; tl += TILES) {
        const int t0 = it.z + tl * kOutTokens;
        const int t1 = min(it.w, t0 + kOutTokens);
        // Byte ranges: rows tt .. min(tt + 16, t1) - 1 of this head's q^ / o
        // slices (one token row is H * DK elements; at most 16 rows, so every
        // offset stays far below 2^31 under the host's H * d <= 2^20).
        const int rowB = H * Sh::RB;
        auto rsrc = [&](const G* base, int tt) __attribute__((always_inline)) {
            const int rows = __builtin_amdgcn_readfirstlane(min(16, t1 - tt));
            const int bytes = rows > 0 ? (rows - 1) * rowB + Sh::RB : 0;
            const G* p = rows > 0 ? base + static_cast<size_t>(tt) * H * DK : base;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<G*>(p), 0, bytes, 0x00020000);
        };
        const G* const qh = qhat + static_cast<size_t>(h) * DK;
        G* const oh = o + static_cast<size_t>(h) * DV;
        // this lane's row and 16-byte column block in load instruction j
        const int lrow = lane / LPR, lcol = (lane % LPR) * 16;
        auto voff = [&](int j) __attribute__((always_inline)) { return (j * RPI + lrow) * rowB + lcol; };

        u32x4_t qn[NI], on[NI];
        auto fetch = [&](int tt) __attribute__((always_inline)) {
            const auto rq = rsrc(qh, tt);
            const auto ro = rsrc(oh, tt);
#pragma unroll
            for (int j = 0; j < NI; ++j) qn[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff(j), 0, 0);
#pragma unroll
            for (int j = 0; j < NI; ++j) on[j] = __builtin_amdgcn_raw_buffer_load_b128(ro, voff(j), 0, 0);
        };

        int tt = t0 + 16 * wave;
        fetch(tt);
        for (; tt < t1; tt += 64) {
            u32x4_t qc[NI], oc[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                qc[j] = qn[j];
                oc[j] = on[j];
            }
            fetch(tt + 64);  // the next tile (an empty range past the end)
            // q^ rows -> staging -> operand fragments (lane: token ln, k slots)
#pragma unroll
            for (int j = 0; j < NI; ++j)
                *reinterpret_cast<u32x4_t*>(stage + (j * RPI + lrow) * Sh::LDQ + lcol) = qc[j];
            F8 b[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                b[kb] = lds_frag8<BF16>(reinterpret_cast<const E*>(stage) + 32 * kb, Sh::LDQ / Sh::ES, lane);
            // o^T tiles: lane holds columns 16 ct + 4 lgp .. + 3 of token ln;
            // staged as fp32 rows (the q^ rows above are consumed)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc = mma8<BF16>(acc, lds_frag8<BF16>(sBt + (16 * ct) * LDB + 32 * kb, LDB, lane), b[kb]);
                *reinterpret_cast<f32x4_t*>(stage + ln * Sh::LDA + (16 * ct + 4 * lgp) * 4) = acc;
            }
            // row order again: o += products, 16 bytes per lane along each row
            const auto ro = rsrc(oh, tt);
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const unsigned char* src = stage + (j * RPI + lrow) * Sh::LDA + (lcol / Sh::ES) * 4;
                float add[OE];
#pragma unroll
                for (int e = 0; e < OE; e += 4) {
                    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + 4 * e);
                    add[e] = v[0];
                    add[e + 1] = v[1];
                    add[e + 2] = v[2];
                    add[e + 3] = v[3];
                }
                u32x4_t out;
                if constexpr (BF16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned x = oc[j][e];
                        const float lo = __uint_as_float(x << 16) + add[2 * e];
                        const float hi = __uint_as_float(x & 0xFFFF0000u) + add[2 * e + 1];
                        out[e] = static_cast<unsigned>(f32_to_bf16(lo)) | (static_cast<unsigned>(f32_to_bf16(hi)) << 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(__uint_as_float(oc[j][e]) + add[e]);
                }
                __builtin_amdgcn_raw_buffer_store_b128(out, ro, voff(j), 0, 0);
            }
        }
    }
}

}  // namespace

// Segments pay only while the (sequence, head) pairs fill less than half of
// the compute units: with more, the identity runs' extra work and the
// fix-up traffic cost more than the shorter critical path saves.
bool prefill_segmented(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, int cus) {
    return d_k == d_v && T_tot > kSegMinTokens && 2 * static_cast<int64_t>(N) * H < cus;
}

size_t prefill_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16,
                               int cus) {
    if (!prefill_segmented(N, T_tot, H, d_k, d_v, cus)) return 0;
    return seg_layout(N, T_tot, H, d_k, d_v, bf16).bytes;
}

// Plans the segments and returns the view the prefill kernel takes.
hipError_t launch_seg_plan(const PrefillArgs& a, SegView* view) {
    const SegLayout L = seg_layout(a.N, a.T_tot, a.H, a.d_k, a.d_v, a.bf16);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int* counts = reinterpret_cast<int*>(ws);
    int4* units = reinterpret_cast<int4*>(ws + L.off_units);
    int4* longs = reinterpret_cast<int4*>(ws + L.off_longs);
    hipLaunchKernelGGL(seg_plan_kernel, dim3(1), dim3(kPlanThreads), 0, static_cast<hipStream_t>(a.stream),
                       a.cu_seqlens, a.N, units, counts, longs, L.umax, L.lmax);
    view->units = units;
    view->count = counts;
    view->qhat = ws + L.off_qhat;
    view->mstate = reinterpret_cast<float*>(ws + L.off_m);
    view->dstate = reinterpret_cast<float*>(ws + L.off_d);
    view->umax = L.umax;
    return hipGetLastError();
}

template <bool BF16, int DK>
static hipError_t launch_fixup_t(const PrefillArgs& a, const SegView& v) {
    using G = typename Elem<BF16>::G;
    const SegLayout L = seg_layout(a.N, a.T_tot, a.H, a.d_k, a.d_v, a.bf16);
    const unsigned char* ws = static_cast<const unsigned char*>(a.workspace);
    const int4* longs = reinterpret_cast<const int4*>(ws + L.off_longs);
    const hipStream_t st = static_cast<hipStream_t>(a.stream);
    const unsigned gchain = static_cast<unsigned>(L.lmax) * static_cast<unsigned>(a.H) *
                            static_cast<unsigned>(a.d_v / kFixCols);
    hipLaunchKernelGGL((seg_chain_kernel<DK>), dim3(gchain), dim3(ChainShape<DK>::NT), 0, st, v.count, longs,
                       v.mstate, v.dstate, a.H, a.d_v, a.S_T);
    const unsigned gout = static_cast<unsigned>(L.umax) * static_cast<unsigned>(a.H) *
                          static_cast<unsigned>(kOutGroups);
    hipLaunchKernelGGL((seg_out_kernel<BF16, DK>), dim3(gout), dim3(kFixThreads), 0, st, v.units, v.count,
                       static_cast<const G*>(v.qhat), v.dstate, a.H, static_cast<G*>(a.o));
    return hipGetLastError();
}

hipError_t launch_seg_fixup(const PrefillArgs& a, const SegView& v) {
    switch (a.d_k) {
        case 32: return a.bf16 ? launch_fixup_t<true, 32>(a, v) : launch_fixup_t<false, 32>(a, v);
        case 64: return a.bf16 ? launch_fixup_t<true, 64>(a, v) : launch_fixup_t<false, 64>(a, v);
        case 128: return a.bf16 ? launch_fixup_t<true, 128>(a, v) : launch_fixup_t<false, 128>(a, v);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
