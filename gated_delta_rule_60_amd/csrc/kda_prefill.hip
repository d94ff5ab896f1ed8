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
//     K~ = K * Gamma,  K^ = K / Gamma,  Q~ = Q * Gamma,  Kbar = K^ * Gamma_C
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
// walks its sequence chunk by chunk (or per segment of a long sequence, see
// kda_segment.hip: a later segment from the zero state, or its identity run
// with V = 0 and S0 = I).  Its waves have two roles:
//   * consumer waves (NC of them) carry the state.  Each owns CT 16-column
//     tiles of S for the whole sequence, in fp32 registers (MFMA C layout);
//     the columns of S evolve independently.  The consumers also share the
//     S-independent MFMA work of the chunk (the Gram products L and A_qk and
//     the diagonal-block inverses, one job per wave): the jobs of chunk i+1
//     are computed alongside the recurrence of chunk i (R, U, O and the next
//     S of the wave's columns) and published through an LDS counter.  O^T
//     quads are staged in the consumer's own rows of the slot's V^T tile.
//   * producer waves (NP of them) do the vector-ALU part of the prep into
//     LDS tiles that rotate through three slots: global loads (issued a
//     chunk ahead), the per-channel cumulative decay (a wave-local prefix
//     scan: each producer wave owns a strip of key channels for all rows),
//     the decayed operand tiles and V^T; when refilling a slot they store
//     the staged O of the chunk that used it, in row order.
// The roles meet only at monotonic counters in LDS (tiles ready, jobs done,
// slot released), so the producers' prep of chunks i+1 and i+2 runs at the
// same time as the consumers' recurrence of chunk i on every SIMD.
//
// Only consumer waves issue MFMAs (one per SIMD) and only producer waves do
// the transcendental-heavy vector work, so the two roles mostly use
// different execution units of a SIMD.
// All MFMA operands are bf16 (or fp32 for f32 inputs); accumulation and the
// carried state are fp32.
//
// Variants (template flags): SG takes one gate per token and head (Gated
// DeltaNet); WIDE takes the exponents of strongly decaying channels from the
// chunk's middle row (the wide-decay contract of kda_prefill_ex); MAP (with
// WIDE) walks the chunk lists of kda_anymap.hip instead of fixed C-token
// chunks, so that a token with a strong decay is always a chunk's first row
// (the any-decay prefill).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

// No implicit a*b+c -> fma contraction in this file: every launch shape
// (template instance) then performs the same roundings, which makes results
// bit-identical across value-slice splits.  Fused operations are written out.
#pragma clang fp contract(off)

namespace kda {

namespace {

constexpr size_t align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// Sequence-length ordering (longest first) is computed in-kernel for up to
// this many sequences; larger batches run in natural order.
constexpr int kSortMax = 64;
constexpr size_t kLdsBudget = 160 * 1024;
// Pacing of a launch that fills the GPU (see the producer loop): the chunk
// period assumed for the batch's longest sequence, in ns.  It lies below the
// period measured for that sequence with every CU busy (about 2.1 us for bf16,
// d_k = 128, 128 value columns), so paced workgroups finish before it.
constexpr int kPaceNs = 1700;
// Wide-decay variant: a channel whose decay over one chunk is below
// -kRefSwitchLog2 (log2 units, about e^-69) takes its exponents relative to
// the chunk's middle row.
constexpr float kRefSwitchLog2 = 100.f;

template <int V>
using ic = std::integral_constant<int, V>;

// A load the compiler must issue as a scalar memory load (the address is
// wave-uniform): it is counted apart from the vector loads in flight, so
// reading a chunk bound never waits for them.
typedef const __attribute__((address_space(4))) int ConstI32;
__device__ __forceinline__ int scalar_load(const int* p) { return *(ConstI32*)(p); }

// Per-chunk tiles in LDS.  The producers' tiles (decayed operands, V^T,
// Gamma_C, beta) rotate through three slots, so the producers can run two
// chunks ahead of the recurrence (the consumers read chunk i+1's tiles for
// its Gram products while they run chunk i); the consumers' job results
// (L, A_qk, -T_bb) alternate between two buffers.  Each tile's copies are
// adjacent (tile-major): copy s of tile X at O_X + s * SZ_X.
//
// Operand tiles (the producers' tiles) are unpadded and swizzled in 16-byte
// units (see quad_off): UK units per row of a [C][DK] tile, UT per row of a
// [rows][C] tile.  Job tiles are padded row-major.
template <bool BF16, int DK, int NC, int CT, int C_, bool WIDE>
struct Layout {
    using E = typename Elem<BF16>::E;
    static constexpr int C = C_;
    static constexpr int NB = C / 16;
    static constexpr int BV = 16 * CT * NC;
    static constexpr int NSLOT = 3;
    static constexpr size_t ES = sizeof(E);
    static constexpr int UK = static_cast<int>(DK * ES / 16);
    static constexpr int UT = static_cast<int>(C * ES / 16);
    static_assert(UT >= 4, "a [rows][C] operand tile row spans at least 4 units");
    static constexpr int PAD = 16 / static_cast<int>(sizeof(E));  // 16 bytes of row padding
    static constexpr int LDJ = C + PAD;
    static constexpr int LDT = 16 + PAD;
    static constexpr size_t SZ_KB = C * DK * ES;                 // K~, Q~, K^  [C][DK]
    static constexpr size_t SZ_KBT = DK * C * ES;                // Kbar^T      [DK][C]
    static constexpr size_t SZ_VT = BV * C * ES;                 // V^T         [BV][C]
    static constexpr size_t SZ_GC = align16(DK * 4);             // Gamma_C     [DK]
    static constexpr size_t SZ_BETA = align16(C * 4);            // beta        [C]
    static constexpr size_t SZ_GM = WIDE ? align16(DK * 4) : 0;  // 2^ref       [DK] (wide decay)
    static constexpr size_t SZ_L = align16(C * LDJ * ES);        // L, A_qk     [C][LDJ]
    static constexpr size_t SZ_T = align16(NB * 16 * LDT * ES);  // -T_bb       [NB][16][LDT]
    // producer tiles, tile-major: the NSLOT copies of a tile are adjacent
    // (slot s at O_X + s * SZ_X), so that with the slot known at compile
    // time a tile access is a lane offset plus an immediate
    static constexpr size_t O_KB = 0;
    static constexpr size_t O_Q = O_KB + NSLOT * SZ_KB;
    static constexpr size_t O_KBT = O_Q + NSLOT * SZ_KB;
    static constexpr size_t O_VT = O_KBT + NSLOT * SZ_KBT;
    static constexpr size_t O_KH = O_VT + NSLOT * SZ_VT;
    static constexpr size_t O_GC = O_KH + NSLOT * SZ_KB;
    static constexpr size_t O_BETA = O_GC + NSLOT * SZ_GC;
    static constexpr size_t O_GM = O_BETA + NSLOT * SZ_BETA;
    // job buffers, the same way: buffer b of X at OFF_JOB + O_X + b * SZ_X
    static constexpr size_t OFF_JOB = O_GM + NSLOT * SZ_GM;
    static constexpr size_t O_L = 0;
    static constexpr size_t O_A = O_L + 2 * SZ_L;
    static constexpr size_t O_T = O_A + 2 * SZ_L;
    static constexpr size_t OFF_SCAN = OFF_JOB + O_T + 2 * SZ_T;  // producers' scan scratch: [8][64] float4
    static constexpr size_t OFF_SEQ = OFF_SCAN + 8 * 64 * 16;
    static constexpr size_t OFF_CTR = OFF_SEQ + align16((kSortMax + 1) * 4);
    static constexpr size_t BYTES = OFF_CTR + 64;
};

// The chunk length depends only on the storage type and d_k (sized for the
// widest value slice, 128 columns, of the larger wide-decay layout), so that
// every value-slice split and both decay variants of a problem run the same
// chunk algebra and give the same bits.
template <bool BF16, int DK>
constexpr int kChunk = Layout<BF16, DK, 4, 2, 32, true>::BYTES <= kLdsBudget ? 32 : 16;

template <bool BF16, int DK, int NC, int CT, bool WIDE>
using ChosenLayout = Layout<BF16, DK, NC, CT, kChunk<BF16, DK>, WIDE>;

// Wave roles, in this order: NC consumers (all MFMA work), NP producers
// (vector ALU and memory only).
template <bool BF16, int DK, int NC, int CT, bool WIDE = false>
struct PrefillShape : ChosenLayout<BF16, DK, NC, CT, WIDE> {
    using Base = ChosenLayout<BF16, DK, NC, CT, WIDE>;
    static_assert(Base::BYTES <= kLdsBudget, "LDS budget of one gfx950 workgroup");
    static constexpr int NRG = Base::C / 4;  // row groups of 4 rows
    static constexpr int QW = 64 / NRG;      // channel quads per producer wave
    static constexpr int NQ = DK / 4;        // channel quads
    static constexpr int NPS = NQ > QW ? NQ / QW : 1;  // channel strips: producer waves per chunk
    static_assert(NQ <= QW || NQ % QW == 0, "channel strips tile d_k");
    // With one 16-column state tile per consumer wave, the consumers'
    // registers leave room for a third wave per SIMD: two producer waves per
    // strip then take alternate chunks, each with two chunk periods for its
    // loads and prep.
    static constexpr int PP = CT == 1 && NC == 4 ? 2 : 1;
    static constexpr int NP = PP * NPS;
    static_assert(NP <= 8, "scan scratch and progress counters hold eight producer waves");
    static constexpr int NJOB = Base::NB * (Base::NB + 1) / 2;  // Gram/inverse jobs per chunk
    static constexpr int NW = NC + NP;
    static constexpr int NT = 64 * NW;
    static_assert(NW <= 16, "at most 16 waves per workgroup");
    static constexpr int VITEMS = (Base::C / 4) * (Base::BV / 4);  // 4x4 blocks of V
    static constexpr int VPT = (VITEMS + 64 * NPS - 1) / (64 * NPS);
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

// ---------------------------------------------------------------------------
// Swizzled operand tiles.  A row of an operand tile is a sequence of 16-byte
// units; a "quad" is four consecutive elements along the row (logical quad
// Q holds elements 4Q .. 4Q+3).
//   bf16: the quads of each 32-element block kb are interleaved so that a
//         lane's eight MFMA operand values (quads g and g + 4 of the block,
//         the slot order of the fragments) are one 16-byte unit:
//         quad Q -> unit 4 (Q >> 3) + (Q & 3), half (Q >> 2) & 1.
//   fp32: quad Q -> unit Q.
// The unit index is then XORed with swz<U>(row), U = units per row.  The
// swizzles keep the consumers' 16-byte fragment reads (16 rows by two
// quad groups per LDS cycle) and the producers' 8-byte quad writes (eight
// rows 4 apart, or eight quads of one row) free of bank conflicts on gfx950
// (64 banks of 4 bytes for 16-byte reads and for writes).
// ---------------------------------------------------------------------------
template <int U>
__device__ __forceinline__ int swz(int r) {
    static_assert(U >= 4 && (U & (U - 1)) == 0, "units per row: a power of two >= 4");
    if constexpr (U >= 16) return 2 * ((r ^ (r >> 2)) & 7);
    else if constexpr (U == 8) return (r ^ (r >> 2)) & 7;
    else return (2 * ((r >> 2) & 1)) ^ ((r >> 3) & 1);
}

// byte offset of logical quad Q of row r in a tile with U units per row
template <bool BF16, int U>
__device__ __forceinline__ int quad_off(int r, int Q) {
    if constexpr (BF16) {
        const int unit = 4 * (Q >> 3) + (Q & 3);
        return 16 * (U * r + (unit ^ swz<U>(r))) + 8 * ((Q >> 2) & 1);
    } else {
        return 16 * (U * r + (Q ^ swz<U>(r)));
    }
}

template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::E* tile_at(void* tile, int off) {
    return reinterpret_cast<typename Elem<BF16>::E*>(static_cast<unsigned char*>(tile) + off);
}

// MFMA fragment of a 32-deep block kb of row r, lane group g (frag8 slot order)
template <bool BF16, int U>
__device__ __forceinline__ typename Elem<BF16>::F8 tile_frag8(const void* tile, int r, int kb, int g) {
    const unsigned char* t = static_cast<const unsigned char*>(tile);
    if constexpr (BF16) {
        return *reinterpret_cast<const bf16x8_t*>(t + 16 * (U * r + ((4 * kb + g) ^ swz<U>(r))));
    } else {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(t + 16 * (U * r + ((8 * kb + g) ^ swz<U>(r))));
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(t + 16 * (U * r + ((8 * kb + g + 4) ^ swz<U>(r))));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// one quad (a 16-deep fragment, or four C-layout values) of row r
template <bool BF16, int U>
__device__ __forceinline__ typename Elem<BF16>::F4 tile_quad(const void* tile, int r, int Q) {
    return *reinterpret_cast<const typename Elem<BF16>::F4*>(static_cast<const unsigned char*>(tile) +
                                                              quad_off<BF16, U>(r, Q));
}

// Byte offset of quad Q (four consecutive tokens) of row r of a V^T tile.
// bf16 (32-token rows of eight 8-byte quads): rows are paired into 128-byte
// blocks m = r / 2, whose 16 quads are permuted by
//     slot = (8 (r & 1) + Q) ^ h(m),   h(m) = ((m >> 1) & 15) ^ ((m & 1) << 2),
// so that each of the tile's 8-byte accesses is free of LDS bank conflicts:
// the producers' V transpose and O read-back (rows 4 l + c of lane l) and the
// consumers' V reads and O staging (rows r0 + 0..15).  fp32 tiles (16-byte
// quads) keep the row layout of quad_off.
template <bool BF16, int U>
__device__ __forceinline__ int vt_off(int r, int Q) {
    if constexpr (BF16) {
        static_assert(U == 4, "V^T rows of 32 bf16 tokens");
        const int m = r >> 1;
        const int h = ((m >> 1) & 15) ^ ((m & 1) << 2);
        return 128 * m + 8 * ((((r & 1) << 3) | Q) ^ h);
    } else {
        return quad_off<BF16, U>(r, Q);
    }
}

// Byte offset of quad Q (four consecutive tokens) of row r of the Kbar^T
// tile.  bf16 (32-token rows, one 32-deep block): rows are paired into
// 128-byte blocks m = r / 2 of eight 16-byte units, and a unit keeps the two
// quads g and g + 4 that one MFMA operand fragment reads:
//     unit = (4 (r & 1) + (Q & 3)) ^ h(m),   h(m) = x ^ ((x & 1) << 1), x = (m >> 1) & 7,
// half (Q >> 2) & 1.  The producers' quad writes (rows i0 + c of eight lanes
// 4 rows apart) and the consumers' fragment reads (rows r0 + 0..15) are then
// free of LDS bank conflicts.  fp32 tiles keep the row layout of quad_off.
template <bool BF16, int U>
__device__ __forceinline__ int kbt_off(int r, int Q) {
    if constexpr (BF16) {
        static_assert(U == 4, "Kbar^T rows of 32 bf16 tokens");
        const int m = r >> 1, x = (m >> 1) & 7;
        const int h = x ^ ((x & 1) << 1);
        return 128 * m + 16 * ((((r & 1) << 2) | (Q & 3)) ^ h) + 8 * ((Q >> 2) & 1);
    } else {
        return quad_off<BF16, U>(r, Q);
    }
}

// MFMA fragment of lane group g of row r of the Kbar^T tile (one 32-deep block)
template <bool BF16, int U>
__device__ __forceinline__ typename Elem<BF16>::F8 kbt_frag8(const void* tile, int r, int g) {
    if constexpr (BF16) {
        return *reinterpret_cast<const bf16x8_t*>(static_cast<const unsigned char*>(tile) + kbt_off<BF16, U>(r, g));
    } else {
        return tile_frag8<BF16, U>(tile, r, 0, g);
    }
}

// Transposes a 4x4 block given as four raw row quads into four column quads.
template <bool BF16>
__device__ __forceinline__ void transpose4(const typename Elem<BF16>::R4 (&rows)[4],
                                           typename Elem<BF16>::R4 (&cols)[4]) {
    if constexpr (BF16) {
        // rows[r] = {x: c0 | c1 << 16, y: c2 | c3 << 16}.  v_perm_b32 picks
        // bytes of {S0 (bytes 4..7), S1 (bytes 0..3)}: the low or high 16
        // bits of two rows form one 32-bit word of a column.
        constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
        cols[0].x = __builtin_amdgcn_perm(rows[1].x, rows[0].x, kLo);
        cols[0].y = __builtin_amdgcn_perm(rows[3].x, rows[2].x, kLo);
        cols[1].x = __builtin_amdgcn_perm(rows[1].x, rows[0].x, kHi);
        cols[1].y = __builtin_amdgcn_perm(rows[3].x, rows[2].x, kHi);
        cols[2].x = __builtin_amdgcn_perm(rows[1].y, rows[0].y, kLo);
        cols[2].y = __builtin_amdgcn_perm(rows[3].y, rows[2].y, kLo);
        cols[3].x = __builtin_amdgcn_perm(rows[1].y, rows[0].y, kHi);
        cols[3].y = __builtin_amdgcn_perm(rows[3].y, rows[2].y, kHi);
    } else {
        cols[0] = make_float4(rows[0].x, rows[1].x, rows[2].x, rows[3].x);
        cols[1] = make_float4(rows[0].y, rows[1].y, rows[2].y, rows[3].y);
        cols[2] = make_float4(rows[0].z, rows[1].z, rows[2].z, rows[3].z);
        cols[3] = make_float4(rows[0].w, rows[1].w, rows[2].w, rows[3].w);
    }
}

// four consecutive storage elements from LDS, raw
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::R4 lds_get_raw4(const typename Elem<BF16>::E* p) {
    if constexpr (BF16) {
        return *reinterpret_cast<const uint2*>(p);
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

// four fp32 values as four consecutive storage elements (bf16: round to
// nearest even)
template <bool BF16>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, int voff, const f32x4_t& x) {
    if constexpr (BF16) {
        bf16x4_t h;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = static_cast<__bf16>(x[j]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, h), r, voff, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, voff, 0, 0);
    }
}

// four consecutive storage elements, raw (stores past the range are
// dropped); a 16-byte store takes its whole offset in voffset (store_voffset)
template <bool BF16>
__device__ __forceinline__ void buf_store_raw4(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                               const typename Elem<BF16>::R4& x) {
    if constexpr (BF16) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{x.x, x.y}, r, voff, soff, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)}, r,
            store_voffset(voff, soff), 0, 0);
    }
}

// four consecutive storage elements, raw
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::R4 buf_load_raw4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (BF16) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return make_uint2(x[0], x[1]);
    } else {
        return buf_load_f4(r, voff, soff);
    }
}

// Inter-wave hand-off through monotonic counters in LDS.  A counter is
// either a sum (every wave of a group adds one per chunk: only sound among
// waves that cannot run a whole chunk ahead of one another) or one wave's
// own progress (it stores the number of chunks it has completed).  signal: once this
// wave's earlier LDS reads and writes have completed, add one.  wait: spin
// until the counter reaches target.  LDS accesses of one wave are performed
// in order, so data written before a signal is visible after the wait.
__device__ __forceinline__ void ctr_signal(int* ctr, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

//
// Every wait is bounded: a wait that has not been satisfied after kSpinMax
// sleeps (far beyond any legitimate hand-off) marks the workgroup as failed
// in *fault and returns, so the kernel always drains.  Once the flag is set,
// every later wait of the workgroup gives up within kFaultPoll sleeps
// instead of its own full bound; the consumers then write NaN final states
// and the producers store NaN outputs from then on, so a failed workgroup
// cannot return a plausible result.
constexpr int kSpinMax = 1 << 24;
constexpr int kFaultPoll = 64;  // sleeps between two reads of the fault flag

__device__ __forceinline__ void ctr_publish(int* ctr, int value, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(ctr, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void ctr_wait(int* ctr, int target, int* fault) {
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        ++spins;
        if (spins > kSpinMax ||
            (spins % kFaultPoll == 0 && __hip_atomic_load(fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0)) {
            __hip_atomic_store(fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Waits until each of n progress counters has reached target.  Four
// counters (16-byte aligned) are read with one LDS access: each 32-bit
// counter is read whole, and they only grow, so a snapshot whose minimum
// has reached the target means every one of them has.
__device__ __forceinline__ void ctr_wait_each(int* ctrs, int n, int target, int* fault) {
    if (n == 4) {
        typedef int i32x4_t __attribute__((ext_vector_type(4)));
        typedef const volatile __attribute__((address_space(3))) i32x4_t Lds4;
        Lds4* const p4 = (Lds4*)(ctrs);
        int spins = 0;
        for (;;) {
            const i32x4_t c = *p4;
            // (the same value in every lane: a scalar branch)
            if (__builtin_amdgcn_readfirstlane(min(min(c[0], c[1]), min(c[2], c[3]))) >= target) break;
            ++spins;
            if (spins > kSpinMax ||
                (spins % kFaultPoll == 0 && __hip_atomic_load(fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0)) {
                __hip_atomic_store(fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
        return;
    }
    for (int w = 0; w < n; ++w) ctr_wait(ctrs + w, target, fault);
}

}  // namespace

// SG: scalar gate (one log alpha per token and head, [T, H]: Gated DeltaNet);
// otherwise one per key channel ([T, H, d_k]: KDA).  A scalar gate is the
// per-channel computation with the value repeated over the channels.
// WIDE: wide-decay variant (exponents of strongly decaying channels taken
// relative to the chunk's middle row, the state operand scaled to match).
template <bool BF16, int DK, int NC, int CT, bool SG, bool WIDE, bool CK = false, bool MAP = false>
__global__ __launch_bounds__((PrefillShape<BF16, DK, NC, CT, WIDE>::NT)) void prefill_kernel(
    const typename Elem<BF16>::G* __restrict__ q, const typename Elem<BF16>::G* __restrict__ k,
    const typename Elem<BF16>::G* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, const float* __restrict__ S0, const int32_t* __restrict__ cu,
    int N, int H, int dv, int v_split, typename Elem<BF16>::G* __restrict__ o,
    float* __restrict__ S_T, SegView seg, CkptView ck, ChunkMap cm, int pace16) {
    static_assert(!MAP || (WIDE && !CK), "chunk lists need the wide-decay variant and outputs");
    using Sh = PrefillShape<BF16, DK, NC, CT, WIDE>;
    using T = Elem<BF16>;
    using E = typename T::E;
    using G = typename T::G;
    using R4 = typename T::R4;
    using F8 = typename T::F8;
    using F4 = typename T::F4;
    constexpr int C = Sh::C, NB = Sh::NB, NT = Sh::NT, BV = Sh::BV;
    constexpr int NP = Sh::NP, NPS = Sh::NPS, PP = Sh::PP;
    constexpr int LDJ = Sh::LDJ, LDT = Sh::LDT, UK = Sh::UK, UT = Sh::UT;
    constexpr int KB = DK / 32;  // 32-deep k blocks over key channels
    constexpr int NRG = Sh::NRG, QW = Sh::QW, NQ = Sh::NQ, VPT = Sh::VPT, VITEMS = Sh::VITEMS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::BYTES];
#define KDA_TILE(name, type, base, stride, off) \
    auto name = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<type*>(smem + (base) + b * (stride) + (off)); }
    // producer slots 0..2
    KDA_TILE(tKb, E, Sh::O_KB, Sh::SZ_KB, 0);
    KDA_TILE(tQ, E, Sh::O_Q, Sh::SZ_KB, 0);
    KDA_TILE(tKh, E, Sh::O_KH, Sh::SZ_KB, 0);
    KDA_TILE(tKbT, E, Sh::O_KBT, Sh::SZ_KBT, 0);
    KDA_TILE(tVt, E, Sh::O_VT, Sh::SZ_VT, 0);
    KDA_TILE(sGC, float, Sh::O_GC, Sh::SZ_GC, 0);
    KDA_TILE(sGM, float, Sh::O_GM, Sh::SZ_GM, 0);
    KDA_TILE(sBeta, float, Sh::O_BETA, Sh::SZ_BETA, 0);
    // job buffers 0..1
    KDA_TILE(tL, E, Sh::OFF_JOB + Sh::O_L, Sh::SZ_L, 0);
    KDA_TILE(tA, E, Sh::OFF_JOB + Sh::O_A, Sh::SZ_L, 0);
    KDA_TILE(tT, E, Sh::OFF_JOB + Sh::O_T, Sh::SZ_T, 0);
#undef KDA_TILE
    int* const sSeq = reinterpret_cast<int*>(smem + Sh::OFF_SEQ);
    // Monotonic counters, one signal per wave per chunk:
    int* const ctr = reinterpret_cast<int*>(smem + Sh::OFF_CTR);
    // Sum counters are only used among consumer waves, which bound one
    // another at every chunk; producers never wait for one another, so each
    // producer wave reports its own progress.
    int* const nSolved = ctr + 0;   // consumers: their L, A_qk, -T_bb jobs written
    int* const nFree = ctr + 1;     // consumers: producer slot of the chunk released
    int* const fault = ctr + 2;     // a bounded wait gave up
    int* const prodDone = ctr + 4;  // [NP] chunks completed by each producer wave (ctr + 4 .. ctr + 11)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lg = lane >> 4;

    // ---- work assignment -------------------------------------------------
    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs.
    // Units are laid out so the value slices of one unit run back to back on
    // the same XCD (shared q/k/log alpha lines in its L2), and lower unit ids
    // (dispatched first) are the longer sequences or segments.
    //
    // Whole sequences: a unit is (sequence, head), with v_split value slices.
    // Segments (seg.units set): a unit is (segment, head), with v_split value
    // slices and, for a segment after the first, v_split slices of the
    // identity run (V = 0, S0 = I over the d_k = d_v columns).  A later
    // segment starts from the zero state; the segment fix-up adds what the
    // true entering state contributes (linearity in (S0, V)).
    auto xcd_map = [&](int units, int per_unit, int& unit_id, int& sub) __attribute__((always_inline)) {
        const int b = blockIdx.x;
        if ((units & 7) == 0) {
            const int x = b & 7, qq = b >> 3;
            unit_id = 8 * (qq / per_unit) + x;
            sub = qq % per_unit;
        } else {
            unit_id = b / per_unit;
            sub = b % per_unit;
        }
    };
    int n, h, slice, t_beg, t_end;
    int mode = 0;  // 0: S0 (or zero) start; 1: later segment, zero start; 2: identity run
    const float* s0p;
    float* sdst;  // this head's [DK][dv] block of the final state
    G* obase;     // [T][H][dv] outputs (o, or the identity runs' q^ for mode 2)
    if (seg.units == nullptr) {
        int unit;
        xcd_map(N * H, v_split, unit, slice);
        h = unit % H;
        const int rank = unit / H;
        n = rank;
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
            if constexpr (MAP) n = __builtin_amdgcn_readfirstlane(n);  // addresses of scalar loads
        }
        t_beg = cu[n];
        t_end = cu[n + 1];
        const size_t pair = static_cast<size_t>(n) * H + h;
        s0p = S0 ? S0 + pair * DK * dv : nullptr;
        sdst = S_T + pair * DK * dv;
        obase = o;
    } else {
        int uh, sub;
        xcd_map(seg.umax * H, 2 * v_split, uh, sub);
        const int u = uh / H;
        h = uh % H;
        if (u >= *seg.count) return;  // whole workgroup: before any barrier
        const int4 it = seg.units[u];
        n = it.x;
        t_beg = it.z;
        t_end = it.w;
        if (sub >= v_split) {
            if (it.y == 0) return;  // the first segment needs no identity run
            mode = 2;
            slice = sub - v_split;
        } else {
            mode = it.y == 0 ? 0 : 1;
            slice = sub;
        }
        const size_t pair = static_cast<size_t>(n) * H + h;
        const size_t blk = static_cast<size_t>(u) * H + h;
        s0p = mode == 0 && S0 ? S0 + pair * DK * dv : nullptr;
        sdst = mode == 0 ? S_T + pair * DK * dv : (mode == 1 ? seg.dstate : seg.mstate) + blk * DK * dv;
        obase = mode == 2 ? static_cast<G*>(seg.qhat) : o;
    }
    int nchunks = (t_end - t_beg + C - 1) / C;
    const int* cs = nullptr;  // MAP: this (sequence, head)'s chunk starts, then the sequence end
    if constexpr (MAP) {
        // (every value read from the lists is clamped to the sequence, so
        // that accesses stay in bounds whatever the lists hold)
        cs = cm.starts + h * cm.stride + __builtin_amdgcn_readfirstlane(t_beg + 2 * n);
        nchunks = min(max(scalar_load(cm.count + n * H + h), 0), t_end - t_beg);
    }
    const int j0 = slice * BV;  // first value column of this workgroup
    // first token and length of chunk i (length 0 past the last chunk)
    auto list_at = [&](int i) __attribute__((always_inline)) { return min(max(scalar_load(cs + i), t_beg), t_end); };
    auto chunk_beg = [&](int i) __attribute__((always_inline)) {
        if constexpr (MAP) return i < nchunks ? list_at(i) : t_end;
        else return t_beg + i * C;
    };
    auto chunk_len = [&](int i) __attribute__((always_inline)) {
        if constexpr (MAP) return i < nchunks ? min(max(list_at(i + 1) - list_at(i), 0), C) : 0;
        else return min(C, t_end - (t_beg + i * C));
    };

    // Per-token offsets below fit in 32 bits (the host rejects tensors of
    // 2^31 elements or more).
    const int strideK = H * DK;
    const int strideV = H * dv;

    // Upper block-triangles of L and A_qk stay zero for the whole kernel.
    for (int idx = tid; idx < C * LDJ; idx += NT) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            tL(b)[idx] = T::to_e(0.f);
            tA(b)[idx] = T::to_e(0.f);
        }
    }
    if (tid < 16) ctr[tid] = 0;
    __syncthreads();

    // Issue priority follows the critical path: the consumers' recurrence is
    // the serial chain of the sequence; the producers work ahead with slack.
    if (wave < NC) {
        // =====================================================================
        // consumer: the recurrence of value columns j0 + 16 (CT wave + ct) + ...
        // =====================================================================
        __builtin_amdgcn_s_setprio(3);
        auto col0 = [&](int ct) __attribute__((always_inline)) { return 16 * (CT * wave + ct); };
        // Sr[ct][it][j] = S[16 it + 4 lg + j][col]
        f32x4_t Sr[CT][DK / 16];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const size_t col = static_cast<size_t>(j0 + col0(ct) + ln);
#pragma unroll
            for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                {
                    const size_t row = 16 * it + 4 * lg + j;
                    Sr[ct][it][j] = s0p ? s0p[row * dv + col] : (mode == 2 && row == col ? 1.f : 0.f);
                }
            }
        }

        // Job (st, rt), st <= rt, computes the tiles at block (rt, st) of
        // L = strictly_lower(beta K~ K^T) and A_qk = lower_incl(Q~ K^T),
        // sharing the K^ operand (the LDS tile holds K~; beta is applied to
        // the rows of the product).  They are computed transposed,
        // P[s][r] = K^_s . X_r, so that each lane's four C-layout values are
        // four consecutive columns of row r.
        //
        // A diagonal job also forms -T_bb = -(I + N)^-1, N = L_bb (strictly
        // lower, nilpotent: N^16 = 0), as (I + N^8)(I + N^4)(I - N)(I + N^2)
        // with MFMA, four products deep.  The factors are polynomials in N
        // and commute, so every product can take its A operand from a
        // C-layout tile already held: the A operand of X is the C layout of
        // X^T, the B operand of X is the C layout of X.  Both layouts of N
        // come from the Gram MFMAs (P and P^T).
        //
        // Results of one job, kept in registers until they are stored.
        struct Job {
            f32x4_t l, a, t;  // L and A_qk values of the block; -T_bb (diagonal jobs)
        };
        static_assert(NB <= 2, "job table covers chunks of up to two 16-row blocks");
        constexpr int NJOB = Sh::NJOB;
        constexpr int JPW = (NJOB + NC - 1) / NC;  // jobs per consumer wave
        // job -> block: 0 -> (0,0), 1 -> (1,1), 2 -> (st 0, rt 1); jobs past the
        // last one compute the last job again and are never stored.
        auto job_of = [&](int t) __attribute__((always_inline)) { return wave + NC * t; };
        auto job_st = [&](int jc) __attribute__((always_inline)) { return jc == 2 ? 0 : jc; };
        auto job_rt = [&](int jc) __attribute__((always_inline)) { return jc == 2 ? 1 : jc; };
        // Straight-line (no branches), so that it interleaves with the recurrence.
        auto prep3_compute = [&](int S, int t) __attribute__((always_inline)) {  // S: producer slot
            const int jc = min(job_of(t), NJOB - 1);
            const int st = job_st(jc), rt = job_rt(jc);
            f32x4_t accL = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f}, accN = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const F8 a = tile_frag8<BF16, UK>(tKh(S), 16 * st + ln, kb, lg);
                const F8 bk = tile_frag8<BF16, UK>(tKb(S), 16 * rt + ln, kb, lg);
                accL = mma8<BF16>(accL, a, bk);
                if constexpr (!CK)  // the checkpointing pass forms no outputs
                    accA = mma8<BF16>(accA, a, tile_frag8<BF16, UK>(tQ(S), 16 * rt + ln, kb, lg));
                accN = mma8<BF16>(accN, bk, a);  // P^T: C layout of N (used by diagonal jobs)
            }
            Job res;
            const int r = 16 * rt + ln;
            // L = strictly_lower(beta K~ K^T): beta of row r, per lane in P,
            // per value (rows 16 rt + 4 lg + j) in P^T
            const float br = sBeta(S)[r];
            const float4 bn = *reinterpret_cast<const float4*>(sBeta(S) + 16 * rt + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s2 = 16 * st + 4 * lg + j;
                res.l[j] = (s2 < r) ? br * accL[j] : 0.f;
                res.a[j] = (s2 <= r) ? accA[j] : 0.f;
            }
            // C layout: lane (ln, lg), value j is element (row 4 lg + j, col ln).
            f32x4_t Nt, Nc;  // C layouts of N^T and N (strictly lower N)
            const float bnj[4] = {bn.x, bn.y, bn.z, bn.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Nt[j] = res.l[j];
                Nc[j] = (ln < 4 * lg + j) ? bnj[j] * accN[j] : 0.f;
            }
            auto eye = [&](f32x4_t x, float sgn) __attribute__((always_inline)) {
                f32x4_t y;
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = sgn * x[j] + ((4 * lg + j == ln) ? 1.f : 0.f);
                return y;
            };
            auto f4 = [&](const f32x4_t& x) __attribute__((always_inline)) { return acc_frag4<BF16>(x); };
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            // depth 1
            const f32x4_t N2 = mma4<BF16>(z, f4(Nt), f4(Nc));
            const f32x4_t N2t = mma4<BF16>(z, f4(Nc), f4(Nt));
            // depth 2: P1 = (I - N)(I + N^2)
            const f32x4_t P1 = mma4<BF16>(z, f4(eye(Nt, -1.f)), f4(eye(N2, 1.f)));
            const f32x4_t N4 = mma4<BF16>(z, f4(N2t), f4(N2));
            const f32x4_t N4t = mma4<BF16>(z, f4(N2), f4(N2t));
            // depth 3: P2 = (I + N^4) P1, and (N^8)^T
            const f32x4_t P2 = mma4<BF16>(z, f4(eye(N4t, 1.f)), f4(P1));
            const f32x4_t N8t = mma4<BF16>(z, f4(N4), f4(N4t));
            // depth 4: T^T = P2^T (I + N^8)^T
            const f32x4_t Tt = mma4<BF16>(z, f4(P2), f4(eye(N8t, 1.f)));
#pragma unroll
            for (int j = 0; j < 4; ++j) res.t[j] = -Tt[j];
            return res;
        };
        auto prep3_store = [&](int S, int t, const Job& res) __attribute__((always_inline)) {  // S: job buffer
            const int job = job_of(t);
            if (job < NJOB) {
                const int st = job_st(job), rt = job_rt(job);
                const int r = 16 * rt + ln;
                lds_store4<BF16>(tL(S) + r * LDJ + 16 * st + 4 * lg, res.l[0], res.l[1], res.l[2], res.l[3]);
                lds_store4<BF16>(tA(S) + r * LDJ + 16 * st + 4 * lg, res.a[0], res.a[1], res.a[2], res.a[3]);
                // lane (ln, lg) holds T[ln][4 lg + j]: -T row-major
                if (st == rt) lds_store4<BF16>(tT(S) + r * LDT + 4 * lg, res.t[0], res.t[1], res.t[2], res.t[3]);
            }
        };

        F8 sf[CT][KB];
        f32x4_t Rp[CT][NB], U[CT][NB];
        f32x4_t accQS[CT][NB];  // Q~ S of the chunk's rows, formed beside R'
        F4 uf[CT][NB];

        // Checkpoints for the chunked backward pass (CK): per chunk, the
        // entering state S in the layout of its A operand with the value
        // columns as the reduction index (each 16 x 16 tile transposed by an
        // MFMA with the identity, which is exact), and W0 = V - K~ S in the C
        // layout.  Slot of chunk i: t_beg / C + n + i (distinct over the
        // sequences of a batch).
        using Ev = typename Elem<BF16>::E;
        auto ck_slot = [&](int i) __attribute__((always_inline)) {
            return static_cast<size_t>(t_beg / C + n + i) * H + h;
        };
        auto ck_store_state = [&](int i) __attribute__((always_inline)) {
            Ev* const base = static_cast<Ev*>(ck.s) + ck_slot(i) * DK * dv;
            F4 eye;
#pragma unroll
            for (int j = 0; j < 4; ++j) eye[j] = T::to_e(4 * lg + j == ln ? 1.f : 0.f);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int ctile = (j0 + col0(ct)) >> 4;
#pragma unroll
                for (int it = 0; it < DK / 16; ++it) {
                    // lane (ln, lg): S[16 it + ln][16 ctile + 4 lg .. + 3]
                    const f32x4_t tr = mma4<BF16>(z, acc_frag4<BF16>(Sr[ct][it]), eye);
                    const size_t e = (static_cast<size_t>(it * (dv >> 5) + (ctile >> 1)) * 64 + lane) * 8 + 4 * (ctile & 1);
                    lds_store4<BF16>(base + e, tr[0], tr[1], tr[2], tr[3]);
                }
            }
        };
        auto ck_store_w0 = [&](int i, int ct, int rt, const f32x4_t& rpv) __attribute__((always_inline)) {
            Ev* const base = static_cast<Ev*>(ck.w0) + ck_slot(i) * C * dv;
            const int ctile = (j0 + col0(ct)) >> 4;
            const size_t e = (static_cast<size_t>(ctile * NB + rt) * 64 + lane) * 4;
            lds_store4<BF16>(base + e, -rpv[0], -rpv[1], -rpv[2], -rpv[3]);
        };

        // R' = beta (K~ S - V)  (= -R), and beside it Q~ S for the outputs: the
        // same S fragments, independent accumulators (off the U and S chain)
        auto chain_R = [&](int B, int ci) __attribute__((always_inline)) {
            if constexpr (WIDE) {
                // the S operand of K~ S and Q~ S with its rows (key channels)
                // scaled by 2^ref of the chunk (exactly 1 for a channel with
                // the start reference)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(sGM(B) + 32 * kb + 4 * lg);
                    const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(sGM(B) + 32 * kb + 16 + 4 * lg);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        sf[ct][kb] = acc_frag8<BF16>(Sr[ct][2 * kb] * e0, Sr[ct][2 * kb + 1] * e1);
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        sf[ct][kb] = acc_frag8<BF16>(Sr[ct][2 * kb], Sr[ct][2 * kb + 1]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const f32x4_t v4 = lds_load4<BF16>(tile_at<BF16>(tVt(B), vt_off<BF16, UT>(col0(ct) + ln, 4 * rt + lg)));
                    Rp[ct][rt] = f32x4_t{-v4[0], -v4[1], -v4[2], -v4[3]};
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const F8 a = tile_frag8<BF16, UK>(tKb(B), 16 * rt + ln, kb, lg);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Rp[ct][rt] = mma8<BF16>(Rp[ct][rt], a, sf[ct][kb]);
                }
                if constexpr (!CK) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) accQS[ct][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const F8 aq = tile_frag8<BF16, UK>(tQ(B), 16 * rt + ln, kb, lg);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) accQS[ct][rt] = mma8<BF16>(accQS[ct][rt], aq, sf[ct][kb]);
                    }
                }
                if constexpr (CK) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) ck_store_w0(ci, ct, rt, Rp[ct][rt]);
                }
                // rows of R' scaled by beta (lane holds rows 16 rt + 4 lg + j)
                const float4 b4 = *reinterpret_cast<const float4*>(sBeta(B) + 16 * rt + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    Rp[ct][rt] = f32x4_t{b4.x * Rp[ct][rt][0], b4.y * Rp[ct][rt][1], b4.z * Rp[ct][rt][2],
                                         b4.w * Rp[ct][rt][3]};
            }
        };
        auto u_frag8 = [&](int ct, int b) __attribute__((always_inline)) {
            return F8(__builtin_shufflevector(uf[ct][b], uf[ct][b + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // U_b = (-T_bb) (R'_b + sum_{c<b} L_bc U_c);  then O^T = (Q~ S)^T + U^T A_qk^T,
        // written to global memory from the C layout: lane (ln, lg) holds
        // four consecutive value columns of token row 16 rt + ln.
        auto chain_UO = [&](int B, int J) __attribute__((always_inline)) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4_t Y[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Y[ct] = Rp[ct][b];
#pragma unroll
                for (int kp = 0; kp + 1 < b; kp += 2) {
                    const F8 a = lds_frag8<BF16>(tL(J) + 16 * b * LDJ + 16 * kp, LDJ, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[ct] = mma8<BF16>(Y[ct], a, u_frag8(ct, kp));
                }
                if (b & 1) {
                    const F4 a = lds_frag4<BF16>(tL(J) + 16 * b * LDJ + 16 * (b - 1), LDJ, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[ct] = mma4<BF16>(Y[ct], a, uf[ct][b - 1]);
                }
                const F4 tb = lds_frag4<BF16>(tT(J) + 16 * b * LDT, LDT, lane);
                const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) U[ct][b] = mma4<BF16>(z, tb, acc_frag4<BF16>(Y[ct]));
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) uf[ct][b] = acc_frag4<BF16>(U[ct][b]);
            }
            // O = Q~ S + A_qk U for this wave's columns.  In the C layout lane
            // (ln, lg) holds tokens 16 rt + 4 lg .. + 3 of value column
            // 16 ct + ln: one O^T quad, staged in the wave's own rows of this
            // slot's V^T tile (read above, in chain_R).  The producers store
            // it to global memory, in row order, when they refill the slot.
            // (The checkpointing variant has no outputs.)
            if constexpr (CK) return;
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
                f32x4_t acc[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) acc[ct] = accQS[ct][rt];
#pragma unroll
                for (int sp = 0; sp + 1 <= rt; sp += 2) {
                    const F8 aa = lds_frag8<BF16>(tA(J) + 16 * rt * LDJ + 16 * sp, LDJ, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[ct] = mma8<BF16>(acc[ct], aa, u_frag8(ct, sp));
                }
                if (!(rt & 1)) {
                    const F4 aa = lds_frag4<BF16>(tA(J) + 16 * rt * LDJ + 16 * rt, LDJ, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[ct] = mma4<BF16>(acc[ct], aa, uf[ct][rt]);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    lds_store4<BF16>(tile_at<BF16>(tVt(B), vt_off<BF16, UT>(col0(ct) + ln, 4 * rt + lg)),
                                     acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
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
                    const F8 a = kbt_frag8<BF16, UT>(tKbT(B), 16 * it + ln, lg);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[ct] = mma8<BF16>(acc[ct], a, u_frag8(ct, 2 * kb));
                }
                if constexpr (NB & 1) {
                    const F4 a = tile_quad<BF16, UT>(tKbT(B), 16 * it + ln, 4 * (NB - 1) + lg);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[ct] = mma4<BF16>(acc[ct], a, uf[ct][NB - 1]);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Sr[ct][it] = acc[ct];
            }
        };

        // Software pipeline: the jobs of chunk i+1 are computed in registers
        // alongside the recurrence of chunk i (from the next producer slot)
        // and stored after it.  On the last chunk they run on stale tiles and
        // are not stored.  Chunk i: producer slot P = i mod 3, job buffer i & 1.
        // tiles of chunk m: written by the NPS producer waves of its parity
        auto wait_tiles = [&](int m) __attribute__((always_inline)) {
            ctr_wait_each(prodDone + (PP == 2 ? (m & 1) * NPS : 0), NPS, m + 1, fault);
        };
        // With at least as many consumer waves as jobs, the waves without a
        // job run a copy of the loop that has none (a wave-uniform branch);
        // otherwise every wave runs its jobs, the extra ones on a repeated
        // job index whose results are never stored.
        auto run = [&](auto WithJobs) __attribute__((always_inline)) {
            constexpr bool kJobs = decltype(WithJobs)::value;
            Job jobs[JPW];
            if (nchunks > 0) {
                wait_tiles(0);
                if constexpr (kJobs) {
#pragma unroll
                    for (int t = 0; t < JPW; ++t) {
                        jobs[t] = prep3_compute(0, t);
                        prep3_store(0, t, jobs[t]);
                    }
                }
                ctr_signal(nSolved, lane);
                if constexpr (CK) ck_store_state(0);
            }
            // Chunk i: producer slot P = i mod 3 and job buffer J = i & 1.
            auto chunk = [&](auto PC, int i) __attribute__((always_inline)) {
                const int P = PC;  // a compile-time constant in the unrolled loop below
                const int Pn = P == 2 ? 0 : P + 1;
                const int J = i & 1;
                const bool has_next = i + 1 < nchunks;
                // R' and Q~ S need only this chunk's tiles (awaited before):
                // formed ahead of the waits, they give the producers that
                // time to finish the next chunk's tiles, and the other
                // consumers to store this chunk's jobs.
                chain_R(P, i);
                ctr_wait(nSolved, NC * (i + 1), fault);  // jobs of chunk i stored
                if (has_next) wait_tiles(i + 1);
                if constexpr (kJobs) {
#pragma unroll
                    for (int t = 0; t < JPW; ++t) jobs[t] = prep3_compute(Pn, t);
                }
                chain_UO(P, J);
                chain_S(P);
                ctr_signal(nFree, lane);
                if (has_next) {
                    if constexpr (kJobs) {
#pragma unroll
                        for (int t = 0; t < JPW; ++t) prep3_store(1 - J, t, jobs[t]);
                    }
                    ctr_signal(nSolved, lane);
                    // the state entering the next chunk, stored while the
                    // next chunk's hand-offs are awaited
                    if constexpr (CK) ck_store_state(i + 1);
                }
            };
            // Unrolled over three chunks the slot is a constant in each copy,
            // and with the tile-major layout a tile read is a lane offset plus
            // an immediate.  The shapes whose registers are tighter (one state
            // tile per wave, or the checkpointing pass) keep the rolled loop:
            // unrolled, they spill; so does the wide-decay variant, which
            // measured slower unrolled over chunk lists (0.597 against 0.559
            // ms on the any-decay batch).
            if constexpr (CT >= 2 && !CK && !WIDE) {
                for (int i = 0; i < nchunks; i += 3) {
                    chunk(ic<0>{}, i);
                    if (i + 1 >= nchunks) break;
                    chunk(ic<1>{}, i + 1);
                    if (i + 2 >= nchunks) break;
                    chunk(ic<2>{}, i + 2);
                }
            } else {
                int P = 0;
                for (int i = 0; i < nchunks; ++i) {
                    chunk(P, i);
                    P = P == 2 ? 0 : P + 1;
                }
            }
        };
        if (NC < NJOB || wave < NJOB)
            run(std::true_type{});
        else
            run(std::false_type{});

        // Every wave's last signal follows all of its waits, so a fault
        // recorded by any wave is visible after the last rendezvous.
        if (__hip_atomic_load(fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int it = 0; it < DK / 16; ++it) Sr[ct][it] = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            }
        }
        if constexpr (!CK) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const size_t col = static_cast<size_t>(j0 + col0(ct) + ln);
#pragma unroll
                for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sdst[(16 * it + 4 * lg + j) * dv + col] = Sr[ct][it][j];
                }
            }
        }
    } else if (wave < NC + NP) {
        // =====================================================================
        // producer: raw loads, decay prefix and decayed operand tiles
        // =====================================================================
        // Lane geometry: lane = rg * QW + cq owns rows 4 rg .. 4 rg + 3 and
        // key channels i0 .. i0 + 3 of this wave's channel strip, so that
        // consecutive lanes load consecutive bytes of a row.
        const int pw = wave - NC;
        // Pacing (pace16 > 0: 16 x 10-ns ticks per chunk of the longest
        // sequence; whole sequences, sorted by length).  The launch is one
        // round of workgroups whose makespan is the longest sequence's chain
        // of chunks; a shorter sequence has slack.  Its producers issue the
        // loads of chunk j no earlier than j T / n after the start (n its
        // chunks, T the longest sequence's chunks x kPaceNs), so its memory
        // traffic spreads over the whole launch instead of competing with
        // the longest chains at the start.
        int pace = 0;  // ticks x 16 per chunk of this sequence
        uint64_t pt0 = 0;
        if (pace16 > 0 && seg.units == nullptr && N > 1 && N <= kSortMax) {
            int lmax = 0;
            for (int j = 0; j < N; ++j) lmax = max(lmax, sSeq[j]);
            const int lc = (lmax + C - 1) / C;
            if (nchunks > 0 && nchunks * 10 < lc * 9)
                pace = static_cast<int>(static_cast<int64_t>(lc) * pace16 / nchunks);
            pt0 = __builtin_amdgcn_s_memrealtime();  // 100 MHz
        }
        const int strip = pw % NPS;  // channel strip
        const int par = pw / NPS;    // parity of the chunks this wave prepares (PP == 2)
        const int rg = lane / QW;
        const int cq = lane % QW;
        const int gq = strip * QW + cq;
        const bool qok = NQ >= QW || gq < NQ;  // idle lanes only when d_k < one strip
        const int i0 = 4 * min(gq, NQ - 1);
        const int vlane = strip * 64 + lane;
        const G* const qh = q + static_cast<size_t>(h) * DK;
        const G* const kh = k + static_cast<size_t>(h) * DK;
        const float* const lah = log_alpha + static_cast<size_t>(h) * (SG ? 1 : DK);
        const float* const bh = beta + h;
        const G* const vh = v + static_cast<size_t>(h) * dv + j0;

        // Raw inputs of the next chunks are in flight while chunk m is
        // prepared: NSET register sets used in turn (chunk m in set m mod
        // NSET), each reloaded right after its chunk's prep consumed it
        // (one set, one chunk ahead, where the raw tiles are large: fp32).
        // Every load is unconditional (rows past the end of the sequence, and
        // chunks past the last, fall outside the buffer ranges and read as
        // zero), so the compiler's wait counts stay exact and a wait for one
        // set never waits for the other.
        constexpr int GS = static_cast<int>(sizeof(G));
        const int rowK = strideK * GS;  // bytes per token row of q and k
        const int strideLA = SG ? H : strideK;  // floats per token row of log alpha
        const int rowLA = strideLA * 4;
        const int rowV = strideV * GS;
        const int rowB = H * 4;
        const int offK = 4 * rg * rowK + i0 * GS;
        const int offLA = 4 * rg * rowLA + (SG ? 0 : i0 * 4);
        const bool loads_beta = strip == 0 && lane < C;  // beta of row `lane`, for the consumers
        // (three where the V items are few, d_k >= 64: the raw loads of three
        // chunks in flight keep more bytes moving per CU when every CU is busy)
        constexpr int NSET = BF16 && PP == 1 ? (DK >= 64 ? 3 : 2) : 1;
        float4 rla[NSET][4];
        R4 rk[NSET][4], rq[NSET][4], rv[NSET][VPT][4];
        float rbeta[NSET];
        struct Rsrc {
            __amdgpu_buffer_rsrc_t k, q, la, v, b;
        };
        auto rsrc_of = [&](int m) __attribute__((always_inline)) {
            const int c0 = chunk_beg(m);
            // chunks past the end: empty ranges, no access (kept in a scalar register)
            const int len = __builtin_amdgcn_readfirstlane(max(0, chunk_len(m)));
            const size_t tok = static_cast<size_t>(c0) * strideK;
            // (the checkpointing pass forms no outputs and reads no q: empty range)
            return Rsrc{buffer_rsrc(kh + tok, len * rowK), buffer_rsrc(qh + tok, CK ? 0 : len * rowK),
                        buffer_rsrc(lah + static_cast<size_t>(c0) * strideLA, len * rowLA),
                        buffer_rsrc(vh + static_cast<size_t>(c0) * strideV, mode == 2 ? 0 : len * rowV),
                        buffer_rsrc(bh + static_cast<size_t>(c0) * H, len * rowB)};
        };
        auto load_chunk = [&](auto X, int m) __attribute__((always_inline)) {
            constexpr int x = decltype(X)::value;
            const Rsrc r = rsrc_of(m);
            rbeta[x] = buf_load_f1(r.b, loads_beta ? lane * rowB : kNoAccess, 0);
#pragma unroll
            for (int vv = 0; vv < VPT; ++vv) {
                const int idx = vlane + 64 * NPS * vv;
                const bool ok = VITEMS % (64 * NPS) == 0 || idx < VITEMS;
                const int c4 = 4 * (idx % (BV / 4));  // value-column quad (fastest: coalesced rows)
                const int r0 = 4 * (idx / (BV / 4));
                const int off = ok ? r0 * rowV + c4 * GS : kNoAccess;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rv[x][vv][rr] = buf_load_raw4<BF16>(r.v, off, rr * rowV);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                if constexpr (SG) {
                    const float a = buf_load_f1(r.la, offLA, rr * rowLA);
                    rla[x][rr] = make_float4(a, a, a, a);
                } else {
                    rla[x][rr] = buf_load_f4(r.la, offLA, rr * rowLA);
                }
                rk[x][rr] = buf_load_raw4<BF16>(r.k, offK, rr * rowK);
                rq[x][rr] = buf_load_raw4<BF16>(r.q, offK, rr * rowK);
            }
        };

        // beta, V^T, cumulative decay and the decayed operand tiles of slot S
        auto prep12 = [&](auto X, int S) __attribute__((always_inline)) {
            constexpr int x = decltype(X)::value;
            if (loads_beta) sBeta(S)[lane] = rbeta[x];
#pragma unroll
            for (int vv = 0; vv < VPT; ++vv) {
                const int idx = vlane + 64 * NPS * vv;
                if (VITEMS % (64 * NPS) == 0 || idx < VITEMS) {
                    const int c4 = 4 * (idx % (BV / 4));
                    const int r0 = 4 * (idx / (BV / 4));
                    R4 cols[4];
                    transpose4<BF16>(rv[x][vv], cols);
#pragma unroll
                    for (int c = 0; c < 4; ++c) T::lds_put_raw4(tile_at<BF16>(tVt(S), vt_off<BF16, UT>(c4 + c, r0 / 4)), cols[c]);
                }
            }
            if (!qok) return;
            // log alpha in log2 units: row-group sums, then the exclusive
            // prefix over the NRG row groups of each channel (QW lanes apart)
            // through this wave's LDS scratch, summed in row-group order.
            float la[4][4], tot[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                la[rr][0] = rla[x][rr].x;
                la[rr][1] = rla[x][rr].y;
                la[rr][2] = rla[x][rr].z;
                la[rr][3] = rla[x][rr].w;
            }
            // Chunk lists (MAP): a strong decay (below kStrongLogAlpha) can
            // only be row 0's.  It acts on the entering state alone (no row
            // of the chunk precedes it), so it is taken out of the rows'
            // exponents and applied through Gamma_C and the state operand's
            // scale 2^ref: the exponents keep the precision of the ordinary
            // rows, and a decay that underflows alpha to 0 (even one whose
            // log2 overflows to -inf) zeroes the entering state exactly.
            float d0[4] = {0.f, 0.f, 0.f, 0.f};  // row 0's strong decay, log2 units
            if constexpr (MAP) {
                float z[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool strong = rg == 0 && la[0][c] < kStrongLogAlpha;
                    z[c] = strong ? la[0][c] * kLog2e : 0.f;
                    if (strong) la[0][c] = 0.f;
                }
                // lane cq (row group 0) holds row 0 of channel quad cq
#pragma unroll
                for (int c = 0; c < 4; ++c) d0[c] = __shfl(z[c], cq);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) tot[c] = ((la[0][c] + la[1][c]) + (la[2][c] + la[3][c])) * kLog2e;
            float4* const scan = reinterpret_cast<float4*>(smem + Sh::OFF_SCAN) + 64 * pw;
            scan[lane] = make_float4(tot[0], tot[1], tot[2], tot[3]);
            // One running sum: the groups before this one (g) are the sum
            // after group rg - 1, and in the wide-decay variant the first
            // half of the chunk (mid) the sum after group NRG / 2 - 1.
            float g[4] = {0.f, 0.f, 0.f, 0.f}, sum[4] = {0.f, 0.f, 0.f, 0.f}, mid[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < NRG; ++r) {
                const float4 t4 = scan[QW * r + cq];
                const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    sum[c] += tv[c];
                    g[c] = r < rg ? sum[c] : g[c];
                    if (r == NRG / 2 - 1) mid[c] = sum[c];
                }
            }
            float Gc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) Gc[c] = __builtin_amdgcn_exp2f(MAP ? d0[c] + sum[c] : sum[c]);
            if (rg == 0) *reinterpret_cast<float4*>(sGC(S) + i0) = make_float4(Gc[0], Gc[1], Gc[2], Gc[3]);
            // Reference point of each channel's exponents: the chunk start; in
            // the wide-decay variant, the middle row for a channel whose decay
            // over the chunk would put 2^-g outside the fp32 range (every
            // exponent is then bounded by the decay of C/2 tokens).
            float ref[4] = {0.f, 0.f, 0.f, 0.f}, GcR[4] = {Gc[0], Gc[1], Gc[2], Gc[3]};
            if constexpr (WIDE) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ref[c] = sum[c] < -kRefSwitchLog2 ? mid[c] : 0.f;
                    GcR[c] = __builtin_amdgcn_exp2f(sum[c] - ref[c]);
                }
                if (rg == 0)
                    *reinterpret_cast<float4*>(sGM(S) + i0) =
                        make_float4(__builtin_amdgcn_exp2f(MAP ? d0[0] + ref[0] : ref[0]),
                                    __builtin_amdgcn_exp2f(MAP ? d0[1] + ref[1] : ref[1]),
                                    __builtin_amdgcn_exp2f(MAP ? d0[2] + ref[2] : ref[2]),
                                    __builtin_amdgcn_exp2f(MAP ? d0[3] + ref[3] : ref[3]));
            }
            float kbar[4][4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 4 * rg + rr;
                float kk[4], qq[4];
                T::unpack4(rk[x][rr], kk);
                T::unpack4(rq[x][rr], qq);
                float gam[4], kh4[4], kg[4], qg[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // exp(+-(g - ref)) as 2^(+-(g2 - ref2)): one v_exp_f32 each;
                    // within the numerical contract the results are normal.
                    g[c] = __builtin_fmaf(la[rr][c], kLog2e, g[c]);
                    if constexpr (WIDE) {
                        gam[c] = __builtin_amdgcn_exp2f(g[c] - ref[c]);
                        kh4[c] = kk[c] * __builtin_amdgcn_exp2f(ref[c] - g[c]);
                        kbar[rr][c] = kh4[c] * GcR[c];
                    } else {
                        gam[c] = __builtin_amdgcn_exp2f(g[c]);
                        kh4[c] = kk[c] * __builtin_amdgcn_exp2f(-g[c]);
                        kbar[rr][c] = kh4[c] * Gc[c];
                    }
                    kg[c] = kk[c] * gam[c];
                    qg[c] = qq[c] * gam[c];
                }
                const int off = quad_off<BF16, UK>(r, i0 / 4);
                lds_store4<BF16>(tile_at<BF16>(tKb(S), off), kg[0], kg[1], kg[2], kg[3]);
                lds_store4<BF16>(tile_at<BF16>(tKh(S), off), kh4[0], kh4[1], kh4[2], kh4[3]);
                lds_store4<BF16>(tile_at<BF16>(tQ(S), off), qg[0], qg[1], qg[2], qg[3]);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                lds_store4<BF16>(tile_at<BF16>(tKbT(S), kbt_off<BF16, UT>(i0 + c, rg)), kbar[0][c], kbar[1][c], kbar[2][c],
                                 kbar[3][c]);
        };

        // Chunk m uses LDS slot m mod 3.  With two producer waves per strip
        // (PP == 2) each takes the chunks of its parity; with one, its NSET
        // register sets take turns, and a chunk count that is not a multiple
        // of NSET ends with up to NSET - 1 virtual chunks past the end (zero
        // inputs): their tiles go to slots every consumer has released and
        // nothing reads them.
        constexpr int STRIDE = PP * NSET;  // chunks between two uses of one register set
        const int m0 = PP == 2 ? par : 0;
        load_chunk(ic<0>{}, m0);
        if constexpr (NSET >= 2) {
            // issued in this order on every path into the loop, so the waits
            // for set 0 count the later sets' loads as issued after it
            asm volatile("" ::: "memory");
            load_chunk(ic<1>{}, m0 + 1);
        }
        if constexpr (NSET >= 3) {
            asm volatile("" ::: "memory");
            load_chunk(ic<2>{}, m0 + 2);
        }
        // O of chunk j, staged by the consumers as O^T quads in the V^T tile
        // of slot S: exactly the quads this wave's V items cover (so no other
        // wave writes them before this wave has read them), transposed back
        // to rows and stored like the V loads, coalesced.  Rows past the end
        // of the sequence fall outside the range and are dropped.
        G* const ohp = obase + static_cast<size_t>(h) * dv + j0;
        auto store_o = [&](int j, int S) __attribute__((always_inline)) {
            const int c0 = chunk_beg(j);
            const int len = __builtin_amdgcn_readfirstlane(chunk_len(j));
            const auto r = buffer_rsrc(ohp + static_cast<size_t>(c0) * strideV, len * rowV);
            // after a failed hand-off in this workgroup: NaN rows instead
            const bool failed =
                __builtin_amdgcn_readfirstlane(__hip_atomic_load(fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
#pragma unroll
            for (int vv = 0; vv < VPT; ++vv) {
                const int idx = vlane + 64 * NPS * vv;
                const bool ok = VITEMS % (64 * NPS) == 0 || idx < VITEMS;
                const int c4 = ok ? 4 * (idx % (BV / 4)) : 0;
                const int r0 = ok ? 4 * (idx / (BV / 4)) : 0;
                R4 q4[4], rows[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) q4[c] = lds_get_raw4<BF16>(tile_at<BF16>(tVt(S), vt_off<BF16, UT>(c4 + c, r0 / 4)));
                transpose4<BF16>(q4, rows);
                if (failed) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) rows[rr] = T::nan4();
                }
                const int off = ok ? r0 * rowV + c4 * GS : kNoAccess;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) buf_store_raw4<BF16>(r, off, rr * rowV, rows[rr]);
            }
        };

        int P = m0;
        auto step = [&](auto X, int m) __attribute__((always_inline)) {
            // slot P last held chunk m - 3: wait until every consumer released
            // it, then store that chunk's O from it
            if (m >= 3) {
                ctr_wait(nFree, NC * (m - 2), fault);
                if constexpr (!CK) store_o(m - 3, P);
            }
            prep12(X, P);
            ctr_publish(prodDone + pw, m + 1, lane);
            if (pace > 0 && m + STRIDE < nchunks) {
                const uint64_t due = pt0 + ((static_cast<uint64_t>(m + STRIDE) * pace) >> 4);
                while (__builtin_amdgcn_s_memrealtime() < due) __builtin_amdgcn_s_sleep(1);
            }
            load_chunk(X, m + STRIDE);
            P += PP;
            if (P >= 3) P -= 3;
        };
        int m = m0;
        for (; m < nchunks; m += STRIDE) {
            step(ic<0>{}, m);
            if constexpr (NSET >= 2) step(ic<1>{}, m + 1);
            if constexpr (NSET >= 3) step(ic<2>{}, m + 2);
        }
        // The last chunks' O stay in slots nobody refills: once every chunk is
        // done, this wave stores those a continued loop would have.
        if (!CK && m - 3 < nchunks) {
            ctr_wait(nFree, NC * nchunks, fault);
            for (; m - 3 < nchunks; m += PP) {
                if (m >= 3) {
                    const int j = m - 3;
                    store_o(j, j % 3);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host launchers.  Consumer waves follow the value slice width
// BV = d_v / v_split: 4 waves x 2 tiles (128), 4 x 1 (64), 2 x 1 (32),
// 1 x 1 (16); producer waves follow d_k.
// ---------------------------------------------------------------------------
template <bool BF16, int DK, int NC, int CT, bool SG, bool WIDE, bool CK = false, bool MAP = false>
static hipError_t launch_prefill_t(const PrefillArgs& a, const SegView& seg, const CkptView& ck = CkptView{},
                                   const ChunkMap& cm = ChunkMap{}) {
    using G = typename Elem<BF16>::G;
    using Sh = PrefillShape<BF16, DK, NC, CT, WIDE>;
    const unsigned units = seg.units ? static_cast<unsigned>(seg.umax) : static_cast<unsigned>(a.N);
    const unsigned per_unit = static_cast<unsigned>(a.v_split) * (seg.units ? 2u : 1u);
    const unsigned grid = units * static_cast<unsigned>(a.H) * per_unit;
    // pacing: the shape whose fully occupied chunk period was measured, on
    // whole sequences (ordered in-kernel), when the launch fills the GPU
    const bool pace = BF16 && DK == 128 && NC == 4 && CT == 2 && seg.units == nullptr && a.N > 1 &&
                      a.N <= kSortMax && grid >= static_cast<unsigned>(a.cus);
    hipLaunchKernelGGL((prefill_kernel<BF16, DK, NC, CT, SG, WIDE, CK, MAP>), dim3(grid), dim3(Sh::NT), 0,
                       static_cast<hipStream_t>(a.stream), static_cast<const G*>(a.q),
                       static_cast<const G*>(a.k), static_cast<const G*>(a.v), a.log_alpha, a.beta,
                       a.S0, a.cu_seqlens, a.N, a.H, a.d_v, a.v_split, static_cast<G*>(a.o), a.S_T, seg, ck, cm,
                       pace ? kPaceNs * 16 / 10 : 0);
    return hipGetLastError();
}

template <bool BF16, int DK, int NC, int CT>
static hipError_t launch_ckpt_sg(const PrefillArgs& a, const CkptView& ck) {
    return a.scalar_gate ? launch_prefill_t<BF16, DK, NC, CT, true, false, true>(a, SegView{}, ck)
                         : launch_prefill_t<BF16, DK, NC, CT, false, false, true>(a, SegView{}, ck);
}

template <bool BF16, int DK>
static hipError_t launch_ckpt_dk(const PrefillArgs& a, const CkptView& ck) {
    switch (a.d_v) {  // whole value columns: v_split 1
        case 128: return launch_ckpt_sg<BF16, DK, 4, 2>(a, ck);
        case 64: return launch_ckpt_sg<BF16, DK, 4, 1>(a, ck);
        case 32: return launch_ckpt_sg<BF16, DK, 2, 1>(a, ck);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_ckpt(const PrefillArgs& a0, const CkptView& ck) {
    PrefillArgs a = a0;
    a.v_split = 1;
    switch (a.d_k) {
        case 32: return a.bf16 ? launch_ckpt_dk<true, 32>(a, ck) : launch_ckpt_dk<false, 32>(a, ck);
        case 64: return a.bf16 ? launch_ckpt_dk<true, 64>(a, ck) : launch_ckpt_dk<false, 64>(a, ck);
        case 128: return a.bf16 ? launch_ckpt_dk<true, 128>(a, ck) : launch_ckpt_dk<false, 128>(a, ck);
        default: return hipErrorInvalidValue;
    }
}

int prefill_chunk_len(int32_t d_k, bool bf16) {
    switch (d_k) {
        case 32: return bf16 ? kChunk<true, 32> : kChunk<false, 32>;
        case 64: return bf16 ? kChunk<true, 64> : kChunk<false, 64>;
        case 128: return bf16 ? kChunk<true, 128> : kChunk<false, 128>;
        default: return 0;
    }
}

template <bool BF16, int DK, int NC, int CT>
static hipError_t launch_prefill_sg(const PrefillArgs& a, const SegView& seg) {
    if (a.wide_decay)
        return a.scalar_gate ? launch_prefill_t<BF16, DK, NC, CT, true, true>(a, seg)
                             : launch_prefill_t<BF16, DK, NC, CT, false, true>(a, seg);
    return a.scalar_gate ? launch_prefill_t<BF16, DK, NC, CT, true, false>(a, seg)
                         : launch_prefill_t<BF16, DK, NC, CT, false, false>(a, seg);
}

template <bool BF16, int DK>
static hipError_t launch_prefill_dk(const PrefillArgs& a, const SegView& seg) {
    switch (a.d_v / a.v_split) {
        case 128: return launch_prefill_sg<BF16, DK, 4, 2>(a, seg);
        case 64: return launch_prefill_sg<BF16, DK, 4, 1>(a, seg);
        case 32: return launch_prefill_sg<BF16, DK, 2, 1>(a, seg);
        case 16: return launch_prefill_sg<BF16, DK, 1, 1>(a, seg);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
static hipError_t launch_prefill_dt(const PrefillArgs& a, const SegView& seg) {
    switch (a.d_k) {
        case 32: return launch_prefill_dk<BF16, 32>(a, seg);
        case 64: return launch_prefill_dk<BF16, 64>(a, seg);
        case 128: return launch_prefill_dk<BF16, 128>(a, seg);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs& a) {
    SegView seg{};
    const bool segmented = prefill_segmented(a.N, a.T_tot, a.H, a.d_k, a.d_v, a.cus);
    if (segmented) {
        if (a.workspace == nullptr) return hipErrorInvalidValue;
        const hipError_t e = launch_seg_plan(a, &seg);
        if (e != hipSuccess) return e;
    }
    const hipError_t e = a.bf16 ? launch_prefill_dt<true>(a, seg) : launch_prefill_dt<false>(a, seg);
    if (e != hipSuccess || !segmented) return e;
    return launch_seg_fixup(a, seg);
}

template <bool BF16, int DK, int NC, int CT>
static hipError_t launch_mapped_sg(const PrefillArgs& a, const ChunkMap& cm) {
    return a.scalar_gate ? launch_prefill_t<BF16, DK, NC, CT, true, true, false, true>(a, SegView{}, CkptView{}, cm)
                         : launch_prefill_t<BF16, DK, NC, CT, false, true, false, true>(a, SegView{}, CkptView{}, cm);
}

template <bool BF16, int DK>
static hipError_t launch_mapped_dk(const PrefillArgs& a, const ChunkMap& cm) {
    switch (a.d_v / a.v_split) {
        case 128: return launch_mapped_sg<BF16, DK, 4, 2>(a, cm);
        case 64: return launch_mapped_sg<BF16, DK, 4, 1>(a, cm);
        case 32: return launch_mapped_sg<BF16, DK, 2, 1>(a, cm);
        default: return hipErrorInvalidValue;
    }
}

// Any-decay prefill: the chunk lists, then one workgroup per (sequence,
// head, value slice) over them (never segmented).  The value split follows
// the rule of default_v_split for whole sequences.
hipError_t launch_prefill_mapped(const PrefillArgs& a0) {
    PrefillArgs a = a0;
    a.v_split = a.d_v == 128 && static_cast<int64_t>(a.N) * a.H * 2 <= a.cus / 2 ? 2 : 1;
    ChunkMap cm{};
    const hipError_t e = launch_any_map(a, &cm);
    if (e != hipSuccess) return e;
    switch (a.d_k) {
        case 32: return a.bf16 ? launch_mapped_dk<true, 32>(a, cm) : launch_mapped_dk<false, 32>(a, cm);
        case 64: return a.bf16 ? launch_mapped_dk<true, 64>(a, cm) : launch_mapped_dk<false, 64>(a, cm);
        case 128: return a.bf16 ? launch_mapped_dk<true, 128>(a, cm) : launch_mapped_dk<false, 128>(a, cm);
        default: return hipErrorInvalidValue;
    }
}

int32_t default_v_split(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16, int cus) {
    (void)bf16;
    // Segmented runs: one unit per segment (at most seg_units_max of them).
    const int64_t seqs = prefill_segmented(N, T_tot, H, d_k, d_v, cus) ? seg_units_max(N, T_tot) : N;
    const int64_t units = seqs * H;
    // The chunk period of a workgroup barely depends on how many value
    // columns it carries, so extra workgroups do not shorten a sequence's
    // chain; they repeat the chunk's producer and job work.  The 64-column
    // shape (two producer waves per channel strip) has the shortest period
    // while the GPU is lightly loaded (measured, 4096-token workload: 1.88
    // us per chunk against 2.2 us with 128 columns and 2.1 us with 16), but
    // not at full occupancy.  So 128 value columns split in two only when
    // the launch then fills at most half of the CUs; every split gives the
    // same bits.
    if (d_v == 128 && units * 2 <= cus / 2) return 2;
    return 1;
}

}  // namespace kda
