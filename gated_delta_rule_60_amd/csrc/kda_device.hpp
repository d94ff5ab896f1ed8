// kda_device.hpp -- device-side helpers for the gfx950 KDA kernels:
// storage types, bf16 conversion, and 16x16 MFMA tile fragments.
//
// MFMA tile conventions (wave64, gfx950).  A 16x16 fp32 accumulator tile is
// held as four floats per lane: lane l holds column (l & 15), rows
// 4*(l >> 4) + {0,1,2,3}.  This is the "C layout".
//
// A reduction over a 32-deep block of k is one "frag8" per operand: eight
// values per lane.  Lane l (row or column index l & 15, group g = l >> 4)
// supplies slot s = 4*h + j for logical k = 16*h + 4*g + j (h in {0,1},
// j in {0..3}).  Because both operands of a product use this same slot -> k
// map, the hardware's own k ordering inside the instruction is irrelevant,
// and two C-layout tiles stacked along k (rows 0..15 and 16..31) *are* a
// frag8 operand with no data movement.  A 16-deep block is a "frag4":
// slot j <-> k = 4*g + j, which is exactly one C-layout tile.
//
//   bf16: frag8 -> v_mfma_f32_16x16x32_bf16, frag4 -> the same with the upper k half zero
//   f32 : frag8 -> 8 x v_mfma_f32_16x16x4_f32,  frag4 -> 4 x v_mfma_f32_16x16x4_f32
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs are finite in this library).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) { return exp2f(x * kLog2e); }

// ---------------------------------------------------------------------------
// Storage traits.  G = element type in global memory for q, k, v, o;
// E = element type of MFMA operand tiles in LDS.
// ---------------------------------------------------------------------------
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
    using G = uint16_t;
    using E = __bf16;
    using F8 = bf16x8_t;
    using F4 = bf16x4_t;
    using R4 = uint2;  // four consecutive global elements, raw
    __device__ static __forceinline__ R4 raw4(const G* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ static __forceinline__ void unpack4(const R4& r, float (&x)[4]) {
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xFFFF0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xFFFF0000u);
    }
    // raw global quad -> four LDS operand elements (bit copy)
    __device__ static __forceinline__ void lds_put_raw4(E* p, const R4& r) { *reinterpret_cast<uint2*>(p) = r; }
    // four quiet-NaN elements, raw
    __device__ static __forceinline__ R4 nan4() { return make_uint2(0x7FC07FC0u, 0x7FC07FC0u); }
    // four consecutive global elements -> floats
    __device__ static __forceinline__ void load4(const G* p, float (&x)[4]) {
        const uint2 r = *reinterpret_cast<const uint2*>(p);
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xFFFF0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xFFFF0000u);
    }
    // round to nearest even (v_cvt_pk_bf16_f32)
    __device__ static __forceinline__ void store4(G* p, const float (&x)[4]) {
        bf16x4_t r;
        r[0] = static_cast<__bf16>(x[0]);
        r[1] = static_cast<__bf16>(x[1]);
        r[2] = static_cast<__bf16>(x[2]);
        r[3] = static_cast<__bf16>(x[3]);
        *reinterpret_cast<bf16x4_t*>(p) = r;
    }
    __device__ static __forceinline__ float to_f32(G x) { return bf16_to_f32(x); }
    __device__ static __forceinline__ E to_e(float x) { return static_cast<__bf16>(x); }
    __device__ static __forceinline__ float e_to_f32(E x) { return static_cast<float>(x); }
};

template <>
struct Elem<false> {
    using G = float;
    using E = float;
    using F8 = f32x8_t;
    using F4 = f32x4_t;
    using R4 = float4;
    __device__ static __forceinline__ R4 raw4(const G* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static __forceinline__ void unpack4(const R4& r, float (&x)[4]) {
        x[0] = r.x;
        x[1] = r.y;
        x[2] = r.z;
        x[3] = r.w;
    }
    __device__ static __forceinline__ void lds_put_raw4(E* p, const R4& r) { *reinterpret_cast<float4*>(p) = r; }
    __device__ static __forceinline__ R4 nan4() {
        const float n = __builtin_nanf("");
        return make_float4(n, n, n, n);
    }
    __device__ static __forceinline__ void load4(const G* p, float (&x)[4]) {
        const float4 r = *reinterpret_cast<const float4*>(p);
        x[0] = r.x;
        x[1] = r.y;
        x[2] = r.z;
        x[3] = r.w;
    }
    __device__ static __forceinline__ void store4(G* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
    __device__ static __forceinline__ float to_f32(G x) { return x; }
    __device__ static __forceinline__ E to_e(float x) { return x; }
    __device__ static __forceinline__ float e_to_f32(E x) { return x; }
};

// ---------------------------------------------------------------------------
// Fragment loads from LDS.  `base` points at element [row 0][k 0] of a
// row-major tile with row stride `ld` elements; the lane reads row (l & 15)
// and k slots as described above.  Works for both A operands (rows = m) and
// B operands given as their transpose (rows = n).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::F8 lds_frag8(const typename Elem<BF16>::E* base,
                                                             int ld, int lane) {
    const typename Elem<BF16>::E* p = base + (lane & 15) * ld + 4 * (lane >> 4);
    if constexpr (BF16) {
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(p);
        const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(p);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::F4 lds_frag4(const typename Elem<BF16>::E* base,
                                                             int ld, int lane) {
    const typename Elem<BF16>::E* p = base + (lane & 15) * ld + 4 * (lane >> 4);
    return *reinterpret_cast<const typename Elem<BF16>::F4*>(p);
}

// Fragments built from C-layout accumulator tiles (fp32 -> operand type).
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::F8 acc_frag8(const f32x4_t& lo, const f32x4_t& hi) {
    typename Elem<BF16>::F8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = Elem<BF16>::to_e(lo[j]);
        r[4 + j] = Elem<BF16>::to_e(hi[j]);
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::F4 acc_frag4(const f32x4_t& t) {
    typename Elem<BF16>::F4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = Elem<BF16>::to_e(t[j]);
    return r;
}

// acc += A * B over a 32-deep k block.
template <bool BF16>
__device__ __forceinline__ f32x4_t mma8(f32x4_t acc, const typename Elem<BF16>::F8& a,
                                        const typename Elem<BF16>::F8& b) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
        return acc;
    }
}

// acc += A * B over a 16-deep k block.
//
// bf16: issued as v_mfma_f32_16x16x32_bf16 with the upper k half zeroed
// rather than as v_mfma_f32_16x16x16_bf16.  Accumulation chains that mix the
// two opcodes (a 16x16x32 result fed straight into a 16x16x16 as its
// accumulator) were compiled with no wait states between them and produced
// wrong accumulator values on gfx950; keeping one opcode per chain avoids
// the mixed-opcode dependency altogether.
template <bool BF16>
__device__ __forceinline__ f32x4_t mma4(f32x4_t acc, const typename Elem<BF16>::F4& a,
                                        const typename Elem<BF16>::F4& b) {
    if constexpr (BF16) {
        const bf16x4_t zero = {};
        const bf16x8_t a8 = __builtin_shufflevector(a, zero, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t b8 = __builtin_shufflevector(b, zero, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
        return acc;
    }
}

// ---------------------------------------------------------------------------
// Raw buffer resource over [base, base + bytes): a load at a byte offset at
// or past `bytes` returns zero without touching memory, and a store there is
// dropped.  Per-chunk resources make every load one instruction (a per-lane
// offset fixed for the whole sequence plus a scalar row offset) and zero the
// rows past a sequence end.  kNoAccess is a buffer offset beyond every range
// the kernels build: ranges span at most one chunk's rows of one tensor (C
// rows of H * max(d_k, d_v) elements, at most 2^27 bytes under the host's
// limit H * max(d_k, d_v) <= 2^20), and the offset plus a few rows' stride
// stays below 2^32.
// ---------------------------------------------------------------------------
constexpr int kNoAccess = 0x7FFFFF00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 buf_load_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                       __uint_as_float(x[3]));
}

__device__ __forceinline__ float buf_load_f1(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Stores through a buffer range: a store whose offset (voffset + soffset)
// falls past the range is dropped by the hardware, like the loads above read
// zero there.
__device__ __forceinline__ void buf_store_f1(__amdgpu_buffer_rsrc_t r, int voff, int soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}

// A buffer store of more than 8 bytes followed by a vector-ALU write of its
// data registers needs a wait state between them.  The compiler inserts it
// only for stores whose soffset is not a register (it takes the hazard to
// be absent otherwise), and on gfx950 it is not: with a register soffset a
// data register overwritten by the next instruction was measured to corrupt
// one element of some lanes' stores.  Wide stores therefore pass their whole
// offset in voffset, with an immediate soffset of 0; the sum is formed
// unsigned, so an offset past the range (kNoAccess) stays past it.
__device__ __forceinline__ int store_voffset(int voff, int soff) {
    return static_cast<int>(static_cast<unsigned>(voff) + static_cast<unsigned>(soff));
}

__device__ __forceinline__ void buf_store_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff, float a, float b, float c,
                                             float d) {
    const u32x4_t x = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, store_voffset(voff, soff), 0, 0);
}

}  // namespace kda
