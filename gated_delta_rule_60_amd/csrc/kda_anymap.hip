// kda_anymap.hip -- chunk lists of the any-decay prefill.
//
// The chunked prefill evaluates exp(+-(g_r - ref)) of each channel's
// cumulative decay g inside a chunk in fp32; the wide-decay variant bounds
// every such exponent by the decay of half a chunk, taken from the middle
// row ("Kimi Linear：让长上下文大模型真正实用的线性注意力架构", section 三.2
// names chunk-parallel evaluation; the bound is this implementation's).  A
// token with a strong decay (log alpha below kStrongLogAlpha on some channel,
// up to a hard reset) breaks that bound only if rows of the chunk lie on
// both sides of it: the rows after it then need 2^(ref - g) with g far below
// ref.  Put at row 0 of a chunk it is harmless: no row of the chunk precedes
// it, so the prefill applies its decay to the entering state alone (through
// the chunk's total decay and the state operand's scale) and keeps it out of
// the rows' exponents, and the other rows decay by at most kStrongLogAlpha
// per token.
//
// So the any-decay prefill cuts each (sequence, head) into chunks that
// start at the sequence start, at every strong token, and every C tokens
// after either: the chunk starts are the tokens t with
// (t - A(t)) mod C == 0, A(t) the last anchor (sequence start or strong
// token) at or before t.  A chunk shorter than C (one that ends at the next
// anchor) is padded with zero rows, exactly like the last chunk of a
// sequence, so the chunk algebra is unchanged; the recurrence over the real
// tokens is computed exactly (the zero rows are identity steps).
//
// Two kernels.  The first reads log alpha once, fully parallel over blocks
// of 256 tokens and heads (a min over the key channels, coalesced, every
// load in flight at once), and writes one strong-token flag byte per token
// and head.  The second, one workgroup per (sequence, head), walks the flag
// bytes in blocks of 1024 tokens: a max-scan for A(t) and a sum-scan for the
// list positions, carried from block to block.  Output per (sequence, head):
// count = number of chunks, and starts[0 .. count] = the chunk starts
// followed by the sequence end.
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kFlagTokens = 256;   // tokens per flag workgroup (one head)
constexpr int kFlagThreads = 256;
constexpr int kListThreads = 1024;  // tokens per block of the list scan
constexpr int kListWaves = kListThreads / 64;

// Workspace: counts [N H] int32 | starts [H][T_tot + 2 N] int32 | flags [H][T_tot] bytes
struct MapLayout {
    size_t off_starts, off_flags, bytes;
};
MapLayout map_layout(int32_t N, int64_t T_tot, int32_t H) {
    auto up256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    MapLayout L{};
    L.off_starts = up256(static_cast<size_t>(N) * H * 4);
    L.off_flags = L.off_starts + up256(static_cast<size_t>(H) * static_cast<size_t>(T_tot + 2 * static_cast<int64_t>(N)) * 4);
    L.bytes = L.off_flags + static_cast<size_t>(H) * static_cast<size_t>(T_tot);
    return L;
}

// Strong-token flags of kFlagTokens tokens of one head.  Rows past the end
// of the batch fall outside the buffer range and read as zero (not strong).
// Offsets fit in 32 bits: a row of log alpha holds at most 2^20 channels x
// heads (checked on the host), so 256 rows span at most 2^30 bytes.
template <int DK, bool SG>
__global__ __launch_bounds__(kFlagThreads) void strong_flags_kernel(const float* __restrict__ log_alpha,
                                                                   int64_t T_tot, int H,
                                                                   unsigned char* __restrict__ flags) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x % H;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x / H) * kFlagTokens;
    const int rows = static_cast<int>(T_tot - t0 < kFlagTokens ? T_tot - t0 : kFlagTokens);
    unsigned char* const fl = flags + static_cast<size_t>(h) * T_tot + t0;
    if constexpr (SG) {
        const auto r = buffer_rsrc(log_alpha + t0 * H + h, rows * H * 4);
        const float x = buf_load_f1(r, tid * H * 4, 0);
        if (tid < rows) fl[tid] = x < kStrongLogAlpha;
    } else {
        // QPT lanes read one token's DK channels as float4s; each wave covers
        // 64 tokens, TPI per load instruction
        constexpr int QPT = DK / 4, TPI = 64 / QPT, NI = 64 / TPI;
        static_assert(kFlagThreads == 256 && kFlagTokens == 256, "four waves of 64 tokens");
        const int sub = lane / QPT, quad = lane % QPT;
        const int rowB = H * DK * 4;
        const auto r = buffer_rsrc(log_alpha + (t0 * H + h) * DK, rows * rowB);
        float mn[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float4 x = buf_load_f4(r, (64 * wave + TPI * i + sub) * rowB + 16 * quad, 0);
            mn[i] = fminf(fminf(x.x, x.y), fminf(x.z, x.w));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float m = mn[i];
#pragma unroll
            for (int d = 1; d < QPT; d <<= 1) m = fminf(m, __shfl_xor(m, d));
            const int row = 64 * wave + TPI * i + sub;
            if (quad == 0 && row < rows) fl[row] = m < kStrongLogAlpha;
        }
    }
}

__device__ __forceinline__ int wave_incl_max(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x = max(x, y);
    }
    return x;
}

__device__ __forceinline__ int wave_incl_sum(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

// Chunk list of one (sequence, head) from its flag bytes.
__global__ __launch_bounds__(kListThreads) void chunk_list_kernel(const unsigned char* __restrict__ flags,
                                                                  const int32_t* __restrict__ cu, int64_t T_tot,
                                                                  int H, int cmask, int64_t stride,
                                                                  int* __restrict__ count,
                                                                  int* __restrict__ starts) {
    __shared__ int sMax[kListWaves], sSum[kListWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    const int t_beg = cu[n], t_end = cu[n + 1];
    const unsigned char* const fl = flags + static_cast<size_t>(h) * T_tot;
    int* const list = starts + h * stride + t_beg + 2 * n;
    int carryA = t_beg;  // the sequence start is an anchor
    int carryN = 0;      // chunk starts found so far
    int strong = t_beg + tid < t_end ? fl[t_beg + tid] : 0;
    for (int blk = t_beg; blk < t_end; blk += kListThreads) {
        const int t = blk + tid;
        const bool valid = t < t_end;
        const int cur = strong;
        // the next block's flag, in flight during this block's scans
        strong = t + kListThreads < t_end ? fl[t + kListThreads] : 0;
        // last anchor at or before each token, then the chunk starts
        int a = valid && cur ? t : -1;
        a = wave_incl_max(a, lane);
        if (lane == 63) sMax[wave] = a;
        __syncthreads();
        int before = carryA;
        for (int w = 0; w < wave; ++w) before = max(before, sMax[w]);
        a = max(a, before);
        const int st = valid && ((t - a) & cmask) == 0;
        const int pos = wave_incl_sum(st, lane);
        if (lane == 63) sSum[wave] = pos;
        __syncthreads();
        int base = carryN;
        for (int w = 0; w < wave; ++w) base += sSum[w];
        if (st) list[base + pos - 1] = t;
        // carry: the block's last anchor and its chunk starts
        int bmax = carryA, bsum = 0;
        for (int w = 0; w < kListWaves; ++w) {
            bmax = max(bmax, sMax[w]);
            bsum += sSum[w];
        }
        carryA = bmax;
        carryN += bsum;
        __syncthreads();  // sMax and sSum are rewritten by the next block
    }
    if (tid == 0) {
        list[carryN] = t_end;
        count[static_cast<size_t>(n) * H + h] = carryN;
    }
}

template <int DK>
hipError_t launch_flags_dk(const PrefillArgs& a, unsigned char* flags) {
    const int64_t blocks = (a.T_tot + kFlagTokens - 1) / kFlagTokens;
    if (blocks == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(blocks * a.H);
    const hipStream_t st = static_cast<hipStream_t>(a.stream);
    if (a.scalar_gate)
        hipLaunchKernelGGL((strong_flags_kernel<DK, true>), dim3(grid), dim3(kFlagThreads), 0, st, a.log_alpha, a.T_tot,
                           a.H, flags);
    else
        hipLaunchKernelGGL((strong_flags_kernel<DK, false>), dim3(grid), dim3(kFlagThreads), 0, st, a.log_alpha,
                           a.T_tot, a.H, flags);
    return hipGetLastError();
}

}  // namespace

size_t any_map_bytes(int32_t N, int64_t T_tot, int32_t H) { return map_layout(N, T_tot, H).bytes; }

hipError_t launch_any_map(const PrefillArgs& a, ChunkMap* m) {
    const MapLayout L = map_layout(a.N, a.T_tot, a.H);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    unsigned char* flags = ws + L.off_flags;
    m->count = reinterpret_cast<const int*>(ws);
    m->starts = reinterpret_cast<const int*>(ws + L.off_starts);
    m->stride = a.T_tot + 2 * static_cast<int64_t>(a.N);
    hipError_t e;
    switch (a.d_k) {
        case 32: e = launch_flags_dk<32>(a, flags); break;
        case 64: e = launch_flags_dk<64>(a, flags); break;
        case 128: e = launch_flags_dk<128>(a, flags); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int C = prefill_chunk_len(a.d_k, a.bf16);
    const unsigned grid = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H);
    hipLaunchKernelGGL(chunk_list_kernel, dim3(grid), dim3(kListThreads), 0, static_cast<hipStream_t>(a.stream), flags,
                       a.cu_seqlens, a.T_tot, a.H, C - 1, m->stride, const_cast<int*>(m->count),
                       const_cast<int*>(m->starts));
    return hipGetLastError();
}

}  // namespace kda
