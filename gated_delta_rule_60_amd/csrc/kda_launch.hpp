// kda_launch.hpp -- internal host interface between the C ABI layer and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Segmented prefill.  When a batch has too few (sequence, head) pairs to
// fill the GPU (N * H below half the device's compute units), a sequence longer than its segment
// length runs as segments (the last one shorter), each segment of each head
// in its own workgroups, so one long sequence spreads over many CUs.  The
// segment length depends on the sequence's own length only: about a quarter
// of it, a multiple of 512 tokens between kSegMinTokens and kSegTokens
// (seg_len_for in kda_segment.hip).  A segment after the first starts from the zero state, and an
// identity run over it (V = 0, S0 = I) gives its transition M and
// q^_t = M_t^T q_t; fix-up passes then add the true entering state's
// contribution.  With enough pairs the extra identity work and fix-up
// traffic cost more than the shorter critical path saves.  Few, long
// segments keep that extra work small: a 128k-token sequence runs as four
// 32k-token segments, seven runs per head (one round of workgroups for 32
// heads on 256 compute units), three identity runs and three chain steps.
constexpr int kSegTokens = 32768;    // longest segment
constexpr int kSegMinTokens = 1024;  // shortest segment length a sequence is cut at
// Compute units assumed when the current device cannot be queried (MI355X).
constexpr int kDefaultCUs = 256;

// Upper bound on the segments of a batch of N sequences of T_tot tokens in
// all.  A sequence of len tokens is cut into P <= ceil(len / kSegMinTokens)
// segments, and P <= 4 unless its segments are kSegTokens long, when
// P - 1 <= floor(len / kSegTokens); summed over the sequences,
//     sum P <= N + min(T_tot / kSegMinTokens, 3 N + T_tot / kSegTokens).
inline int64_t seg_units_max(int32_t N, int64_t T_tot) {
    const int64_t a = T_tot / kSegMinTokens, b = 3 * static_cast<int64_t>(N) + T_tot / kSegTokens;
    return N + (a < b ? a : b);
}

// Sets the text kda_last_error returns on the calling thread.
void set_last_error(const char* msg);

// Compute units of the current device, queried once per device.
hipError_t device_cus(int* cus);
// The same, or kDefaultCUs when no device can be queried (host-side queries).
int device_cus_or_default();

// The device plan and workspace a segmented launch uses (units == nullptr:
// whole sequences, one workgroup per (sequence, head, value slice)).
struct SegView {
    const int4* units;  // [count] {sequence, segment, token begin, token end}
    const int* count;   // number of units
    void* qhat;         // [T_tot][H][d_k] identity-run outputs q^ (storage type)
    float* mstate;      // [umax][H][d_k][d_k] identity-run final states M
    float* dstate;      // [umax][H][d_k][d_v] final states of later segments from the
                        // zero state; the chain pass replaces them with entering states
    int umax;           // units the grid covers
};

// Checkpoints the forward pass writes for the chunked backward pass (both
// null for an ordinary prefill).  Per chunk slot (t_beg / C + n + i for
// chunk i of sequence n, C the prefill's chunk length) and head:
//   s   [DK / 16][DV / 32][64 lanes][8]  storage type: the state entering the
//       chunk, as MFMA A-operand fragments with the value columns as the
//       reduction index (lane l: row 16 it + (l & 15), columns
//       32 kb + 4 (l >> 4) + {0..3} and 32 kb + 16 + 4 (l >> 4) + {0..3});
//   w0  [DV / 16][C / 16][64 lanes][4]   storage type: W0 = V - K~ S in the
//       C layout (lane l: column 16 ct + (l & 15), rows 16 rt + 4 (l >> 4) + {0..3}).
struct CkptView {
    void* s;
    void* w0;
};

// Chunk lists of the any-decay prefill (kda_anymap.hip).  For sequence n and
// head h: count[n H + h] chunks, starting at the tokens
// starts[h stride + cu[n] + 2 n + i] (i < count, ascending), followed by the
// sequence end; each chunk holds at most C tokens (the prefill's chunk
// length).  A chunk ends early where a token with a strong decay follows, so
// that such a token is always the first row of its chunk.
struct ChunkMap {
    const int* count;
    const int* starts;
    int64_t stride;  // T_tot + 2 N
};
// A token whose log alpha is below this on some channel (natural log units)
// starts a chunk of the any-decay prefill.  The wide-decay contract allows
// -80 over 16 consecutive tokens, so runs of the other tokens stay within it.
constexpr float kStrongLogAlpha = -5.f;

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S0;  // may be null
    const int32_t* cu_seqlens;
    int32_t N;
    int64_t T_tot;
    int32_t H, d_k, d_v;
    bool bf16;
    void* o;
    float* S_T;
    int32_t v_split;  // 1, 2, 4, 8; d_v / v_split >= 16
    void* stream;
    void* workspace;  // at least prefill_workspace_bytes(...) bytes
    int cus = kDefaultCUs;     // compute units of the device the launch rules assume
    bool scalar_gate = false;  // log_alpha is [T_tot, H] (one gate per token and head)
    bool wide_decay = false;   // exponents of strongly decaying channels from the chunk's middle row
    bool any_decay = false;    // any finite log_alpha: chunk lists + chunked kernel, or token-recurrent
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    float* S;
    int32_t N, H, d_k, d_v;
    bool bf16;
    void* o;
    void* stream;
    bool scalar_gate = false;  // log_alpha is [N, H] (one gate per sequence and head)
};

struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S0;    // may be null (zero initial state)
    const int32_t* cu_seqlens;
    const void* dO;     // [T_tot, H, d_v], storage type of q/k/v
    const float* dS_T;  // may be null (no gradient reaches the final states)
    int32_t N;
    int64_t T_tot;
    int32_t H, d_k, d_v;
    bool bf16;
    float *dq, *dk, *dv, *dlog_alpha, *dbeta, *dS0;
    void* workspace;  // at least prefill_bwd_workspace_bytes(...) bytes, 256-byte aligned
    void* stream;
    bool scalar_gate = false;  // log_alpha and dlog_alpha are [T_tot, H] (one gate per token and head)
};

hipError_t launch_prefill(const PrefillArgs& a);
// The forward pass with checkpoints instead of outputs (o and S_T are not
// written): one pass, whole value columns (v_split 1), never segmented.
hipError_t launch_prefill_ckpt(const PrefillArgs& a, const CkptView& ck);
// Chunk length of the prefill kernel for these sizes (the checkpoint slot size).
int prefill_chunk_len(int32_t d_k, bool bf16);
// Token-recurrent prefill for any decay range (kda_backward.hip).
hipError_t launch_prefill_recurrent(const PrefillArgs& a);
// Chunked prefill for any decay range: the chunk lists (kda_anymap.hip), then
// the wide-decay prefill kernel over those chunks.  The workspace holds the
// lists: any_map_bytes(...) bytes, 256-byte aligned.
hipError_t launch_prefill_mapped(const PrefillArgs& a);
hipError_t launch_any_map(const PrefillArgs& a, ChunkMap* m);
size_t any_map_bytes(int32_t N, int64_t T_tot, int32_t H);

// Whether a prefill of these sizes runs segmented on a device with `cus`
// compute units, and the workspace bytes it then needs (0 when it does not).
bool prefill_segmented(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, int cus);
size_t prefill_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16,
                               int cus);
// Segmented prefill passes around the prefill kernel (kda_segment.hip): the
// plan (before it) and the state chain plus output correction (after it).
hipError_t launch_seg_plan(const PrefillArgs& a, SegView* view);
hipError_t launch_seg_fixup(const PrefillArgs& a, const SegView& v);
hipError_t launch_decode(const DecodeArgs& a);
// Token-recurrent backward pass of the prefill (kda_backward.hip), for any
// decay range, and the workspace it needs: fp32 state checkpoints every 16
// tokens and one residual row per token-head.
hipError_t launch_prefill_bwd(const BackwardArgs& a);
size_t prefill_bwd_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v);
// Chunked backward pass (kda_bwd_chunk.hip): the forward with checkpoints,
// then the reverse walk over the chunks; its workspace holds the checkpoints
// (the entering state and W0 of every chunk, storage type).
hipError_t launch_prefill_bwd_chunk(const BackwardArgs& a);
size_t prefill_bwd_chunk_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                         bool bf16);

// Launch shape kda_prefill picks for these sizes on a device with `cus`
// compute units (see kda_prefill.hip).
int32_t default_v_split(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16, int cus);

}  // namespace kda
