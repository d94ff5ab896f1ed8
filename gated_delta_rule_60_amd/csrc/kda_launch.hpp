// kda_launch.hpp -- internal host interface between the C ABI layer and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Segmented prefill.  When a batch has too few (sequence, head) pairs to
// fill the GPU (N * H < kSegMaxPairs), a sequence longer than its segment
// length runs as segments (the last one shorter), each segment of each head
// in its own workgroups, so one long sequence spreads over many CUs.  The
// segment length depends on the sequence's own length only: about a quarter
// of it, a multiple of 512 tokens between kSegMinTokens and kSegTokens
// (seg_len_for in kda_segment.hip).  A segment after the first starts from the zero state, and an
// identity run over it (V = 0, S0 = I) gives its transition M and
// q^_t = M_t^T q_t; fix-up passes then add the true entering state's
// contribution.  With enough pairs the extra identity work and fix-up
// traffic cost more than the shorter critical path saves.
constexpr int kSegTokens = 4096;     // longest segment
constexpr int kSegMinTokens = 1024;  // shortest segment length a sequence is cut at
constexpr int kSegMaxPairs = 128;

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
    bool scalar_gate = false;  // log_alpha is [T_tot, H] (one gate per token and head)
    bool wide_decay = false;   // exponents of strongly decaying channels from the chunk's middle row
    bool any_decay = false;    // token-recurrent kernel: any finite log_alpha (kda_backward.hip)
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
// Token-recurrent prefill for any decay range (kda_backward.hip).
hipError_t launch_prefill_recurrent(const PrefillArgs& a);

// Whether a prefill of these sizes runs segmented, and the workspace bytes it
// then needs (0 when it does not).
bool prefill_segmented(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v);
size_t prefill_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16);
// Segmented prefill passes around the prefill kernel (kda_segment.hip): the
// plan (before it) and the state chain plus output correction (after it).
hipError_t launch_seg_plan(const PrefillArgs& a, SegView* view);
hipError_t launch_seg_fixup(const PrefillArgs& a, const SegView& v);
hipError_t launch_decode(const DecodeArgs& a);
// Backward pass of the prefill (kda_backward.hip) and the workspace it needs:
// fp32 state checkpoints every 16 tokens and one residual row per token-head.
hipError_t launch_prefill_bwd(const BackwardArgs& a);
size_t prefill_bwd_workspace_bytes(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v);

// Launch shape kda_prefill picks for these sizes (see kda_prefill.hip).
int32_t default_v_split(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v, bool bf16);

}  // namespace kda
