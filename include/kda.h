/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward pass.
 *
 * What is computed.  For every sequence n and head h, token by token, the
 * KDA update rule of "Kimi Linear：让长上下文大模型真正实用的线性注意力架构"
 * (juejin.cn), section 三.5:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                                   (read-out after the update)
 *
 * alpha_t = exp(log_alpha_t) holds one retention factor per key channel (the
 * fine-grained gate of section 三.1); beta_t is one scalar step size per token
 * and head (section 三.5 reads the update as one online gradient-descent step
 * of size beta_t).  S is a d_k x d_v matrix per (sequence, head): row i is key
 * channel i, column j is value channel j.  The pages apply no rotary position
 * encoding (section 三.4, NoPE), and neither does this library: q and k are
 * used as given (scaling and normalisation are the caller's).  The read-out
 * rule is not printed on the pages; o_t = S_t^T q_t is the numerator of the
 * kernelised linear-attention form Q (K^T V) on the xdnf.cn page, section 2.2.
 *
 * Conventions shared by every entry point.
 *  - Pointers named "device" are HIP device pointers on the current device;
 *    the caller owns every buffer.  The library allocates no device memory
 *    and keeps no global mutable state apart from a thread-local error text
 *    and a per-device cache of the compute-unit count.
 *  - All tensors are dense, contiguous and row-major with the shapes given.
 *    Floating-point pointers must be 16-byte aligned.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the default stream) and never synchronises.  Arguments are
 *    validated on the host before any kernel is launched (the only HIP
 *    calls before that are queries of the current device's compute-unit
 *    count); a kernel fault surfaces at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give the same bits.
 *  - Numerical contract: log_alpha finite and <= 0 with the sum of log_alpha
 *    over any 32 consecutive tokens of a sequence >= -80 per channel (the
 *    chunked prefill evaluates exp(+-that sum) in fp32); beta finite.  The
 *    wide-decay option of kda_prefill_ex halves the window to 16 tokens.
 *    The decode step has no such limit.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 6

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, small workspace */
    KDA_ERR_UNSUPPORTED = 2, /* head dimension or dtype this build does not support */
    KDA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} kda_status;

typedef enum {
    KDA_DTYPE_BF16 = 0, /* q, k, v, o stored as bfloat16 */
    KDA_DTYPE_F32 = 1   /* q, k, v, o stored as float32 */
} kda_dtype;

/*
 * kda_prefill -- chunk-parallel forward pass over a packed batch of
 * variable-length sequences (section 三.2 of the same page: the specialised
 * diagonal-plus-low-rank transition admits chunk-parallel evaluation).
 *
 *   q          device [T_tot, H, d_k]  dtype      queries
 *   k          device [T_tot, H, d_k]  dtype      keys
 *   v          device [T_tot, H, d_v]  dtype      values
 *   log_alpha  device [T_tot, H, d_k]  float32    log of the per-channel decay
 *   beta       device [T_tot, H]       float32    step size
 *   S0         device [N, H, d_k, d_v] float32    initial states; NULL = zero
 *   cu_seqlens device [N + 1]          int32      sequence offsets: cu[0] = 0,
 *              non-decreasing, cu[N] = T_tot.  Its contents are read on the
 *              device only and are not checked (the caller's contract).
 *   N, T_tot, H        >= 1, >= 0, >= 1; T_tot * H * max(d_k, d_v) < 2^31
 *                      and H * max(d_k, d_v) <= 2^20 (32-bit element offsets
 *                      and 32-bit byte ranges of one chunk's rows)
 *   d_k, d_v           each one of 32, 64, 128
 *   dtype              storage type of q, k, v and o
 *   o          device [T_tot, H, d_v]  dtype      outputs (written)
 *   S_T        device [N, H, d_k, d_v] float32    final states (written); may
 *              be the same pointer as S0.  An empty sequence gives S_T = S0.
 *   workspace, workspace_bytes   device scratch of at least
 *              kda_prefill_workspace_size(...) bytes, 256-byte aligned (NULL
 *              allowed when that size is 0).  Owned by the caller; the
 *              library uses it until the work queued on `stream` ends, so
 *              calls that may overlap need separate workspaces.
 *   stream     hipStream_t or NULL
 * q, k, v, log_alpha, beta and o may be NULL when T_tot == 0.  No state
 * crosses a sequence boundary.
 *
 * Long sequences.  When d_k == d_v, T_tot > 1024 and 2 N H is below the
 * current device's compute-unit count (256 on MI355X: N H < 128; too few
 * (sequence, head) pairs to fill the GPU), a sequence longer than its
 * segment length runs as segments (the last one shorter) that are processed
 * in parallel.  A sequence of len tokens has segments of about len / 4
 * tokens, rounded up to a multiple of 512 and kept within [1024, 4096]: a later segment starts from the zero state, an
 * identity run over it (V = 0, S0 = I) gives its transition matrix M and the
 * transformed queries M_t^T q_t, and fix-up passes chain the segments'
 * entering states and add their contribution to the outputs.  The
 * recurrence is linear in (S0, V), so this changes rounding only.  The split
 * of a sequence depends on its own length and on whether the batch runs
 * segmented: a sequence gives the same bits in any batch on the same side
 * of that rule.
 */
kda_status kda_prefill(const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0,
                       const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                       int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_prefill_split -- kda_prefill with an explicit launch shape: the d_v
 * value columns of every (sequence, head) are split over `v_split`
 * workgroups that each run the whole chunk recurrence for d_v / v_split
 * columns (the columns of S evolve independently).  v_split must be 1, 2, 4
 * or 8 with d_v / v_split >= 16.  v_split = 0 selects the same shape as
 * kda_prefill.  Results differ from kda_prefill only by rounding order of
 * no operation: every v_split gives the same bits.
 */
kda_status kda_prefill_split(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const float* S0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                             int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                             void* workspace, size_t workspace_bytes, int32_t v_split,
                             void* stream);

/*
 * kda_prefill_ex -- kda_prefill_split with option flags (0 gives
 * kda_prefill_split exactly):
 *
 *   KDA_PREFILL_SCALAR_GATE  log_alpha is [T_tot, H], one gate per token and
 *                            head (as gdn_prefill_split, below).
 *   KDA_PREFILL_WIDE_DECAY   wide-decay variant.  The numerical contract
 *                            becomes: the sum of log_alpha over any 16
 *                            consecutive tokens >= -80 per channel (twice
 *                            the per-token range of the default 32-token
 *                            window).  A channel whose decay over a 32-token
 *                            chunk is below about -69 takes its exponents
 *                            relative to the chunk's middle row, and the
 *                            state operand of that channel is scaled to
 *                            match; other channels compute exactly as
 *                            without the flag, so inputs within the default
 *                            contract give the same bits either way.  The
 *                            launch costs a few percent more.
 *   KDA_PREFILL_ANY_DECAY    no range contract: any finite log_alpha <= 0,
 *                            including hard resets (a token whose alpha
 *                            underflows to 0 clears the state exactly).
 *                            With a workspace of at least
 *                            kda_prefill_workspace_size_ex(..., flags)
 *                            bytes (256-byte aligned) it runs the chunked
 *                            kernel over chunk lists: a token with
 *                            log_alpha below -5 on some channel starts a
 *                            new chunk (the chunk before it is padded with
 *                            zero rows), which keeps every chunk within the
 *                            wide-decay contract; the workspace holds those
 *                            lists, written by a first kernel on the same
 *                            stream.  The cost grows with the number of such
 *                            tokens (at most one chunk per token).  With a
 *                            smaller (or no) workspace it runs the
 *                            recurrence token by token in fp32 on the
 *                            vector ALU, much slower.  v_split is not used
 *                            (the value split of kda_prefill for whole
 *                            sequences is taken).  Excludes
 *                            KDA_PREFILL_WIDE_DECAY.
 *
 * Unknown flag bits give KDA_ERR_INVALID_ARG.
 */
#define KDA_PREFILL_SCALAR_GATE 1u
#define KDA_PREFILL_WIDE_DECAY 2u
#define KDA_PREFILL_ANY_DECAY 4u
kda_status kda_prefill_ex(const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta, const float* S0,
                          const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                          int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, int32_t v_split,
                          uint32_t flags, void* stream);

/* Bytes of workspace kda_prefill needs for these sizes on the current
 * device: 0 unless the batch runs segmented (d_k == d_v, T_tot > 1024,
 * 2 N H below the device's compute units); then the segment plan, the
 * identity runs' outputs ([T_tot, H, d_k] in dtype) and two fp32 [d_k, d_v]
 * states per (segment, head) for at most
 * N + min(T_tot / 1024, 3 N + T_tot / 4096) segments (integer division).
 * 0 for unsupported sizes.  Where no device can be queried the answer is
 * the one for 256 compute units (MI355X). */
size_t kda_prefill_workspace_size(int32_t N, int64_t T_tot, int32_t H, int32_t d_k,
                                  int32_t d_v, kda_dtype dtype);

/* Bytes of workspace kda_prefill_ex needs for these sizes and flags: with
 * KDA_PREFILL_ANY_DECAY, the chunk lists of its chunked path and one flag
 * byte per token and head: up256(4 N H) + up256(4 H (T_tot + 2 N)) + H T_tot
 * bytes, up256(x) = x rounded up to a multiple of 256; otherwise
 * kda_prefill_workspace_size.  0 for unsupported sizes or invalid flags. */
size_t kda_prefill_workspace_size_ex(int32_t N, int64_t T_tot, int32_t H, int32_t d_k,
                                     int32_t d_v, kda_dtype dtype, uint32_t flags);

/* The v_split kda_prefill would use for these sizes on the current device
 * (1, 2, 4 or 8), or 0 if the sizes are not supported; 256 compute units
 * where no device can be queried. */
int32_t kda_prefill_default_split(int32_t N, int64_t T_tot, int32_t H, int32_t d_k,
                                  int32_t d_v, kda_dtype dtype);

/*
 * kda_prefill_plan -- the launch shape and workspace kda_prefill picks for
 * these sizes on a device with `compute_units` compute units (0: the
 * current device, or 256 where none can be queried).  Writes *v_split
 * (1, 2, 4 or 8) and *workspace_bytes (as kda_prefill_workspace_size).
 * The rules: a batch runs segmented when d_k == d_v, T_tot > 1024 and
 * 2 N H < compute_units; 128 value columns are split over two workgroups
 * when the launch's units (sequences, or at most the segment bound above
 * when segmented) times H times 2 fill at most half of the compute units;
 * otherwise v_split is 1.  KDA_ERR_INVALID_ARG for N < 1, H < 1, T_tot < 0,
 * compute_units < 0 or NULL outputs; KDA_ERR_UNSUPPORTED for unsupported
 * head dimensions or dtypes.  No kernel is launched.
 */
kda_status kda_prefill_plan(int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                            kda_dtype dtype, int32_t compute_units, int32_t* v_split,
                            size_t* workspace_bytes);

/*
 * kda_decode_step -- one token for each of N independent sequences (the same
 * update rule, one step), with the state updated in place.  Each state is
 * read from and written to HBM exactly once.
 *
 *   q, k       device [N, H, d_k]      dtype
 *   v          device [N, H, d_v]      dtype
 *   log_alpha  device [N, H, d_k]      float32
 *   beta       device [N, H]           float32
 *   S          device [N, H, d_k, d_v] float32   read and overwritten
 *   N, H >= 1; d_k, d_v each one of 32, 64, 128
 *   o          device [N, H, d_v]      dtype     written
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* S, int32_t N,
                           int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                           void* stream);

/*
 * Gated DeltaNet: the scalar-gate case of the same recurrence, with one
 * forgetting rate per head instead of one per key channel (the page's
 * section 三.1 contrasts the two):
 *
 *     S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   a_t = exp(log_alpha[t, h])
 *
 * gdn_prefill, gdn_prefill_split and gdn_decode_step take the arguments of
 * kda_prefill, kda_prefill_split and kda_decode_step, with these changes:
 *   - log_alpha is device [T_tot, H] (prefill) or [N, H] (decode), float32,
 *     4-byte aligned;
 *   - the numerical contract applies to the per-head decay;
 *   - the workspace is sized by kda_prefill_workspace_size, and the launch
 *     shape by kda_prefill_default_split.
 * Results are bit-identical to the kda_* calls with log_alpha repeated over
 * the d_k channels.
 */
kda_status gdn_prefill(const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0,
                       const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                       int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

kda_status gdn_prefill_split(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const float* S0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                             int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                             void* workspace, size_t workspace_bytes, int32_t v_split,
                             void* stream);

kda_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* S, int32_t N,
                           int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, void* o,
                           void* stream);

/*
 * kda_prefill_backward -- gradients of a scalar loss L through kda_prefill:
 * given dL/do for every token and dL/dS_T for every final state, it returns
 * dL/d of q, k, v, log_alpha, beta and the initial state.  It is the
 * reverse-mode derivative of the recurrence of "Kimi Linear：让长上下文大模型
 * 真正实用的线性注意力架构" (juejin.cn), section 三.5, per channel (section 三.1),
 * with the read-out o_t = S_t^T q_t after the update.  The training side of
 * the page's reading of the layer as online learning needs it.
 *
 * It runs chunked, on MFMA: the forward pass once more, storing the state
 * entering every chunk and W0 = V - K~ S (in the storage type) in the
 * workspace, then a walk over each sequence's chunks from the last that
 * carries dL/dS in fp32 and forms every product of the chunk's adjoint as a
 * matrix product.  Its numerical contract is kda_prefill's (log_alpha summed
 * over any 32 consecutive tokens >= -80 per channel); kda_prefill_backward_ex
 * with KDA_PREFILL_ANY_DECAY has none.
 *
 * Inputs are those of kda_prefill (same layouts, dtype, alignment and sizes):
 *   q, k, v, log_alpha, beta, S0 (NULL: zero), cu_seqlens, N, T_tot, H, d_k,
 *   d_v, dtype
 *   d_o        device [T_tot, H, d_v]     dtype     dL/do
 *   d_S_T      device [N, H, d_k, d_v]    float32   dL/dS_T; NULL: zero
 * Outputs, all float32, written in full (overwritten, not accumulated):
 *   d_q, d_k   device [T_tot, H, d_k]
 *   d_v        device [T_tot, H, d_v]
 *   d_log_alpha device [T_tot, H, d_k]
 *   d_beta     device [T_tot, H]           4-byte aligned
 *   d_S0       device [N, H, d_k, d_v]     also when S0 is NULL
 *   workspace  device, at least kda_prefill_backward_workspace_size(...)
 *              bytes, 256-byte aligned, owned by the caller; its contents on
 *              entry do not matter and are clobbered.
 * Outputs must not alias inputs or one another.  Errors as for kda_prefill
 * (validation before any kernel is launched).  Asynchronous on `stream`.
 * Results are identical from run to run.
 */
kda_status kda_prefill_backward(const void* q, const void* k, const void* v,
                                const float* log_alpha, const float* beta, const float* S0,
                                const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                                int32_t d_k, int32_t d_v, kda_dtype dtype, const void* d_o,
                                const float* d_S_T, float* d_q, float* d_k_out, float* d_v_out,
                                float* d_log_alpha, float* d_beta, float* d_S0, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kda_prefill_backward_ex -- kda_prefill_backward with option flags (0 gives
 * kda_prefill_backward exactly):
 *   KDA_PREFILL_SCALAR_GATE  one gate per token and head (as
 *                            gdn_prefill_backward: log_alpha and d_log_alpha
 *                            are [T_tot, H]).
 *   KDA_PREFILL_ANY_DECAY    the token-recurrent backward: fp32 on the vector
 *                            ALU, no range contract (any finite log_alpha
 *                            <= 0, including hard resets), much slower; its
 *                            workspace holds fp32 states every 16 tokens and
 *                            one fp32 row of d_v per token and head.
 * Other bits give KDA_ERR_INVALID_ARG.  The workspace is sized by
 * kda_prefill_backward_workspace_size_ex with the same flags.
 */
kda_status kda_prefill_backward_ex(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* S0,
                                   const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                                   int32_t d_k, int32_t d_v, kda_dtype dtype, const void* d_o,
                                   const float* d_S_T, float* d_q, float* d_k_out, float* d_v_out,
                                   float* d_log_alpha, float* d_beta, float* d_S0, void* workspace,
                                   size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * gdn_prefill_backward -- the backward pass of gdn_prefill (one gate per token
 * and head).  Arguments as for kda_prefill_backward, except that log_alpha
 * and d_log_alpha are device [T_tot, H] float32, 4-byte aligned;
 * d_log_alpha[t, h] is the gradient with respect to the one gate, i.e. the
 * sum over the key channels of the per-channel gradient.  The other
 * gradients are bit-identical to kda_prefill_backward's with log_alpha
 * repeated over the d_k channels.  Workspace as for kda_prefill_backward.
 */
kda_status gdn_prefill_backward(const void* q, const void* k, const void* v,
                                const float* log_alpha, const float* beta, const float* S0,
                                const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                                int32_t d_k, int32_t d_v, kda_dtype dtype, const void* d_o,
                                const float* d_S_T, float* d_q, float* d_k_out, float* d_v_out,
                                float* d_log_alpha, float* d_beta, float* d_S0, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace bytes kda_prefill_backward needs: the state entering every chunk
 * (d_k x d_v) and W0 of every chunk (C x d_v), in the storage type, for at
 * most T_tot / C + N + 1 chunks per head, C the prefill's chunk length (32
 * tokens; 16 for float32 with d_k >= 64).  0 for unsupported sizes. */
size_t kda_prefill_backward_workspace_size(int32_t N, int64_t T_tot, int32_t H, int32_t d_k,
                                           int32_t d_v, kda_dtype dtype);

/* Workspace bytes kda_prefill_backward_ex needs with these flags: as above,
 * or with KDA_PREFILL_ANY_DECAY fp32 states at the start of every 16-token
 * block (at most T_tot / 16 + N + 1 blocks per head) and one fp32 row of d_v
 * per token and head. */
size_t kda_prefill_backward_workspace_size_ex(int32_t N, int64_t T_tot, int32_t H, int32_t d_k,
                                              int32_t d_v, kda_dtype dtype, uint32_t flags);

/*
 * kda_prefill_noalloc -- kda_prefill for callers that cannot allocate device
 * memory: code under HIP stream capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments as kda_prefill without the workspace; results
 * are bit-identical to kda_prefill's.  The segmented path's workspace comes
 * from a fixed device array of KDA_PREFILL_NOALLOC_WORKSPACE_BYTES bytes
 * that the library holds on each device it runs on until the process ends
 * (its address is looked up on the first call made with that device
 * current).  This call allocates nothing.
 *
 * Limit: sizes whose kda_prefill_workspace_size exceeds the fixed workspace
 * (for example one 128k-token sequence at H = 32, d = 128) return
 * KDA_ERR_INVALID_ARG before any launch; a batch that runs in one pass
 * needs no workspace and has no such limit.  The 4096-token sequence at
 * H = 32, d = 128, bf16 needs about 52 MiB and fits.
 *
 * Every call on one device shares that device's array, which keeps the
 * last call's contents (each call writes every part it reads before
 * reading it).  Calls that overlap on one device (on different streams, or
 * from different threads without ordering) race on it: order them.
 */
#define KDA_PREFILL_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* S0,
                               const int32_t* cu_seqlens, int32_t N, int64_t T_tot, int32_t H,
                               int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, float* S_T,
                               void* stream);

/* Static text for a status code. */
const char* kda_status_string(kda_status status);

/* Detail of the last failed call on the calling thread ("" if none). */
const char* kda_last_error(void);

/* KDA_VERSION of the library. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
