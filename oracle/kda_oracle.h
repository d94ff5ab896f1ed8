/*
 * kda_oracle.h -- plain fp64 CPU reference of the Kimi Delta Attention (KDA)
 * forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the GPU library and must never be used to produce a product result.
 *
 * Source of the computation: the KDA update rule printed in
 * "Kimi Linear：让长上下文大模型真正实用的线性注意力架构" (juejin.cn), section
 * 三.5 ("Attention as Learning"):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * with alpha_t one retention factor per key channel (same page, section 三.1)
 * and beta_t a scalar step size per token and head.  The read-out
 * o_t = S_t^T q_t (taken after the update) is not printed on the pages; it is
 * the numerator of the kernelised linear-attention form Q (K^T V) on the
 * xdnf.cn page, section 2.2, applied to the gated state.
 *
 * Inputs are float32 arrays holding the exact device input values (bf16
 * inputs widened exactly); all arithmetic is fp64.  Every pointer is a host
 * pointer.  Layouts (row-major, contiguous):
 *   q, k       [T_tot, H, d_k]      v          [T_tot, H, d_v]
 *   log_alpha  [T_tot, H, d_k]      beta       [T_tot, H]
 *   S0, S_T    [N, H, d_k, d_v]     o          [T_tot, H, d_v]
 *   cu_seqlens [N + 1], cu[0] = 0, non-decreasing, cu[N] = T_tot
 * S0 may be NULL (zero initial state).  S_T may alias S0.  pair_mask, when
 * not NULL, is [N, H] bytes: only pairs with a non-zero byte are computed
 * and written.  nthreads <= 0 means one thread.
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int kda_oracle_prefill(const float* q, const float* k, const float* v,
                       const float* log_alpha, const float* beta,
                       const double* S0, const int32_t* cu_seqlens,
                       int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                       const uint8_t* pair_mask, double* o, double* S_T, int32_t nthreads);

/* One decode step: one token per sequence, S [N, H, d_k, d_v] fp64 updated in
 * place, o [N, H, d_v].  Inputs are [N, H, .] as in the prefill with T_tot = N. */
int kda_oracle_decode_step(const float* q, const float* k, const float* v,
                           const float* log_alpha, const float* beta, double* S,
                           int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                           const uint8_t* pair_mask, double* o, int32_t nthreads);

/* Backward pass of kda_oracle_prefill: gradients of a scalar loss given
 * dO = dL/do [T_tot, H, d_v] and dS_T = dL/dS_T [N, H, d_k, d_v] (NULL: zero).
 * Outputs (fp64, same layouts as the matching inputs): dq, dk [T_tot, H, d_k],
 * dv [T_tot, H, d_v], dlog_alpha [T_tot, H, d_k], dbeta [T_tot, H], and
 * dS0 [N, H, d_k, d_v], the gradient with respect to the initial state (also
 * when S0 is NULL, i.e. zero).  Reverse-mode differentiation of the token
 * recurrence, token by token from the last; see kda_oracle.c. */
int kda_oracle_prefill_backward(const float* q, const float* k, const float* v,
                                const float* log_alpha, const float* beta,
                                const double* S0, const int32_t* cu_seqlens,
                                int32_t N, int64_t T_tot, int32_t H, int32_t d_k, int32_t d_v,
                                const double* dO, const double* dS_T, const uint8_t* pair_mask,
                                double* dq, double* dk, double* dv, double* dlog_alpha,
                                double* dbeta, double* dS0, int32_t nthreads);

#ifdef __cplusplus
}
#endif

#endif /* KDA_ORACLE_H */
