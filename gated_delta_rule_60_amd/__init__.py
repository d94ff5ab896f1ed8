"""MI355X-native (gfx950) Kimi Delta Attention forward pass.

The KDA recurrence S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
+ beta_t k_t v_t^T with read-out o_t = S_t^T q_t ("Kimi Linear：让长上下文大模型
真正实用的线性注意力架构", section 三.5; per-channel alpha, section 三.1), as a
chunk-parallel prefill and an in-place decode step (and the scalar-gate
Gated DeltaNet case of the same recurrence), in hand-written HIP
kernels behind the C ABI of include/kda.h (libkda.so).

``import gated_delta_rule_60_amd`` does not load the library; the first call
does, and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    KDA_DTYPE_BF16,
    KDA_DTYPE_F32,
    KDA_ERR_HIP,
    KDA_ERR_INVALID_ARG,
    KDA_ERR_UNSUPPORTED,
    KDA_OK,
    KDA_PREFILL_ANY_DECAY,
    KDA_PREFILL_SCALAR_GATE,
    KDA_PREFILL_WIDE_DECAY,
    KDAError,
    decode_step,
    gdn_decode_step,
    gdn_decode_step_t,
    gdn_prefill_backward,
    gdn_prefill_backward_t,
    gdn_prefill,
    gdn_prefill_split,
    gdn_prefill_t,
    kda_decode_step,
    kda_last_error,
    kda_prefill,
    kda_prefill_backward,
    kda_prefill_backward_ex,
    kda_prefill_backward_workspace_size,
    kda_prefill_backward_workspace_size_ex,
    kda_prefill_default_split,
    kda_prefill_ex,
    kda_prefill_plan,
    kda_prefill_split,
    kda_prefill_workspace_size,
    kda_prefill_workspace_size_ex,
    kda_status_string,
    kda_version,
    library_path,
    load,
    prefill,
    prefill_backward,
    prefill_plan,
)

__version__ = "0.1.0"
