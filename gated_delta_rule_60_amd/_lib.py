"""ctypes binding of libkda.so (include/kda.h).

The functions named ``kda_*`` mirror the C ABI one to one and take raw
device pointers (ints) and a stream handle.  ``prefill`` and ``decode_step``
are argument-marshalling conveniences over torch tensors: they check shapes
and dtypes, allocate outputs with torch when none are given, and call the C
ABI on the given stream (torch's current stream by default), allocating
every temporary under that stream.  Every arithmetic step runs in the library's
HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_HIP = 3
KDA_DTYPE_BF16 = 0
KDA_DTYPE_F32 = 1
KDA_PREFILL_SCALAR_GATE = 1
KDA_PREFILL_WIDE_DECAY = 2
KDA_PREFILL_ANY_DECAY = 4
KDA_PREFILL_NOALLOC_WORKSPACE_BYTES = 64 << 20  # include/kda.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# (name, restype, argtypes) for every symbol declared in include/kda.h
_vp, _fp, _ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "kda_prefill": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32, _i32,
                                   ctypes.c_int, _vp, _fp, _vp, _sz, _vp]),
    "kda_prefill_split": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32,
                                         _i32, ctypes.c_int, _vp, _fp, _vp, _sz, _i32, _vp]),
    "kda_prefill_ex": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32, _i32,
                                      ctypes.c_int, _vp, _fp, _vp, _sz, _i32, ctypes.c_uint32, _vp]),
    "kda_prefill_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int]),
    "kda_prefill_workspace_size_ex": (_sz, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int, ctypes.c_uint32]),
    "kda_prefill_default_split": (_i32, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int]),
    "kda_prefill_plan": (ctypes.c_int, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int, _i32, _vp, _vp]),
    "kda_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _i32, _i32, _i32, _i32,
                                       ctypes.c_int, _vp, _vp]),
    "gdn_prefill": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32, _i32,
                                   ctypes.c_int, _vp, _fp, _vp, _sz, _vp]),
    "gdn_prefill_split": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32,
                                         _i32, ctypes.c_int, _vp, _fp, _vp, _sz, _i32, _vp]),
    "gdn_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _i32, _i32, _i32, _i32,
                                       ctypes.c_int, _vp, _vp]),
    "kda_prefill_backward": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32,
                                            _i32, ctypes.c_int, _vp, _fp, _fp, _fp, _fp, _fp, _fp, _fp,
                                            _vp, _sz, _vp]),
    "kda_prefill_backward_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int]),
    "kda_prefill_backward_ex": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32,
                                               _i32, ctypes.c_int, _vp, _fp, _fp, _fp, _fp, _fp, _fp, _fp,
                                               _vp, _sz, ctypes.c_uint32, _vp]),
    "kda_prefill_backward_workspace_size_ex": (_sz, [_i32, _i64, _i32, _i32, _i32, ctypes.c_int,
                                                     ctypes.c_uint32]),
    "gdn_prefill_backward": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32,
                                            _i32, ctypes.c_int, _vp, _fp, _fp, _fp, _fp, _fp, _fp, _fp,
                                            _vp, _sz, _vp]),
    "kda_prefill_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _fp, _fp, _fp, _ip, _i32, _i64, _i32, _i32, _i32,
                                           ctypes.c_int, _vp, _fp, _vp]),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_version": (_i32, []),
}


class KDAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{kda_status_string(status)}: {detail}")


def library_path() -> str:
    return os.path.join(_HERE, "libkda.so")


def load() -> ctypes.CDLL:
    """Open libkda.so; raise if it has not been built (no fallback exists)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_60_amd.build` "
                           "(the KDA forward pass has no other implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


# ---------------------------------------------------------------------------
# C ABI, one to one
# ---------------------------------------------------------------------------
def kda_prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                workspace, workspace_bytes, stream) -> int:
    return load().kda_prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype,
                              o, S_T, workspace, workspace_bytes, stream)


def kda_prefill_split(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                      workspace, workspace_bytes, v_split, stream) -> int:
    return load().kda_prefill_split(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                    dtype, o, S_T, workspace, workspace_bytes, v_split, stream)


def kda_prefill_ex(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                   workspace, workspace_bytes, v_split, flags, stream) -> int:
    return load().kda_prefill_ex(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                 dtype, o, S_T, workspace, workspace_bytes, v_split, flags, stream)


def kda_prefill_workspace_size(N, T_tot, H, d_k, d_v, dtype) -> int:
    return int(load().kda_prefill_workspace_size(N, T_tot, H, d_k, d_v, dtype))


def kda_prefill_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, flags) -> int:
    return int(load().kda_prefill_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, flags))


def kda_prefill_default_split(N, T_tot, H, d_k, d_v, dtype) -> int:
    return int(load().kda_prefill_default_split(N, T_tot, H, d_k, d_v, dtype))


def kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, compute_units, v_split, workspace_bytes) -> int:
    return load().kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, compute_units, v_split, workspace_bytes)


def prefill_plan(N, T_tot, H, d_k, d_v, dtype, compute_units: int = 0):
    """(v_split, workspace bytes) kda_prefill picks on a device with
    ``compute_units`` compute units (0: the current device)."""
    v, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    _check(kda_prefill_plan(N, T_tot, H, d_k, d_v, dtype, compute_units, ctypes.byref(v), ctypes.byref(ws)))
    return int(v.value), int(ws.value)


def kda_decode_step(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream) -> int:
    return load().kda_decode_step(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream)


def gdn_prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                workspace, workspace_bytes, stream) -> int:
    return load().gdn_prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype,
                              o, S_T, workspace, workspace_bytes, stream)


def gdn_prefill_split(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                      workspace, workspace_bytes, v_split, stream) -> int:
    return load().gdn_prefill_split(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                    dtype, o, S_T, workspace, workspace_bytes, v_split, stream)


def gdn_decode_step(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream) -> int:
    return load().gdn_decode_step(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, o, stream)


def kda_prefill_noalloc(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, o, S_T,
                        stream) -> int:
    return load().kda_prefill_noalloc(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype,
                                      o, S_T, stream)


def kda_status_string(status: int) -> str:
    return load().kda_status_string(status).decode()


def kda_last_error() -> str:
    return load().kda_last_error().decode()


def kda_version() -> int:
    return int(load().kda_version())


def kda_prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o,
                         d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace,
                         workspace_bytes, stream) -> int:
    return load().kda_prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                       dtype, d_o, d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta,
                                       d_S0, workspace, workspace_bytes, stream)


def gdn_prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o,
                         d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace,
                         workspace_bytes, stream) -> int:
    return load().gdn_prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                       dtype, d_o, d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta,
                                       d_S0, workspace, workspace_bytes, stream)


def kda_prefill_backward_workspace_size(N, T_tot, H, d_k, d_v, dtype) -> int:
    return int(load().kda_prefill_backward_workspace_size(N, T_tot, H, d_k, d_v, dtype))


def kda_prefill_backward_ex(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v, dtype, d_o,
                            d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta, d_S0, workspace,
                            workspace_bytes, flags, stream) -> int:
    return load().kda_prefill_backward_ex(q, k, v, log_alpha, beta, S0, cu_seqlens, N, T_tot, H, d_k, d_v,
                                          dtype, d_o, d_S_T, d_q, d_k_out, d_v_out, d_log_alpha, d_beta,
                                          d_S0, workspace, workspace_bytes, flags, stream)


def kda_prefill_backward_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, flags) -> int:
    return int(load().kda_prefill_backward_workspace_size_ex(N, T_tot, H, d_k, d_v, dtype, flags))


def _check(status: int) -> None:
    if status != KDA_OK:
        raise KDAError(status, kda_last_error())


# ---------------------------------------------------------------------------
# torch conveniences (marshalling only)
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_of(stream, device):
    """The torch stream a call runs on: ``stream``, or the device's current one.

    The wrappers allocate every temporary (default ``cu_seqlens``, outputs,
    workspaces) under ``torch.cuda.stream`` of this stream, so the caching
    allocator ties those blocks to the stream the kernels run on and does
    not hand them to other work while the kernels may still use them."""
    import torch
    return stream if stream is not None else torch.cuda.current_stream(device)


def _prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, v_split, workspace, stream,
             scalar_gate: bool, wide_decay: bool = False, any_decay: bool = False,
             token_recurrent: bool = False):
    """Chunked prefill on torch tensors; returns (o, S_T).

    q, k: [T, H, d_k]; v: [T, H, d_v] (bf16 or fp32, same dtype);
    log_alpha: [T, H, d_k] fp32 ([T, H] with ``scalar_gate``); beta: [T, H]
    fp32; S0: [N, H, d_k, d_v] fp32
    or None; cu_seqlens: int32 [N + 1] on the device (None = one sequence).
    ``S_T`` may be ``S0`` itself (in-place update of the states).
    ``workspace`` (optional): a uint8 device tensor of at least
    ``kda_prefill_workspace_size_ex(...)`` bytes for these flags; one is
    allocated when needed and not given.  ``wide_decay`` selects the
    wide-decay kernel variant (KDA_PREFILL_WIDE_DECAY); ``any_decay`` drops
    the decay-range contract (KDA_PREFILL_ANY_DECAY): the chunked kernel over
    chunk lists, or with ``token_recurrent`` the token-recurrent kernel (no
    workspace).
    """
    import torch
    if not q.is_cuda:
        raise ValueError("kda prefill runs on a GPU device; q is on the CPU")
    dev = q.device
    st = _stream_of(stream, dev)
    with torch.cuda.device(dev), torch.cuda.stream(st):
        return _prefill_on(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, v_split, workspace, st,
                           scalar_gate, wide_decay, any_decay, token_recurrent)


def _prefill_on(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, v_split, workspace, st,
                scalar_gate, wide_decay, any_decay, token_recurrent):
    import torch
    dev = q.device
    T, H, dk = (int(x) for x in q.shape)
    dv = int(v.shape[-1])
    code = _dtype_code(q)
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = int(cu_seqlens.shape[0]) - 1
    _need(q, "q", (T, H, dk), q.dtype, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (T, H) if scalar_gate else (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _need(o, "o", (T, H, dv), q.dtype, dev)
    _need(S_T, "S_T", (N, H, dk, dv), torch.float32, dev)
    flags = ((KDA_PREFILL_SCALAR_GATE if scalar_gate else 0) | (KDA_PREFILL_WIDE_DECAY if wide_decay else 0)
             | (KDA_PREFILL_ANY_DECAY if any_decay else 0))
    if token_recurrent and not any_decay:
        raise ValueError("token_recurrent applies to any_decay")
    ws = 0 if token_recurrent else kda_prefill_workspace_size_ex(N, T, H, dk, dv, code, flags)
    wbuf = None
    if ws:
        if workspace is None:
            wbuf = torch.empty(ws, dtype=torch.uint8, device=dev)
        else:
            if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
            if workspace.numel() < ws:
                raise ValueError(f"workspace holds {workspace.numel()} bytes; {ws} are needed")
            wbuf = workspace
    _check(kda_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(),
                          beta.data_ptr(), S0.data_ptr() if S0 is not None else None,
                          cu_seqlens.data_ptr(), N, T, H, dk, dv, code, o.data_ptr(),
                          S_T.data_ptr(), wbuf.data_ptr() if wbuf is not None else None, ws,
                          int(v_split), flags, int(st.cuda_stream)))
    return o, S_T


def prefill(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, o=None, S_T=None,
            v_split: int = 0, workspace=None, wide_decay: bool = False, any_decay: bool = False,
            token_recurrent: bool = False, stream=None):
    """KDA chunked prefill (per-channel gates, log_alpha [T, H, d_k]) on torch
    tensors; returns (o, S_T).  Arguments as in ``_prefill``."""
    return _prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, v_split, workspace, stream, False,
                    wide_decay, any_decay, token_recurrent)


def gdn_prefill_t(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *, o=None, S_T=None,
                  v_split: int = 0, workspace=None, wide_decay: bool = False, any_decay: bool = False,
                  token_recurrent: bool = False, stream=None):
    """Gated DeltaNet chunked prefill (one gate per token and head, log_alpha
    [T, H]) on torch tensors; returns (o, S_T).  Arguments as in ``_prefill``."""
    return _prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, v_split, workspace, stream, True,
                    wide_decay, any_decay, token_recurrent)



def _decode(q, k, v, log_alpha, beta, S, o, stream, scalar_gate: bool):
    """One decode step; S [N, H, d_k, d_v] fp32 is updated in place.
    Returns o [N, H, d_v] in q's dtype."""
    import torch
    if not q.is_cuda:
        raise ValueError("kda decode runs on a GPU device; q is on the CPU")
    dev = q.device
    st = _stream_of(stream, dev)
    with torch.cuda.device(dev), torch.cuda.stream(st):
        return _decode_on(q, k, v, log_alpha, beta, S, o, st, scalar_gate)


def _decode_on(q, k, v, log_alpha, beta, S, o, st, scalar_gate):
    import torch
    dev = q.device
    N, H, dk = (int(x) for x in q.shape)
    dv = int(v.shape[-1])
    code = _dtype_code(q)
    _need(q, "q", (N, H, dk), q.dtype, dev)
    _need(k, "k", (N, H, dk), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (N, H) if scalar_gate else (N, H, dk), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    _need(S, "S", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", (N, H, dv), q.dtype, dev)
    call = gdn_decode_step if scalar_gate else kda_decode_step
    _check(call(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(), beta.data_ptr(),
                S.data_ptr(), N, H, dk, dv, code, o.data_ptr(), int(st.cuda_stream)))
    return o


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, stream=None):
    """One KDA decode step (log_alpha [N, H, d_k]); S [N, H, d_k, d_v] fp32 is
    updated in place.  Returns o [N, H, d_v] in q's dtype."""
    return _decode(q, k, v, log_alpha, beta, S, o, stream, False)


def gdn_decode_step_t(q, k, v, log_alpha, beta, S, *, o=None, stream=None):
    """One Gated DeltaNet decode step (log_alpha [N, H]); S is updated in
    place.  Returns o [N, H, d_v] in q's dtype."""
    return _decode(q, k, v, log_alpha, beta, S, o, stream, True)


def prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T=None, *, workspace=None,
                     any_decay: bool = False, stream=None):
    """Backward of ``prefill`` on torch tensors: gradients of a loss given
    d_o = dL/do ([T, H, d_v], dtype of q) and d_S_T = dL/dS_T ([N, H, d_k,
    d_v] fp32, or None).  Returns fp32 (d_q, d_k, d_v, d_log_alpha, d_beta,
    d_S0) shaped like q, k, v, log_alpha, beta and the initial state.
    ``workspace``: optional uint8 device tensor of at least
    ``kda_prefill_backward_workspace_size_ex(...)`` bytes (allocated if None).
    ``any_decay`` selects the token-recurrent backward (KDA_PREFILL_ANY_DECAY),
    which has no decay-range contract."""
    return _backward(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, workspace, stream, False, any_decay)


def gdn_prefill_backward_t(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T=None, *, workspace=None,
                           any_decay: bool = False, stream=None):
    """Backward of ``gdn_prefill_t`` (log_alpha [T, H]); d_log_alpha is [T, H].
    Arguments and results otherwise as in ``prefill_backward``."""
    return _backward(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, workspace, stream, True, any_decay)


def _backward(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, workspace, stream, scalar_gate: bool,
              any_decay: bool = False):
    import torch
    if not q.is_cuda:
        raise ValueError("kda prefill backward runs on a GPU device; q is on the CPU")
    dev = q.device
    st = _stream_of(stream, dev)
    with torch.cuda.device(dev), torch.cuda.stream(st):
        return _backward_on(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, workspace, st, scalar_gate,
                            any_decay)


def _backward_on(q, k, v, log_alpha, beta, S0, cu_seqlens, d_o, d_S_T, workspace, st, scalar_gate, any_decay):
    import torch
    dev = q.device
    T, H, dk = (int(x) for x in q.shape)
    dv = int(v.shape[-1])
    code = _dtype_code(q)
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = int(cu_seqlens.shape[0]) - 1
    _need(q, "q", (T, H, dk), q.dtype, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    _need(log_alpha, "log_alpha", (T, H) if scalar_gate else (T, H, dk), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _need(d_o, "d_o", (T, H, dv), q.dtype, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if d_S_T is not None:
        _need(d_S_T, "d_S_T", (N, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gq, gk, gv = torch.empty((T, H, dk), **f32), torch.empty((T, H, dk), **f32), torch.empty((T, H, dv), **f32)
    gla = torch.empty((T, H) if scalar_gate else (T, H, dk), **f32)
    gb, gS0 = torch.empty((T, H), **f32), torch.empty((N, H, dk, dv), **f32)
    flags = (KDA_PREFILL_SCALAR_GATE if scalar_gate else 0) | (KDA_PREFILL_ANY_DECAY if any_decay else 0)
    ws = kda_prefill_backward_workspace_size_ex(N, T, H, dk, dv, code, flags)
    if workspace is None:
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    ptr = lambda t: t.data_ptr() if t is not None else None
    _check(kda_prefill_backward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(), beta.data_ptr(),
                                   ptr(S0), cu_seqlens.data_ptr(), N, T, H, dk, dv, code, d_o.data_ptr(),
                                   ptr(d_S_T), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(), gla.data_ptr(),
                                   gb.data_ptr(), gS0.data_ptr(), workspace.data_ptr(), workspace.numel(), flags,
                                   int(st.cuda_stream)))
    return gq, gk, gv, gla, gb, gS0
