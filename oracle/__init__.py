"""fp64 CPU oracle of the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and
it shares no code with the GPU library: it is a plain token-by-token fp64
recurrence in C (``kda_oracle.c``) behind ctypes.

What it computes is the KDA update rule of
"Kimi Linear：让长上下文大模型真正实用的线性注意力架构" (juejin.cn), section 三.5,
with per-channel gates (section 三.1) and the read-out o_t = S_t^T q_t after
the update.  Every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, special cases, brute-force
expansion on tiny inputs and invariants), not by re-typing its formula.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import build_oracle, library_path

__all__ = ["prefill", "decode_step", "gdn_prefill", "gdn_decode_step", "prefill_backward",
           "gdn_prefill_backward", "build_oracle", "library_path", "load", "bind"]

_LIB = None


def load() -> ctypes.CDLL:
    """Load the oracle library, building it with gcc only if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        build_oracle()
    _LIB = bind(path)
    return _LIB


def bind(path: str) -> ctypes.CDLL:
    """Open an oracle build at ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i32p,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, u8p, f64p, f64p,
                                       ctypes.c_int32]
    lib.kda_oracle_decode_step.restype = ctypes.c_int
    lib.kda_oracle_decode_step.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, u8p, f64p, ctypes.c_int32]
    if hasattr(lib, "kda_oracle_prefill_backward"):
        lib.kda_oracle_prefill_backward.restype = ctypes.c_int
        lib.kda_oracle_prefill_backward.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i32p,
                                                    ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32, f64p, f64p, u8p,
                                                    f64p, f64p, f64p, f64p, f64p, f64p,
                                                    ctypes.c_int32]
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(x, shape):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, log_alpha, beta, S0: Optional[np.ndarray], cu_seqlens,
            pair_mask: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
            lib: Optional[ctypes.CDLL] = None):
    """Run the recurrence over a packed varlen batch.

    q, k: [T, H, d_k]; v: [T, H, d_v]; log_alpha: [T, H, d_k]; beta: [T, H];
    S0: [N, H, d_k, d_v] or None; cu_seqlens: [N + 1].
    Returns (o [T, H, d_v] float64, S_T [N, H, d_k, d_v] float64).  Entries of
    pairs excluded by ``pair_mask`` ([N, H] bool) are NaN.  ``lib`` selects
    another build of the oracle (default: the one next to this file).
    """
    lib = lib or load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = int(cu.shape[0] - 1)
    T = int(cu[-1])
    q = np.asarray(q)
    H, dk = int(q.shape[1]), int(q.shape[2])
    dv = int(np.asarray(v).shape[2])
    q = _f32(q, (T, H, dk))
    k = _f32(k, (T, H, dk))
    v = _f32(v, (T, H, dv))
    la = _f32(log_alpha, (T, H, dk))
    b = _f32(beta, (T, H))
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        if s0.shape != (N, H, dk, dv):
            raise ValueError(f"S0 shape {s0.shape} != {(N, H, dk, dv)}")
    mask = None
    if pair_mask is not None:
        mask = np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(N, H))
    o = np.full((T, H, dv), np.nan, dtype=np.float64)
    ST = np.full((N, H, dk, dv), np.nan, dtype=np.float64)
    rc = lib.kda_oracle_prefill(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                _ptr(v, ctypes.c_float), _ptr(la, ctypes.c_float),
                                _ptr(b, ctypes.c_float), _ptr(s0, ctypes.c_double),
                                _ptr(cu, ctypes.c_int32), N, T, H, dk, dv,
                                _ptr(mask, ctypes.c_uint8), _ptr(o, ctypes.c_double),
                                _ptr(ST, ctypes.c_double),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill failed with status {rc}")
    return o, ST


def decode_step(q, k, v, log_alpha, beta, S: np.ndarray,
                pair_mask: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
                lib: Optional[ctypes.CDLL] = None):
    """One decode step.  S ([N, H, d_k, d_v] float64, C-contiguous) is updated
    in place; returns o [N, H, d_v] float64."""
    lib = lib or load()
    if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous):
        raise ValueError("S must be a C-contiguous float64 numpy array (updated in place)")
    N, H, dk, dv = (int(x) for x in S.shape)
    q = _f32(q, (N, H, dk))
    k = _f32(k, (N, H, dk))
    v = _f32(v, (N, H, dv))
    la = _f32(log_alpha, (N, H, dk))
    b = _f32(beta, (N, H))
    mask = None
    if pair_mask is not None:
        mask = np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(N, H))
    o = np.full((N, H, dv), np.nan, dtype=np.float64)
    rc = lib.kda_oracle_decode_step(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                    _ptr(v, ctypes.c_float), _ptr(la, ctypes.c_float),
                                    _ptr(b, ctypes.c_float), _ptr(S, ctypes.c_double),
                                    N, H, dk, dv, _ptr(mask, ctypes.c_uint8),
                                    _ptr(o, ctypes.c_double), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_step failed with status {rc}")
    return o


def gdn_prefill(q, k, v, log_alpha, beta, S0, cu_seqlens, **kw):
    """Gated DeltaNet: one forgetting rate per head and token (log_alpha
    [T, H]) instead of one per key channel, the contrast drawn in section 三.1
    of the same page.  It is the recurrence above with alpha_t[i] = a_t for
    every channel i, so the same fp64 loop runs on log_alpha repeated over
    the d_k channels."""
    q = np.asarray(q)
    la = np.asarray(log_alpha, dtype=np.float32)
    la = np.ascontiguousarray(np.broadcast_to(la[:, :, None], la.shape + (q.shape[2],)))
    return prefill(q, k, v, la, beta, S0, cu_seqlens, **kw)


def gdn_decode_step(q, k, v, log_alpha, beta, S: np.ndarray, **kw):
    """One Gated DeltaNet decode step (log_alpha [N, H]); S is updated in
    place, as in ``decode_step``."""
    q = np.asarray(q)
    la = np.asarray(log_alpha, dtype=np.float32)
    la = np.ascontiguousarray(np.broadcast_to(la[:, :, None], la.shape + (q.shape[2],)))
    return decode_step(q, k, v, la, beta, S, **kw)


def prefill_backward(q, k, v, log_alpha, beta, S0: Optional[np.ndarray], cu_seqlens, dO,
                     dS_T: Optional[np.ndarray] = None, pair_mask: Optional[np.ndarray] = None,
                     nthreads: Optional[int] = None, lib: Optional[ctypes.CDLL] = None):
    """Gradients of a scalar loss through ``prefill``, given dO = dL/do
    ([T, H, d_v]) and dS_T = dL/dS_T ([N, H, d_k, d_v], None: zero).

    Returns (dq, dk, dv, dlog_alpha, dbeta, dS0) as float64 arrays shaped like
    q, k, v, log_alpha, beta and the initial state.  Reverse-mode
    differentiation of the same token recurrence, last token first."""
    lib = lib or load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = int(cu.shape[0] - 1)
    T = int(cu[-1])
    q = np.asarray(q)
    H, dk = int(q.shape[1]), int(q.shape[2])
    dv = int(np.asarray(v).shape[2])
    q = _f32(q, (T, H, dk))
    k = _f32(k, (T, H, dk))
    v = _f32(v, (T, H, dv))
    la = _f32(log_alpha, (T, H, dk))
    b = _f32(beta, (T, H))
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        if s0.shape != (N, H, dk, dv):
            raise ValueError(f"S0 shape {s0.shape} != {(N, H, dk, dv)}")
    do = np.ascontiguousarray(np.asarray(dO, dtype=np.float64))
    if do.shape != (T, H, dv):
        raise ValueError(f"dO shape {do.shape} != {(T, H, dv)}")
    dst = None
    if dS_T is not None:
        dst = np.ascontiguousarray(np.asarray(dS_T, dtype=np.float64))
        if dst.shape != (N, H, dk, dv):
            raise ValueError(f"dS_T shape {dst.shape} != {(N, H, dk, dv)}")
    mask = None
    if pair_mask is not None:
        mask = np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(N, H))
    outs = [np.full(sh, np.nan, dtype=np.float64) for sh in
            ((T, H, dk), (T, H, dk), (T, H, dv), (T, H, dk), (T, H), (N, H, dk, dv))]
    f64 = ctypes.c_double
    rc = lib.kda_oracle_prefill_backward(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                         _ptr(v, ctypes.c_float), _ptr(la, ctypes.c_float),
                                         _ptr(b, ctypes.c_float), _ptr(s0, f64),
                                         _ptr(cu, ctypes.c_int32), N, T, H, dk, dv,
                                         _ptr(do, f64), _ptr(dst, f64), _ptr(mask, ctypes.c_uint8),
                                         *[_ptr(x, f64) for x in outs],
                                         int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill_backward failed with status {rc}")
    return tuple(outs)


def gdn_prefill_backward(q, k, v, log_alpha, beta, S0, cu_seqlens, dO, dS_T=None, **kw):
    """Backward of ``gdn_prefill``: the per-channel backward with the gate
    repeated over the channels, its log-gate gradient summed over them (the
    chain rule of that repetition).  dlog_alpha is [T, H]."""
    q = np.asarray(q)
    la = np.asarray(log_alpha, dtype=np.float32)
    la = np.ascontiguousarray(np.broadcast_to(la[:, :, None], la.shape + (q.shape[2],)))
    dq, dk, dv, dla, db, dS0 = prefill_backward(q, k, v, la, beta, S0, cu_seqlens, dO, dS_T, **kw)
    return dq, dk, dv, dla.sum(axis=2), db, dS0
