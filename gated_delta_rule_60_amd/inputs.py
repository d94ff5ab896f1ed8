"""Seeded synthetic workloads for the KDA forward pass.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the recurrence's arithmetic.  Both the GPU path and the
fp64 CPU oracle are fed from here, so they see bit-identical inputs.

Recipe (every array is drawn with ``numpy.random.default_rng``, float32
draws, in this order: lengths, q, k, v, log_alpha, beta, S0):

* q, k   ~ N(0, 1), L2-normalised per (token, head) over d_k; q is further
  scaled by 1/sqrt(d_k).
* v      ~ N(0, 1).
* log_alpha = -Uniform(lo, hi) per (token, head, key channel); alpha =
  exp(log_alpha) is one retention factor per channel (the fine-grained gate
  of "Kimi Linear：让长上下文大模型真正实用的线性注意力架构", section 三.1).
* beta   = sigmoid(N(0, 1)) per (token, head): the delta rule's step size.
* S0     = s0_std * N(0, 1) per (sequence, head, d_k, d_v), or absent.

For bf16 workloads q, k, v are rounded to bfloat16 (round to nearest, ties
to even) from the float32 draw; log_alpha, beta and S0 stay float32.  Every
array is returned as float32 holding exactly the values the device sees.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "make_backward_grads",
    "PrefillInputs",
    "DecodeStepInputs",
    "WORKLOADS",
    "round_to_bf16",
    "varlen_lengths",
    "make_prefill_inputs",
    "make_workload",
    "decode_initial_state",
    "decode_step_inputs",
]


def round_to_bf16(x: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16, so a
    later float32 -> bfloat16 cast is exact.  Inputs must be finite (then the
    32-bit integer sum below cannot overflow).  ``out`` may be ``x`` itself.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if out is None:
        out = np.empty_like(x)
    src = x.reshape(-1).view(np.uint32)
    dst = out.reshape(-1).view(np.uint32)
    step = 1 << 22
    for s in range(0, src.shape[0], step):
        u = src[s:s + step].copy()
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        u &= np.uint32(0xFFFF0000)
        dst[s:s + step] = u
    return out


@dataclasses.dataclass
class PrefillInputs:
    q: np.ndarray            # [T_tot, H, d_k] float32 (bf16-exact when dtype == "bf16")
    k: np.ndarray            # [T_tot, H, d_k]
    v: np.ndarray            # [T_tot, H, d_v]
    log_alpha: np.ndarray    # [T_tot, H, d_k] float32, <= 0
    beta: np.ndarray         # [T_tot, H] float32 in (0, 1)
    S0: Optional[np.ndarray]  # [N, H, d_k, d_v] float32 or None (zero state)
    cu_seqlens: np.ndarray   # [N + 1] int32
    dtype: str               # "bf16" or "f32": storage type of q, k, v and o

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def T_tot(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def d_k(self) -> int:
        return int(self.q.shape[2])

    @property
    def d_v(self) -> int:
        return int(self.v.shape[2])


@dataclasses.dataclass
class DecodeStepInputs:
    q: np.ndarray            # [N, H, d_k]
    k: np.ndarray            # [N, H, d_k]
    v: np.ndarray            # [N, H, d_v]
    log_alpha: np.ndarray    # [N, H, d_k]
    beta: np.ndarray         # [N, H]
    dtype: str


def _unit_rows_(x: np.ndarray) -> np.ndarray:
    """Divide each row (last axis) by its L2 norm, in place, block by block;
    the norm is accumulated in float64."""
    flat = x.reshape(-1, x.shape[-1])
    step = 1 << 18
    for s in range(0, flat.shape[0], step):
        blk = flat[s:s + step]
        n = np.sqrt(np.einsum("ij,ij->i", blk, blk, dtype=np.float64))
        blk /= n.astype(np.float32)[:, None]
    return x


def _qkv_gates(rng: np.random.Generator, lead: tuple, d_k: int, d_v: int,
               log_alpha_range: tuple, dtype: str):
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    q = _unit_rows_(rng.standard_normal(lead + (d_k,), dtype=np.float32))
    q *= np.float32(1.0 / np.sqrt(d_k))
    k = _unit_rows_(rng.standard_normal(lead + (d_k,), dtype=np.float32))
    v = rng.standard_normal(lead + (d_v,), dtype=np.float32)
    lo, hi = log_alpha_range
    log_alpha = rng.random(lead + (d_k,), dtype=np.float32)
    log_alpha *= np.float32(-(hi - lo))
    log_alpha -= np.float32(lo)
    z = rng.standard_normal(lead, dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    if dtype == "bf16":
        for a in (q, k, v):
            round_to_bf16(a, out=a)
    return q, k, v, log_alpha, beta


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> list:
    """n sequence lengths uniform on [lo, hi] inclusive (first draw of a workload)."""
    return [int(x) for x in rng.integers(lo, hi, size=n, endpoint=True)]


def make_prefill_inputs(lengths: Sequence[int], H: int, d_k: int, d_v: int, dtype: str,
                        seed, log_alpha_range=(0.001, 0.1), s0_std: Optional[float] = 0.01,
                        rng: Optional[np.random.Generator] = None) -> PrefillInputs:
    """Packed varlen prefill inputs.  ``lengths`` may contain zeros."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q, k, v, la, beta = _qkv_gates(rng, (T, H), d_k, d_v, log_alpha_range, dtype)
    S0 = None
    if s0_std is not None:
        S0 = (np.float32(s0_std) * rng.standard_normal((len(lengths), H, d_k, d_v), dtype=np.float32))
    return PrefillInputs(q, k, v, la, beta, S0, cu, dtype)


def decode_initial_state(N: int, H: int, d_k: int, d_v: int, seed=3, s0_std=0.01) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (np.float32(s0_std) * rng.standard_normal((N, H, d_k, d_v), dtype=np.float32))


def decode_step_inputs(N: int, H: int, d_k: int, d_v: int, step: int, seed=3, dtype="bf16",
                       log_alpha_range=(0.001, 0.1)) -> DecodeStepInputs:
    """Inputs of decode step ``step``; drawn from default_rng([seed, step])."""
    rng = np.random.default_rng([seed, step])
    q, k, v, la, beta = _qkv_gates(rng, (N, H), d_k, d_v, log_alpha_range, dtype)
    return DecodeStepInputs(q, k, v, la, beta, dtype)


# The five workloads: shapes, dtypes, distributions and seeds.
WORKLOADS = {
    # T=256, H=2, d=32, everything fp32, zero initial state.
    "prefill_t256_h2_d32_f32": dict(kind="prefill", seed=0, lengths=[256], H=2, d_k=32, d_v=32,
                                    dtype="f32", log_alpha_range=(0.001, 0.1), s0_std=None),
    # One 4096-token sequence, H=32, d=128, bf16 q/k/v.
    "prefill_t4096_h32_d128_bf16": dict(kind="prefill", seed=1, lengths=[4096], H=32, d_k=128,
                                        d_v=128, dtype="bf16", log_alpha_range=(0.001, 0.1),
                                        s0_std=0.01),
    # Packed batch of 8 sequences, lengths uniform on [1024, 8192] (seed 12 -> 32,677 tokens).
    "prefill_varlen8_32k_h32_d128_bf16": dict(kind="prefill", seed=12,
                                              lengths=("uniform", 8, 1024, 8192), H=32, d_k=128,
                                              d_v=128, dtype="bf16",
                                              log_alpha_range=(0.001, 0.1), s0_std=0.01),
    # 256 sequences x 1 token per step, 1000 consecutive steps, state carried.
    "decode_n256_h32_d128_bf16_x1000": dict(kind="decode", seed=3, N=256, H=32, d_k=128, d_v=128,
                                            dtype="bf16", steps=1000,
                                            log_alpha_range=(0.001, 0.1), s0_std=0.01),
    # One 131,072-token sequence (128k context), weaker decay.
    "prefill_t131072_h32_d128_bf16": dict(kind="prefill", seed=4, lengths=[131072], H=32, d_k=128,
                                          d_v=128, dtype="bf16",
                                          log_alpha_range=(0.0001, 0.05), s0_std=0.01),
}


def make_workload(name: str) -> PrefillInputs:
    """Materialise one of the prefill workloads in WORKLOADS."""
    w = WORKLOADS[name]
    if w["kind"] != "prefill":
        raise ValueError(f"{name} is a decode workload; use decode_step_inputs")
    rng = np.random.default_rng(w["seed"])
    lengths = w["lengths"]
    if isinstance(lengths, tuple) and lengths[0] == "uniform":
        lengths = varlen_lengths(rng, lengths[1], lengths[2], lengths[3])
    return make_prefill_inputs(lengths, w["H"], w["d_k"], w["d_v"], w["dtype"], None,
                               w["log_alpha_range"], w["s0_std"], rng=rng)


def make_any_decay_workload(resets_per_sequence: int = 8, seed: int = 13) -> PrefillInputs:
    """The 32k-token batch of eight sequences (the lengths, heads, head sizes
    and dtype of prefill_varlen8_32k_h32_d128_bf16) with gates outside the
    chunked kernels' contract: log alpha = -U(0, 5) per token, head and
    channel, and hard resets (log alpha = -1000 on every channel of every
    head: document boundaries inside a packed sequence) at
    ``resets_per_sequence`` seeded token positions of each sequence."""
    x = make_workload("prefill_varlen8_32k_h32_d128_bf16")
    rng = np.random.default_rng(seed)
    la = rng.random(x.log_alpha.shape, dtype=np.float32)
    la *= np.float32(-5.0)
    cu = x.cu_seqlens
    for n in range(int(cu.shape[0]) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        rows = rng.choice(b - a, size=min(resets_per_sequence, b - a), replace=False) + a
        la[rows] = np.float32(-1000.0)
    x.log_alpha = la
    return x


def make_backward_grads(x: PrefillInputs, seed, with_dS_T: bool = True):
    """Upstream gradients for a backward pass over the batch ``x``: dL/do
    [T_tot, H, d_v] (N(0,1), rounded to x's storage dtype) and dL/dS_T
    [N, H, d_k, d_v] (N(0,1) fp32, or None)."""
    rng = np.random.default_rng(seed)
    T, H = int(x.q.shape[0]), int(x.q.shape[1])
    d_k, d_v = int(x.q.shape[2]), int(x.v.shape[2])
    N = int(x.cu_seqlens.shape[0] - 1)
    dO = rng.standard_normal((T, H, d_v), dtype=np.float32)
    if x.dtype == "bf16":
        round_to_bf16(dO, out=dO)
    dST = rng.standard_normal((N, H, d_k, d_v), dtype=np.float32) if with_dS_T else None
    return dO, dST
