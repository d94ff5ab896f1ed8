"""Helpers shared by the GPU tests: upload seeded inputs, compare with the
oracle using the tolerance metric max|gpu - ref| / max|ref|."""
from __future__ import annotations

import sys

import numpy as np

# bf16 inputs: 2e-2; fp32 inputs: 1e-4 (relative to the reference's max magnitude)
TOL = {"bf16": 2e-2, "f32": 1e-4}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def upload(x, device="cuda"):
    """PrefillInputs -> dict of device tensors (q/k/v in the storage dtype)."""
    import torch
    td = torch_dtype(x.dtype)
    d = dict(
        q=torch.from_numpy(x.q).to(device).to(td),
        k=torch.from_numpy(x.k).to(device).to(td),
        v=torch.from_numpy(x.v).to(device).to(td),
        log_alpha=torch.from_numpy(x.log_alpha).to(device),
        beta=torch.from_numpy(x.beta).to(device),
        S0=None if x.S0 is None else torch.from_numpy(x.S0).to(device),
        cu_seqlens=torch.from_numpy(x.cu_seqlens).to(device),
    )
    return d


def upload_step(s, device="cuda"):
    import torch
    td = torch_dtype(s.dtype)
    return dict(q=torch.from_numpy(s.q).to(device).to(td), k=torch.from_numpy(s.k).to(device).to(td),
                v=torch.from_numpy(s.v).to(device).to(td),
                log_alpha=torch.from_numpy(s.log_alpha).to(device),
                beta=torch.from_numpy(s.beta).to(device))


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    m = float(np.max(np.abs(ref)))
    e = float(np.max(np.abs(gpu - ref)))
    return e / m if m > 0 else e


def assert_close(gpu, ref, dtype: str, what: str) -> float:
    e = rel_err(gpu, ref)
    log(f"    {what}: rel err {e:.3e} (tol {TOL[dtype]:.0e})")
    assert e <= TOL[dtype], f"{what}: rel err {e:.3e} > {TOL[dtype]:.0e}"
    return e


def valid_splits(d_v: int):
    return [s for s in (1, 2, 4, 8) if d_v // s >= 16]
