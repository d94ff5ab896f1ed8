"""kda_prefill_noalloc (for callers that cannot allocate) against kda_prefill:
the same kernels on the same inputs give the same bits, on two calls in a
row (the second smaller), on the segmented path that uses the fixed
workspace and on the one-pass path that uses none."""
import ctypes

import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
from gated_delta_rule_60_amd import _lib, inputs
from gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _noalloc(d, x, o, S):
    import torch
    code = kda.KDA_DTYPE_BF16 if x.dtype == "bf16" else kda.KDA_DTYPE_F32
    st = torch.cuda.current_stream()
    return _lib.load().kda_prefill_noalloc(
        d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_alpha"].data_ptr(),
        d["beta"].data_ptr(), d["S0"].data_ptr() if d["S0"] is not None else None, d["cu_seqlens"].data_ptr(),
        x.N, x.T_tot, x.H, x.d_k, x.d_v, code, o.data_ptr(), S.data_ptr(), int(st.cuda_stream))


def _case(lengths, H, seed):
    return inputs.make_prefill_inputs(lengths, H, 128, 128, "bf16", seed=seed, s0_std=0.01)


def test_noalloc_matches_kda_prefill_on_two_calls():
    import torch
    cases = [_case([4096], 32, 1), _case([2600], 8, 2), _case([300, 77], 2, 3)]
    # the first two run segmented and use the fixed workspace; the third runs in one pass
    for x in cases[:2]:
        need = kda.kda_prefill_workspace_size(x.N, x.T_tot, x.H, x.d_k, x.d_v, kda.KDA_DTYPE_BF16)
        assert 0 < need <= _lib.KDA_PREFILL_NOALLOC_WORKSPACE_BYTES
    assert kda.kda_prefill_workspace_size(2, 377, 2, 128, 128, kda.KDA_DTYPE_BF16) == 0
    ups = [upload(x) for x in cases]
    refs = [kda.prefill(**d) for d in ups]
    outs = []
    for x, d in zip(cases, ups):  # back to back on one stream, no synchronisation between
        o = torch.full((x.T_tot, x.H, x.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
        S = torch.full((x.N, x.H, x.d_k, x.d_v), float("nan"), dtype=torch.float32, device="cuda")
        rc = _noalloc(d, x, o, S)
        assert rc == kda.KDA_OK, kda.kda_last_error()
        outs.append((o, S))
    torch.cuda.synchronize()
    for i, ((o, S), (ro, rS)) in enumerate(zip(outs, refs)):
        log(f"    case {i}: T={cases[i].T_tot} H={cases[i].H}")
        assert torch.equal(o, ro) and torch.equal(S, rS), f"case {i} differs from kda_prefill"


def test_noalloc_rejects_sizes_beyond_the_fixed_workspace():
    big = kda.kda_prefill_workspace_size(1, 131072, 32, 128, 128, kda.KDA_DTYPE_BF16)
    assert big > _lib.KDA_PREFILL_NOALLOC_WORKSPACE_BYTES
    fake = 0x10000
    rc = _lib.load().kda_prefill_noalloc(fake, fake, fake, fake, fake, None, fake, 1, 131072, 32, 128, 128,
                                         kda.KDA_DTYPE_BF16, fake, fake, None)
    assert rc == kda.KDA_ERR_INVALID_ARG
    assert "fixed workspace" in kda.kda_last_error()
