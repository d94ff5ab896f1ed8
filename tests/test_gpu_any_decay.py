"""KDA_PREFILL_ANY_DECAY: the token-recurrent prefill has no decay-range
contract.  Gates from -U(0, 5) plus reset tokens (log alpha = -1000: alpha
underflows to 0 in fp32 and in the fp64 oracle alike) against the oracle, for
per-channel and per-head gates; and on ordinary gates it agrees with the
chunked kernel."""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload

pytestmark = pytest.mark.gpu

RESET_ROWS = [3, 50, 51, 100]

CASES = [
    # lengths, H, d_k, d_v, dtype
    ([90, 0, 45], 2, 128, 128, "bf16"),
    ([70, 33], 2, 64, 32, "f32"),
    ([64, 17], 3, 32, 64, "f32"),
]


def _strong(lengths, H, dk, dv, dtype, seed):
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=seed, s0_std=1.0, log_alpha_range=(0.0, 5.0))
    rows = [r for r in RESET_ROWS if r < x.q.shape[0]]
    x.log_alpha[rows, :, :] = -1000.0
    return x


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{'-'.join(map(str, c[0]))}_dk{c[2]}_dv{c[3]}_{c[4]}")
def test_any_decay_matches_oracle(case):
    import torch
    lengths, H, dk, dv, dtype = case
    x = _strong(lengths, H, dk, dv, dtype, seed=sum(lengths) + dk)
    log(f"  oracle {lengths} dk={dk} dv={dv} {dtype}")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    o, ST = kda.prefill(**d, any_decay=True)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, dtype, "o")
    assert_close(host(ST), ref_S, dtype, "S_T")


def test_any_decay_scalar_gate_matches_oracle():
    import torch
    x = _strong([80, 40], 2, 128, 64, "bf16", seed=8)
    la = np.ascontiguousarray(x.log_alpha[:, :, 0])
    ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    o, ST = kda.gdn_prefill_t(**dict(d, log_alpha=torch.from_numpy(la).cuda()), any_decay=True)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, "bf16", "o")
    assert_close(host(ST), ref_S, "bf16", "S_T")


def test_any_decay_agrees_with_chunked_kernel_in_place():
    """Ordinary gates: the token-recurrent and chunked kernels agree to the
    tolerance, and S_T may be S0 itself (state updated in place)."""
    import torch
    x = inputs.make_prefill_inputs([200, 31], 2, 128, 128, "bf16", seed=9, s0_std=1.0)
    d = upload(x)
    o_ref, S_ref = kda.prefill(**d)
    S = d["S0"].clone()
    o, ST = kda.prefill(**dict(d, S0=S), S_T=S, any_decay=True)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    assert_close(host(o), host(o_ref), "bf16", "o vs chunked")
    assert_close(host(S), host(S_ref), "bf16", "S_T vs chunked")
