"""Gated DeltaNet (one gate per token and head) through the gdn_* entry
points: parity against the fp64 oracle's scalar-gate functions, and the same
bits as the KDA entry points with the gate repeated over the key channels."""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload, upload_step, valid_splits

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, H, d_k, d_v, dtype, s0
    ([63, 64, 65], 2, 32, 32, "f32", True),
    ([127, 0, 200], 2, 64, 64, "f32", True),
    ([1, 63, 64, 65, 0, 127], 3, 128, 128, "bf16", True),
    ([300], 2, 64, 32, "bf16", True),
    ([77, 190], 2, 32, 128, "bf16", False),
    ([2 * 4096 + 77, 300], 2, 128, 128, "bf16", True),  # runs in segments
]


def _scalar_gate(x):
    """The per-head gate: channel 0 of the generated per-channel gate."""
    return np.ascontiguousarray(x.log_alpha[:, :, 0])


def _id(c):
    return f"L{'-'.join(map(str, c[0]))}_H{c[1]}_dk{c[2]}_dv{c[3]}_{c[4]}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_gdn_prefill_matches_oracle_and_kda(case):
    import torch
    lengths, H, dk, dv, dtype, s0 = case
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths) + dk + 1,
                                   s0_std=1.0 if s0 else None)
    la = _scalar_gate(x)
    log(f"  oracle {lengths} H={H} dk={dk} dv={dv} {dtype}")
    ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    la_d = torch.from_numpy(la).cuda()
    la_full = la_d[:, :, None].expand(-1, -1, dk).contiguous()
    for split in valid_splits(dv):
        log(f"  gdn prefill v_split={split}")
        o, ST = kda.gdn_prefill_t(**dict(d, log_alpha=la_d), v_split=split)
        assert_close(host(o), ref_o, dtype, "o")
        assert_close(host(ST), ref_S, dtype, "S_T")
        o2, ST2 = kda.prefill(**dict(d, log_alpha=la_full), v_split=split)
        assert torch.equal(o, o2) and torch.equal(ST, ST2), "GDN != KDA with the gate repeated"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gdn_decode_matches_oracle_and_kda(dtype):
    import torch
    N, H, dk, dv, steps = 5, 3, 128, 64, 12
    S_ref = np.ascontiguousarray(inputs.decode_initial_state(N, H, dk, dv, seed=9, s0_std=1.0)
                                 .astype(np.float64))
    S = torch.from_numpy(S_ref.astype(np.float32)).cuda()
    S_kda = S.clone()
    for step in range(steps):
        s = inputs.decode_step_inputs(N, H, dk, dv, step, seed=9, dtype=dtype)
        la = np.ascontiguousarray(s.log_alpha[:, :, 0])
        o_ref = oracle.gdn_decode_step(s.q, s.k, s.v, la, s.beta, S_ref)
        d = upload_step(s)
        la_d = torch.from_numpy(la).cuda()
        o = kda.gdn_decode_step_t(**dict(d, log_alpha=la_d), S=S)
        o2 = kda.decode_step(**dict(d, log_alpha=la_d[:, :, None].expand(-1, -1, dk).contiguous()), S=S_kda)
        assert_close(host(o), o_ref, dtype, f"o step {step}")
        assert torch.equal(o, o2) and torch.equal(S, S_kda), f"GDN != KDA at step {step}"
    assert_close(host(S), S_ref, dtype, "S after all steps")


def test_gdn_varlen_32k_sampled_heads():
    """The 32k varlen batch with one gate per head (channel 0 of the
    workload's gates), in the launch shape of the default entry point."""
    import torch
    x = inputs.make_workload("prefill_varlen8_32k_h32_d128_bf16")
    la = _scalar_gate(x)
    heads = [2, 29]
    mask = np.zeros((x.N, x.H), bool)
    mask[:, heads] = True
    log(f"  oracle on heads {heads}")
    ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens, pair_mask=mask)
    d = upload(x)
    o, ST = kda.gdn_prefill_t(**dict(d, log_alpha=torch.from_numpy(la).cuda()))
    assert_close(host(o[:, heads]), ref_o[:, heads], "bf16", "o (sampled heads)")
    assert_close(host(ST[:, heads]), ref_S[:, heads], "bf16", "S_T (sampled heads)")


def test_gdn_wide_decay():
    """One gate of -5 per token and head (the decay summed over 16 tokens at
    the wide-decay limit) through the wide-decay variant."""
    import torch
    x = inputs.make_prefill_inputs([400, 17], 2, 128, 128, "bf16", seed=41, s0_std=1.0)
    la = np.full(x.log_alpha.shape[:2], -5.0, np.float32)
    ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    o, ST = kda.gdn_prefill_t(**dict(d, log_alpha=torch.from_numpy(la).cuda()), wide_decay=True)
    assert_close(host(o), ref_o, "bf16", "o")
    assert_close(host(ST), ref_S, "bf16", "S_T")


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("case", [([70, 0, 33], 2, 64, 64, "f32"), ([150, 40], 2, 128, 128, "bf16"),
                                  ([37], 3, 32, 128, "bf16")], ids=lambda c: f"L{'-'.join(map(str, c[0]))}_dk{c[2]}_dv{c[3]}_{c[4]}")
def test_gdn_backward_matches_oracle_and_kda(case, path):
    """gdn_prefill_backward against the oracle's scalar-gate backward; its
    other gradients carry the same bits as kda_prefill_backward's with the
    gate repeated over the channels, and its gate gradient is their channel sum."""
    import torch
    lengths, H, dk, dv, dtype = case
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths) + 11, s0_std=1.0)
    la = _scalar_gate(x)
    dO, dST = inputs.make_backward_grads(x, seed=sum(lengths) + 12)
    ref = oracle.gdn_prefill_backward(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens, dO.astype(np.float64), dST)
    d = upload(x)
    td = d["q"].dtype
    dO_d, dST_d = torch.from_numpy(dO).cuda().to(td), torch.from_numpy(dST).cuda()
    la_d = torch.from_numpy(la).cuda()
    args = lambda g: (d["q"], d["k"], d["v"], g, d["beta"], d["S0"], d["cu_seqlens"], dO_d, dST_d)
    anyd = path == "recurrent"
    got = kda.gdn_prefill_backward_t(*args(la_d), any_decay=anyd)
    full = kda.prefill_backward(*args(la_d[:, :, None].expand(-1, -1, dk).contiguous()), any_decay=anyd)
    torch.cuda.synchronize()
    names = ("d_q", "d_k", "d_v", "d_log_alpha", "d_beta", "d_S0")
    for name, g, r in zip(names, got, ref):
        assert_close(host(g), r, dtype, name)
    for i in (0, 1, 2, 4, 5):
        assert torch.equal(got[i], full[i]), f"{names[i]}: GDN != KDA with the gate repeated"
    assert_close(host(got[3]), host(full[3]).sum(axis=2), "f32", "d_log_alpha vs channel sum")
