"""Backward pass of the prefill against the fp64 oracle's reverse-mode
recurrence: every gradient, element by element, on seeded inputs covering
ragged chunks, empty sequences and every head size, for both paths: the
chunked MFMA backward (kda_prefill_backward) and the token-recurrent one
(kda_prefill_backward_ex with KDA_PREFILL_ANY_DECAY)."""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload

pytestmark = pytest.mark.gpu

NAMES = ("d_q", "d_k", "d_v", "d_log_alpha", "d_beta", "d_S0")

CASES = [
    # lengths, H, d_k, d_v, dtype, s0, dS_T
    ([1, 17, 40], 2, 32, 32, "f32", True, True),
    ([63, 0, 64, 65], 2, 64, 64, "f32", True, True),
    ([0, 5], 2, 128, 32, "f32", True, True),
    ([40], 1, 32, 128, "f32", True, True),
    ([100, 33], 2, 128, 128, "bf16", True, True),
    ([77], 2, 128, 64, "bf16", False, False),
    ([50, 20], 3, 64, 128, "bf16", True, False),
    ([300], 2, 128, 128, "bf16", True, True),
]


def _id(c):
    return f"L{'-'.join(map(str, c[0]))}_H{c[1]}_dk{c[2]}_dv{c[3]}_{c[4]}{'' if c[5] else '_noS0'}{'' if c[6] else '_nodST'}"


PATHS = ["chunked", "recurrent"]


def _run(x, dO, dST, path="chunked"):
    import torch
    d = upload(x)
    td = d["q"].dtype
    dO_d = torch.from_numpy(dO).cuda().to(td)
    dST_d = None if dST is None else torch.from_numpy(dST).cuda()
    return kda.prefill_backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                d["cu_seqlens"], dO_d, dST_d, any_decay=(path == "recurrent"))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_matches_oracle(case, path):
    import torch
    lengths, H, dk, dv, dtype, s0, dst = case
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths) + dk + 7,
                                   s0_std=1.0 if s0 else None)
    dO, dST = inputs.make_backward_grads(x, seed=sum(lengths) + 3, with_dS_T=dst)
    log(f"  oracle backward {lengths} H={H} dk={dk} dv={dv} {dtype}")
    ref = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  dO.astype(np.float64), dST)
    log(f"  gpu backward ({path})")
    got = _run(x, dO, dST, path)
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        assert_close(host(g), r, dtype, name)


@pytest.mark.parametrize("path", PATHS)
def test_backward_is_deterministic(path):
    """Same bits on every run (the token-recurrent path adds two slices' row
    sums atomically onto zero; the chunked path has no atomics)."""
    import torch
    x = inputs.make_prefill_inputs([200, 61], 2, 128, 128, "bf16", seed=5, s0_std=1.0)
    dO, dST = inputs.make_backward_grads(x, seed=6)
    first = _run(x, dO, dST, path)
    for rep in range(3):
        again = _run(x, dO, dST, path)
        torch.cuda.synchronize()
        for name, a, b in zip(NAMES, first, again):
            assert torch.equal(a, b), f"{name} differs on repeat {rep}"


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 128), ("f32", 32)])
def test_chunked_backward_at_the_decay_limit(dtype, dk):
    """The chunked backward's contract is the prefill's: log alpha summed over
    any 32 consecutive tokens >= -80.  Gates of -2.5 per token reach it."""
    import torch
    x = inputs.make_prefill_inputs([150, 47], 2, dk, 128, dtype, seed=91, s0_std=1.0)
    x.log_alpha[:] = -2.5
    dO, dST = inputs.make_backward_grads(x, seed=92)
    ref = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  dO.astype(np.float64), dST)
    got = _run(x, dO, dST)
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        assert_close(host(g), r, dtype, name)


@pytest.mark.parametrize("path", PATHS)
def test_backward_varlen_32k_sampled_heads(path):
    """The 32k varlen batch (8 sequences, H = 32, d = 128, bf16) in full on the
    GPU; the oracle checks heads 5 and 30 of every sequence."""
    import torch
    x = inputs.make_workload("prefill_varlen8_32k_h32_d128_bf16")
    dO, dST = inputs.make_backward_grads(x, seed=12)
    heads = [5, 30]
    mask = np.zeros((x.N, x.H), bool)
    mask[:, heads] = True
    log(f"  oracle backward on heads {heads}")
    ref = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  dO.astype(np.float64), dST, pair_mask=mask)
    log(f"  gpu backward ({path})")
    got = _run(x, dO, dST, path)
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        assert_close(host(g[:, heads]), r[:, heads], "bf16", name)


def test_backward_strong_decay_and_resets():
    """The token-recurrent backward evaluates no decay products, so any finite
    log alpha works: gates drawn from -U(0, 5), plus tokens with log alpha =
    -1000 (a reset: alpha underflows to 0 in fp32 and fp64 alike)."""
    import torch
    x = inputs.make_prefill_inputs([90, 45], 2, 64, 128, "bf16", seed=77, s0_std=1.0,
                                   log_alpha_range=(0.0, 5.0))
    x.log_alpha[[3, 50, 51, 100], :, :] = -1000.0
    dO, dST = inputs.make_backward_grads(x, seed=78)
    ref = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  dO.astype(np.float64), dST)
    got = _run(x, dO, dST, "recurrent")
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        assert_close(host(g), r, "bf16", name)


@pytest.mark.parametrize("path", PATHS)
def test_backward_all_sequences_empty(path):
    """T_tot = 0: no token gradients, and the initial state's gradient is dL/dS_T."""
    import torch
    x = inputs.make_prefill_inputs([0, 0, 0], 2, 64, 128, "bf16", seed=3, s0_std=1.0)
    dO, dST = inputs.make_backward_grads(x, seed=4)
    got = _run(x, dO, dST, path)
    torch.cuda.synchronize()
    assert all(g.numel() == 0 for g in got[:5])
    assert torch.equal(got[5], torch.from_numpy(dST).cuda())


@pytest.mark.parametrize("path", PATHS)
def test_backward_many_short_sequences(path):
    """Forty sequences of 0 to 40 tokens (many not a multiple of 16) in one
    batch: every sequence's checkpoints land in their own slots."""
    import torch
    rng = np.random.default_rng(5)
    lengths = [int(v) for v in rng.integers(0, 41, size=40)]
    x = inputs.make_prefill_inputs(lengths, 1, 64, 64, "f32", seed=6, s0_std=1.0)
    dO, dST = inputs.make_backward_grads(x, seed=7)
    ref = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  dO.astype(np.float64), dST)
    got = _run(x, dO, dST, path)
    torch.cuda.synchronize()
    for name, g, r in zip(NAMES, got, ref):
        assert_close(host(g), r, "f32", name)
