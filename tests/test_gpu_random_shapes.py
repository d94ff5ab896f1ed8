"""A seeded sweep over shapes and options, each case compared element by
element with the fp64 oracle: ragged lengths (with empty sequences),
1-3 heads, every head size pair, both dtypes, every valid v_split, the
scalar gate and the wide- and any-decay variants, and the backward; then
small batches past 1024 tokens, which run in segments."""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload, valid_splits

pytestmark = pytest.mark.gpu


def _cases(n=60, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 5))
        lengths = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 300, size=N)]
        H = int(rng.integers(1, 4))
        dk = int(rng.choice([32, 64, 128]))
        dv = int(rng.choice([32, 64, 128]))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        split = int(rng.choice(valid_splits(dv)))
        mode = str(rng.choice(["kda", "kda", "gdn", "wide", "any"]))
        out.append((i, lengths, H, dk, dv, dtype, split, mode))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}_{c[7]}_L{'-'.join(map(str, c[1]))}_H{c[2]}_dk{c[3]}_dv{c[4]}_{c[5]}_s{c[6]}")
def test_random_shape_forward_and_backward(case):
    import torch
    i, lengths, H, dk, dv, dtype, split, mode = case
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=1000 + i, s0_std=1.0 if i % 3 else None,
                                   log_alpha_range=(0.0, 4.0) if mode in ("wide", "any") else (0.001, 0.1))
    d = upload(x)
    log(f"  case {case}")
    if mode == "gdn":
        la = np.ascontiguousarray(x.log_alpha[:, :, 0])
        ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens)
        o, ST = kda.gdn_prefill_t(**dict(d, log_alpha=torch.from_numpy(la).cuda()), v_split=split)
    else:
        ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
        o, ST = kda.prefill(**d, v_split=split, wide_decay=(mode == "wide"), any_decay=(mode == "any"))
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, dtype, "o")
    assert_close(host(ST), ref_S, dtype, "S_T")
    if mode in ("kda", "any"):
        dO, dST = inputs.make_backward_grads(x, seed=2000 + i, with_dS_T=bool(i % 2))
        refs = oracle.prefill_backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                       dO.astype(np.float64), dST)
        td = d["q"].dtype
        grads = kda.prefill_backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                     d["cu_seqlens"], torch.from_numpy(dO).cuda().to(td),
                                     None if dST is None else torch.from_numpy(dST).cuda(),
                                     any_decay=(mode == "any"))
        torch.cuda.synchronize()
        for name, g, r in zip(("d_q", "d_k", "d_v", "d_log_alpha", "d_beta", "d_S0"), grads, refs):
            assert_close(host(g), r, dtype, name)


def _segment_cases(n=14, seed=4242):
    """Small batches past 1024 tokens, d_k = d_v: the segmented path. Lengths
    mix the cut points of the 1024-32768-token segments (one token past a
    multiple of 512 or 1024) with random lengths and empty sequences."""
    rng = np.random.default_rng(seed)
    edges = [1025, 1536, 1537, 2049, 4096, 4097, 6145]
    out = []
    for i in range(n):
        N = int(rng.integers(1, 4))
        lengths = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 7000))
                   for _ in range(N)]
        if sum(lengths) <= 1024:
            lengths[0] += 1025
        if i % 4 == 3:
            lengths.insert(int(rng.integers(0, N + 1)), 0)
        H = int(rng.integers(1, 3))
        d = int(rng.choice([32, 64, 128]))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        split = int(rng.choice(valid_splits(d)))
        out.append((i, lengths, H, d, dtype, split))
    return out


@pytest.mark.parametrize("case", _segment_cases(),
                         ids=lambda c: f"{c[0]}_L{'-'.join(map(str, c[1]))}_H{c[2]}_d{c[3]}_{c[4]}_s{c[5]}")
def test_random_segmented_batches(case):
    import torch
    i, lengths, H, d, dtype, split = case
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype, seed=3000 + i, s0_std=1.0 if i % 2 else None)
    code = kda.KDA_DTYPE_BF16 if dtype == "bf16" else kda.KDA_DTYPE_F32
    assert kda.kda_prefill_workspace_size(x.N, x.T_tot, H, d, d, code) > 0, "not the segmented path"
    log(f"  case {case}")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    dd = upload(x)
    o, ST = kda.prefill(**dd, v_split=split)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, dtype, "o")
    assert_close(host(ST), ref_S, dtype, "S_T")
    for n in range(x.N):
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        if b > a:
            assert_close(host(o[a:b]), ref_o[a:b], dtype, f"o sequence {n} (len {b - a})")
