"""GPU prefill parity against the fp64 oracle (through the C ABI).

Small cases span several chunks, ragged tails (lengths 1, 63, 64, 65, 127),
empty sequences, d_k != d_v, both dtypes and every launch shape; the full
workloads compare all outputs (T=256 fp32, T=4096) or oracle-sampled heads
(the 32k varlen batch and the 128k sequence) in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload, valid_splits

pytestmark = pytest.mark.gpu

SMALL = [
    # lengths, H, d_k, d_v, dtype, s0
    ([1], 1, 32, 32, "f32", True),
    ([63, 64, 65], 2, 32, 32, "f32", False),
    ([127, 0, 200], 2, 64, 64, "f32", True),
    ([130, 1, 64], 2, 128, 128, "f32", True),
    ([64, 65], 1, 64, 128, "f32", True),
    ([1, 63, 64, 65, 0, 127], 3, 128, 128, "bf16", True),
    ([300], 2, 64, 32, "bf16", True),
    ([77, 190], 2, 32, 128, "bf16", False),
    ([129, 255], 2, 64, 64, "bf16", True),
    ([513], 1, 128, 64, "bf16", True),
]


def _small_id(c):
    return f"L{'-'.join(map(str, c[0]))}_H{c[1]}_dk{c[2]}_dv{c[3]}_{c[4]}_{'S0' if c[5] else 'zero'}"


def _run_case(lengths, H, dk, dv, dtype, s0, seed):
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=seed,
                                   s0_std=1.0 if s0 else None)
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    for split in valid_splits(dv):
        log(f"  prefill {lengths} H={H} dk={dk} dv={dv} {dtype} v_split={split}")
        o, ST = kda.prefill(**d, v_split=split)
        assert_close(host(o), ref_o, dtype, "o")
        assert_close(host(ST), ref_S, dtype, "S_T")


@pytest.mark.parametrize("case", SMALL, ids=_small_id)
def test_small_cases_every_split(case):
    _run_case(*case, seed=sum(case[0]) + case[2])


# log alpha ranges: "max32" puts the decay summed over each 32-token chunk at
# -80 exactly (the default contract's limit); "max16" puts the decay summed
# over any 16 consecutive tokens at -80 exactly (the wide-decay limit).
DECAY_RANGES = {"mixed32": (0.5, 2.5), "max32": (2.5, 2.5), "mixed16": (0.0, 5.0), "max16": (5.0, 5.0)}


def _strong_decay_case(dk, dtype, la_range, wide):
    x = inputs.make_prefill_inputs([700, 33, 1], 2, dk, dk, dtype, seed=11,
                                   log_alpha_range=la_range, s0_std=1.0)
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    for split in valid_splits(dk):
        log(f"  strong decay {la_range} d={dk} {dtype} wide={wide} v_split={split}")
        o, ST = kda.prefill(**d, v_split=split, wide_decay=wide)
        assert_close(host(o), ref_o, dtype, "o")
        assert_close(host(ST), ref_S, dtype, "S_T")


@pytest.mark.parametrize("dk,dtype", [(128, "bf16"), (128, "f32"), (64, "f32")])
@pytest.mark.parametrize("name", ["mixed32", "max32"])
def test_strong_decay_at_the_contract_limit(dk, dtype, name):
    """log alpha down to -2.5 per token and channel: the chunk's exponentials
    span e^(+-80) at the default contract's limit.  Covers 32-token chunks in
    both storage types and the 16-token chunks of fp32 at d = 128."""
    _strong_decay_case(dk, dtype, DECAY_RANGES[name], False)


@pytest.mark.parametrize("dk,dtype", [(128, "bf16"), (128, "f32"), (64, "f32")])
@pytest.mark.parametrize("name", ["mixed32", "max32", "mixed16", "max16"])
def test_wide_decay_at_its_limit(dk, dtype, name):
    """The wide-decay variant down to -5 per token and channel: exponents of
    the strongly decaying channels are taken from the chunk's middle row, so
    a chunk's exponentials stay within e^(+-80) up to its limit ("max16")."""
    _strong_decay_case(dk, dtype, DECAY_RANGES[name], True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_decay_in_some_channels(dtype):
    """Decay of -5 per token in key channels 0..39 only (the first channel
    strip and part of the second), weak elsewhere: chunks where some channels
    take their exponents from the middle row and the others from the chunk
    start, within one producer strip and across strips."""
    x = inputs.make_prefill_inputs([300, 45], 2, 128, 128, dtype, seed=12, s0_std=1.0)
    x.log_alpha[:, :, :40] = -5.0
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    for split in valid_splits(128):
        log(f"  wide decay, channels 0..39 strong, {dtype} v_split={split}")
        o, ST = kda.prefill(**d, v_split=split, wide_decay=True)
        assert_close(host(o), ref_o, dtype, "o")
        assert_close(host(ST), ref_S, dtype, "S_T")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_decay_with_segments(dtype):
    """A long sequence that runs in segments (identity runs and state chain)
    with gates at the wide-decay limit range, -U(0, 5) per token."""
    x = inputs.make_prefill_inputs([5000, 100], 2, 128, 128, dtype, seed=23,
                                   log_alpha_range=(0.0, 5.0), s0_std=1.0)
    code = kda.KDA_DTYPE_BF16 if dtype == "bf16" else kda.KDA_DTYPE_F32
    assert kda.kda_prefill_workspace_size(x.N, x.T_tot, 2, 128, 128, code) > 0
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = kda.prefill(**upload(x), wide_decay=True)
    assert_close(host(o), ref_o, dtype, "o")
    assert_close(host(ST), ref_S, dtype, "S_T")


@pytest.mark.parametrize("lengths", [[300, 1, 64], [4096 + 500, 77]], ids=["short", "segmented"])
def test_wide_decay_keeps_the_bits_within_the_default_contract(lengths):
    """Within the default contract no channel moves its reference, and the
    wide-decay variant gives exactly the default variant's bits (KDA and
    GDN, every launch shape)."""
    import torch
    x = inputs.make_prefill_inputs(lengths, 2, 128, 128, "bf16", seed=21, s0_std=1.0)
    d = upload(x)
    for split in valid_splits(128):
        o0, S0 = kda.prefill(**d, v_split=split)
        o1, S1 = kda.prefill(**d, v_split=split, wide_decay=True)
        assert torch.equal(o0, o1) and torch.equal(S0, S1), f"KDA v_split={split}"
    la = d["log_alpha"][:, :, 0].contiguous()
    o0, S0 = kda.gdn_prefill_t(**dict(d, log_alpha=la))
    o1, S1 = kda.gdn_prefill_t(**dict(d, log_alpha=la), wide_decay=True)
    assert torch.equal(o0, o1) and torch.equal(S0, S1), "GDN"


SEGMENTED = [
    # lengths (batches past 1024 tokens run in segments of 1024-32768 tokens), H, d_k = d_v, dtype, s0
    ([2 * 4096 + 77, 300, 4096, 4097], 2, 128, "bf16", True),
    ([20000, 300], 2, 64, "bf16", True),  # 5120-token segments: ten output tiles each
    ([3 * 4096 + 5, 10], 1, 128, "f32", True),
    ([4100, 0, 9000], 2, 64, "bf16", True),
    ([8192, 1], 2, 32, "f32", False),
]


@pytest.mark.parametrize("case", SEGMENTED, ids=lambda c: f"L{'-'.join(map(str, c[0]))}_H{c[1]}_d{c[2]}_{c[3]}")
def test_long_sequences_in_segments(case):
    """Long sequences in small batches run as parallel segments chained by
    the fix-up passes: every output and final state against the oracle, and the
    same bits for every launch shape."""
    import torch
    lengths, H, d, dtype, s0 = case
    x = inputs.make_prefill_inputs(lengths, H, d, d, dtype, seed=sum(lengths) + d,
                                   s0_std=1.0 if s0 else None)
    code = kda.KDA_DTYPE_BF16 if dtype == "bf16" else kda.KDA_DTYPE_F32
    assert kda.kda_prefill_workspace_size(x.N, x.T_tot, H, d, d, code) > 0
    log(f"  oracle {lengths} H={H} d={d} {dtype}")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    dd = upload(x)
    first = None
    for split in valid_splits(d):
        log(f"  segmented prefill v_split={split}")
        o, ST = kda.prefill(**dd, v_split=split)
        if first is None:
            assert_close(host(o), ref_o, dtype, "o")
            assert_close(host(ST), ref_S, dtype, "S_T")
            for n in range(x.N):
                a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
                assert_close(host(o[a:b]), ref_o[a:b], dtype, f"o sequence {n} (len {b - a})")
            first = (o, ST)
        else:
            assert torch.equal(o, first[0]) and torch.equal(ST, first[1]), f"v_split={split}"


def test_workload_t256_fp32():
    x = inputs.make_workload("prefill_t256_h2_d32_f32")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = kda.prefill(**upload(x))
    assert_close(host(o), ref_o, "f32", "o")
    assert_close(host(ST), ref_S, "f32", "S_T")


def test_workload_t4096():
    x = inputs.make_workload("prefill_t4096_h32_d128_bf16")
    log("  oracle, 32 heads x 4096 tokens")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = kda.prefill(**upload(x))
    assert_close(host(o), ref_o, "bf16", "o")
    assert_close(host(ST), ref_S, "bf16", "S_T")


def _sampled(x, heads):
    mask = np.zeros((x.N, x.H), bool)
    mask[:, heads] = True
    return mask


def test_workload_varlen_32k_sampled_heads():
    x = inputs.make_workload("prefill_varlen8_32k_h32_d128_bf16")
    heads = [0, 13, 31]
    log(f"  oracle on heads {heads} of all 8 sequences")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  pair_mask=_sampled(x, heads))
    o, ST = kda.prefill(**upload(x))
    o, ST = host(o), host(ST)
    assert_close(o[:, heads], ref_o[:, heads], "bf16", "o (sampled heads)")
    assert_close(ST[:, heads], ref_S[:, heads], "bf16", "S_T (sampled heads)")
    for n in range(x.N):
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        assert_close(o[a:b, heads], ref_o[a:b, heads], "bf16", f"o sequence {n} (len {b - a})")


def test_workload_128k_sampled_heads_windows():
    x = inputs.make_workload("prefill_t131072_h32_d128_bf16")
    heads = [5, 26]
    log(f"  oracle on heads {heads} over 131072 tokens")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens,
                                  pair_mask=_sampled(x, heads))
    d = upload(x)
    del x
    o, ST = kda.prefill(**d)
    o = host(o[:, heads])
    ST = host(ST[:, heads])
    assert_close(ST, ref_S[:, heads], "bf16", "S_T")
    assert_close(o[:4096], ref_o[:4096, heads], "bf16", "o first 4096")
    assert_close(o[-4096:], ref_o[-4096:, heads], "bf16", "o last 4096")
    assert_close(o, ref_o[:, heads], "bf16", "o all tokens")
