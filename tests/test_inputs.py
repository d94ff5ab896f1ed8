"""The seeded workload generators (CPU only)."""
import numpy as np

from gated_delta_rule_60_amd import inputs


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-3], np.float32)
    r = inputs.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even (mantissa ...0)
    assert r[2] == np.float32(1.0 + 4 * 2**-8)  # tie -> even (rounds up)
    assert r[3] == 1.0
    assert r[4] == -2.5
    # every result has a zero low half-word (exactly representable in bf16)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2**-8)


def test_varlen_lengths_of_the_32k_workload():
    rng = np.random.default_rng(12)
    lengths = inputs.varlen_lengths(rng, 8, 1024, 8192)
    assert lengths == [5416, 2822, 7999, 7811, 1485, 2381, 2454, 2309]
    assert sum(lengths) == 32677
    assert all(n % 64 != 0 for n in lengths)


def test_prefill_generator_distributions_and_determinism():
    a = inputs.make_prefill_inputs([100, 0, 37], H=3, d_k=32, d_v=16, dtype="bf16", seed=5)
    b = inputs.make_prefill_inputs([100, 0, 37], H=3, d_k=32, d_v=16, dtype="bf16", seed=5)
    for f in ("q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.cu_seqlens.tolist() == [0, 100, 100, 137]
    assert a.q.shape == (137, 3, 32) and a.v.shape == (137, 3, 16) and a.S0.shape == (3, 3, 32, 16)
    for f in ("q", "k", "v"):
        assert np.all((getattr(a, f).view(np.uint32) & 0xFFFF) == 0), f
    kn = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    qn = np.linalg.norm(a.q.astype(np.float64), axis=-1)
    assert np.allclose(kn, 1.0, atol=1e-2) and np.allclose(qn, 1 / np.sqrt(32), atol=1e-3)
    assert np.all(a.log_alpha <= -0.001) and np.all(a.log_alpha >= -0.1)
    assert np.all(a.beta > 0) and np.all(a.beta < 1)
    assert abs(float(np.std(a.S0)) - 0.01) < 2e-3


def test_fp32_workload_is_unrounded_and_zero_state():
    x = inputs.make_workload("prefill_t256_h2_d32_f32")
    assert x.S0 is None and x.dtype == "f32" and x.T_tot == 256 and x.H == 2
    assert np.any((x.q.view(np.uint32) & 0xFFFF) != 0)


def test_decode_steps_are_independent_streams():
    s0 = inputs.decode_step_inputs(4, 2, 16, 16, step=0)
    s1 = inputs.decode_step_inputs(4, 2, 16, 16, step=1)
    s0b = inputs.decode_step_inputs(4, 2, 16, 16, step=0)
    assert not np.array_equal(s0.q, s1.q)
    assert np.array_equal(s0.q, s0b.q) and np.array_equal(s0.beta, s0b.beta)
    S = inputs.decode_initial_state(4, 2, 16, 16)
    assert S.shape == (4, 2, 16, 16) and S.dtype == np.float32
