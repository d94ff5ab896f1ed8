"""GPU-side properties that need no oracle: determinism, launch-shape
invariance, packing invariance, in-place states, resume, prefill versus
repeated decode steps, linearity, every output written, empty inputs."""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, rel_err, upload, valid_splits

pytestmark = pytest.mark.gpu


def _x(lengths, H=2, dk=128, dv=128, dtype="bf16", seed=3, s0=1.0):
    return inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=seed, s0_std=s0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic_and_split_invariant_bits(dtype):
    import torch
    x = _x([200, 65, 1], dk=64, dv=128, dtype=dtype)
    d = upload(x)
    o0, S0 = kda.prefill(**d, v_split=1)
    for split in valid_splits(128):
        for rep in range(2):
            o, S = kda.prefill(**d, v_split=split)
            assert torch.equal(o, o0) and torch.equal(S, S0), f"v_split={split} rep={rep}"


@pytest.mark.parametrize("lengths", [[100, 0, 130, 64], [9000, 100, 0, 4097], [3000, 3000, 10]],
                         ids=["short", "segmented", "segmented_mid_lengths"])
def test_packing_does_not_change_bits(lengths):
    """A sequence gives the same bits alone or in any batch; in a small
    batch past 1024 tokens the long sequences run in segments, whose length
    depends on the sequence's own length only."""
    import torch
    x = _x(lengths)
    d = upload(x)
    o, S = kda.prefill(**d)
    for n in range(x.N):
        a, b = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        cu = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        on, Sn = kda.prefill(d["q"][a:b].contiguous(), d["k"][a:b].contiguous(), d["v"][a:b].contiguous(),
                             d["log_alpha"][a:b].contiguous(), d["beta"][a:b].contiguous(),
                             d["S0"][n:n + 1].contiguous(), cu)
        assert torch.equal(on, o[a:b]) and torch.equal(Sn[0], S[n]), f"sequence {n}"


def test_paced_batch_keeps_the_bits_of_each_sequence_alone():
    """A batch that fills the GPU (8 sequences x 32 heads, bf16, d = 128) paces
    the loads of its shorter sequences; each sequence alone (32 workgroups,
    unpaced) gives the same bits."""
    import torch
    x = _x([1000, 700, 333, 90, 64, 33, 1, 250], H=32, dk=128, dv=128, seed=17)
    d = upload(x)
    o, S = kda.prefill(**d)
    for n in range(x.N):
        a, b = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        cu = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        on, Sn = kda.prefill(d["q"][a:b].contiguous(), d["k"][a:b].contiguous(), d["v"][a:b].contiguous(),
                             d["log_alpha"][a:b].contiguous(), d["beta"][a:b].contiguous(),
                             d["S0"][n:n + 1].contiguous(), cu)
        assert torch.equal(on, o[a:b]) and torch.equal(Sn[0], S[n]), f"sequence {n}"


@pytest.mark.parametrize("lengths", [[70, 0, 0, 10], [70, 0, 0, 4500]], ids=["short", "segmented"])
def test_in_place_state_and_empty_sequences(lengths):
    import torch
    x = _x(lengths)
    d = upload(x)
    o, S = kda.prefill(**d)
    assert torch.equal(S[1], d["S0"][1]) and torch.equal(S[2], d["S0"][2])
    state = d["S0"].clone()
    o2, S2 = kda.prefill(**dict(d, S0=state), S_T=state)
    assert S2.data_ptr() == state.data_ptr()
    assert torch.equal(o2, o) and torch.equal(state, S)


def test_zero_tokens_copies_state():
    import torch
    dev = "cuda"
    S0 = torch.randn(3, 2, 64, 32, device=dev)
    e = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    o, S = kda.prefill(e(0, 2, 64), e(0, 2, 64), e(0, 2, 32), e(0, 2, 64, dt=torch.float32),
                       e(0, 2, dt=torch.float32), S0, cu)
    assert torch.equal(S, S0)
    o, S = kda.prefill(e(0, 2, 64), e(0, 2, 64), e(0, 2, 32), e(0, 2, 64, dt=torch.float32),
                       e(0, 2, dt=torch.float32), None, cu)
    assert torch.count_nonzero(S) == 0


@pytest.mark.parametrize("lengths", [[1, 63, 64, 65, 127], [1, 4097, 5000, 65]], ids=["short", "segmented"])
def test_every_output_is_written(lengths):
    import torch
    x = _x(lengths, H=3)
    d = upload(x)
    o = torch.full((x.T_tot, 3, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ST = torch.full((x.N, 3, 128, 128), float("nan"), device="cuda")
    kda.prefill(**d, o=o, S_T=ST)
    assert not torch.isnan(o).any() and not torch.isnan(ST).any()


def test_resume_at_chunk_boundary_is_exact_and_anywhere_close():
    import torch
    x = _x([320])
    d = upload(x)
    o, S = kda.prefill(**d)
    for cut in (128, 100):
        sl = lambda t, a, b: t[a:b].contiguous()
        cu1 = torch.tensor([0, cut], dtype=torch.int32, device="cuda")
        cu2 = torch.tensor([0, 320 - cut], dtype=torch.int32, device="cuda")
        o1, S1 = kda.prefill(*(sl(d[f], 0, cut) for f in ("q", "k", "v", "log_alpha", "beta")), d["S0"], cu1)
        o2, S2 = kda.prefill(*(sl(d[f], cut, 320) for f in ("q", "k", "v", "log_alpha", "beta")), S1, cu2)
        oc = torch.cat([o1, o2])
        if cut % 64 == 0:
            assert torch.equal(oc, o) and torch.equal(S2, S), "resume at a chunk boundary"
        else:
            assert rel_err(host(oc), host(o)) < 1e-2 and rel_err(host(S2), host(S)) < 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_equals_repeated_decode(dtype):
    import torch
    T = 150
    x = _x([T], dk=64, dv=64, dtype=dtype)
    d = upload(x)
    o, S = kda.prefill(**d)
    state = d["S0"].clone()
    od = []
    for t in range(T):
        sl = lambda f: d[f][t:t + 1].contiguous()
        od.append(kda.decode_step(sl("q"), sl("k"), sl("v"), sl("log_alpha"), sl("beta"), state))
    od = torch.cat(od)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert rel_err(host(o), host(od)) < tol
    assert rel_err(host(S), host(state)) < tol


def test_state_only_outputs_match_oracle():
    """v = 0 and a unit-scale S0: every output comes from the initial state
    (an S0 mistake cannot hide below the tolerance here)."""
    x = _x([200, 77], s0=1.0, seed=11)
    x.v[:] = 0.0
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, S = kda.prefill(**upload(x))
    assert_close(host(o), ref_o, "bf16", "o (state only)")
    assert_close(host(S), ref_S, "bf16", "S_T (state only)")


def test_linearity_in_state_and_values():
    import torch
    x = _x([190, 40], seed=5)
    d = upload(x)
    o1, S1 = kda.prefill(**d)
    o2, S2 = kda.prefill(**dict(d, S0=None))
    o3, S3 = kda.prefill(**dict(d, v=torch.zeros_like(d["v"])))
    assert rel_err(host(o2) + host(o3), host(o1)) < 2e-2
    assert rel_err(host(S2) + host(S3), host(S1)) < 2e-2


@pytest.mark.parametrize("split", [1, 8])
def test_repeated_long_runs_are_bit_identical(split):
    """The roles of a workgroup hand chunks over through LDS counters; a
    hand-off that let a reader see a tile before every writer finished it
    would show up as run-to-run differences on long sequences (thousands of
    hand-offs per workgroup)."""
    import torch
    x = inputs.make_prefill_inputs([32768], 32, 128, 128, "bf16", seed=31, s0_std=0.1)
    d = upload(x)
    del x
    o0, S0 = kda.prefill(**d, v_split=split)
    for rep in range(6):
        o, S = kda.prefill(**d, v_split=split)
        assert torch.equal(o, o0) and torch.equal(S, S0), f"v_split={split} rep={rep}"


@pytest.mark.parametrize("lengths", [[300, 77], [5000]], ids=["one_pass", "segmented"])
def test_side_stream_gives_the_same_bits(lengths):
    """Prefill (one pass, and segmented with its workspace and default
    cu_seqlens allocated by the binding), backward and decode on a
    non-current stream give the default stream's bits."""
    import torch
    x = _x(lengths)
    d = upload(x)
    dO, dST = inputs.make_backward_grads(x, seed=5)
    gO, gST = torch.from_numpy(dO).cuda().to(torch.bfloat16), torch.from_numpy(dST).cuda()
    single = len(lengths) == 1
    pd = dict(d, cu_seqlens=None) if single else d
    o0, S0 = kda.prefill(**pd)
    g0 = kda.prefill_backward(**d, d_o=gO, d_S_T=gST)
    Sd0 = d["S0"].clone()
    od0 = kda.decode_step(d["q"][:1].expand(x.N, -1, -1).contiguous(), d["k"][:1].expand(x.N, -1, -1).contiguous(),
                          d["v"][:1].expand(x.N, -1, -1).contiguous(),
                          d["log_alpha"][:1].expand(x.N, -1, -1).contiguous(),
                          d["beta"][:1].expand(x.N, -1).contiguous(), Sd0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    dec_in = [t[:1].expand(x.N, *t.shape[1:]).contiguous() for t in (d["q"], d["k"], d["v"], d["log_alpha"])]
    b1 = d["beta"][:1].expand(x.N, -1).contiguous()
    for rep in range(3):
        Sd = d["S0"].clone()  # on the current stream; the side stream waits for it
        side.wait_stream(torch.cuda.current_stream())
        o1, S1 = kda.prefill(**pd, stream=side)
        g1 = kda.prefill_backward(**d, d_o=gO, d_S_T=gST, stream=side)
        od1 = kda.decode_step(*dec_in, b1, Sd, stream=side)
        side.synchronize()
        assert torch.equal(o1, o0) and torch.equal(S1, S0), f"prefill rep {rep}"
        for a, b in zip(g1, g0):
            assert torch.equal(a, b), f"backward rep {rep}"
        assert torch.equal(od1, od0) and torch.equal(Sd, Sd0), f"decode rep {rep}"
