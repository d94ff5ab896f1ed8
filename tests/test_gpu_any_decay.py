"""KDA_PREFILL_ANY_DECAY: the prefill with no decay-range contract, on both of
its kernels: the chunked kernel over chunk lists (a token whose log alpha is
below -5 on some channel starts a chunk; the path taken when a workspace is
given) and the token-recurrent kernel (``token_recurrent=True``: no
workspace).

Gates from -U(0, 5) plus strong tokens of every kind: hard resets (log alpha
-1000, -1e30 and -3e38 on every channel: alpha underflows to 0 in fp32 and in
the fp64 oracle alike), a single strongly decaying channel, values just past
the -5 threshold, runs of consecutive strong tokens, strong tokens at a
sequence's first and last token and at multiples of the chunk length.  Both
kernels against the oracle, per-channel and per-head gates; the chunk lists
against their definition (integers, exact); and on gates within the default
contract the chunked any-decay path gives the bits of the default kernel.
"""
import numpy as np
import pytest

import gated_delta_rule_60_amd as kda
import oracle
from gated_delta_rule_60_amd import inputs
from gpu_util import assert_close, host, log, upload

pytestmark = pytest.mark.gpu

PATHS = ["chunked", "recurrent"]

CASES = [
    # lengths, H, d_k, d_v, dtype
    ([90, 0, 45], 2, 128, 128, "bf16"),
    ([300, 33], 2, 128, 128, "bf16"),
    ([70, 33], 2, 64, 32, "f32"),
    ([64, 17], 3, 32, 64, "f32"),
    ([130, 95], 2, 128, 64, "f32"),
    ([257], 1, 64, 128, "bf16"),
]


def _strong(lengths, H, dk, dv, dtype, seed, density=0.05):
    """-U(0, 5) gates with strong tokens planted at fixed and seeded rows."""
    x = inputs.make_prefill_inputs(lengths, H, dk, dv, dtype, seed=seed, s0_std=1.0, log_alpha_range=(0.0, 5.0))
    rng = np.random.default_rng(seed + 1000)
    la = x.log_alpha
    cu = x.cu_seqlens
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        fixed = [a, a + 1, a + 2, a + 32, a + 48, a + 49, b - 1]  # first rows, chunk multiples, a run, the last
        rows = sorted({r for r in fixed if a <= r < b} | {int(r) for r in np.nonzero(rng.random(b - a) < density)[0] + a})
        for i, r in enumerate(rows):
            kind = (i + n) % 6
            h = int(rng.integers(H))
            if kind == 0:
                la[r] = -1000.0                                         # reset, every head
            elif kind == 1:
                la[r, h] = -1e30                                        # reset of one head
            elif kind == 2:
                la[r, h, int(rng.integers(dk))] = -rng.uniform(5.5, 80.0)  # one channel
            elif kind == 3:
                la[r, h] = -rng.uniform(5.01, 30.0, size=dk)            # every channel of one head
            elif kind == 4:
                la[r, h, : dk // 2] = -5.001                            # just past the threshold
            else:
                la[r, h] = -3e38                                        # near the fp32 limit
    return x


def _run(d, path, scalar_gate=False, **kw):
    run = kda.gdn_prefill_t if scalar_gate else kda.prefill
    return run(**d, any_decay=True, token_recurrent=(path == "recurrent"), **kw)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{'-'.join(map(str, c[0]))}_H{c[1]}_dk{c[2]}_dv{c[3]}_{c[4]}")
def test_any_decay_matches_oracle(case, path):
    import torch
    lengths, H, dk, dv, dtype = case
    x = _strong(lengths, H, dk, dv, dtype, seed=sum(lengths) + dk)
    log(f"  oracle {lengths} dk={dk} dv={dv} {dtype}, {path}")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = _run(upload(x), path)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, dtype, "o")
    assert_close(host(ST), ref_S, dtype, "S_T")


@pytest.mark.parametrize("path", PATHS)
def test_any_decay_every_token_strong(path):
    """Every token a strong one: one chunk per token on the chunked path."""
    import torch
    x = inputs.make_prefill_inputs([40, 7], 2, 64, 64, "f32", seed=21, s0_std=1.0, log_alpha_range=(5.5, 9.0))
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = _run(upload(x), path)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, "f32", "o")
    assert_close(host(ST), ref_S, "f32", "S_T")


@pytest.mark.parametrize("path", PATHS)
def test_any_decay_many_sequences(path):
    """70 ragged sequences (past the in-kernel length ordering) and enough
    pairs for whole value columns per workgroup."""
    import torch
    rng = np.random.default_rng(31)
    lengths = [int(v) for v in rng.integers(0, 90, size=70)]
    x = _strong(lengths, 2, 64, 128, "bf16", seed=31, density=0.08)
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens)
    o, ST = _run(upload(x), path)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, "bf16", "o")
    assert_close(host(ST), ref_S, "bf16", "S_T")


@pytest.mark.parametrize("path", PATHS)
def test_any_decay_scalar_gate_matches_oracle(path):
    import torch
    x = _strong([80, 40, 130], 2, 128, 64, "bf16", seed=8)
    la = np.ascontiguousarray(x.log_alpha.min(axis=2))
    ref_o, ref_S = oracle.gdn_prefill(x.q, x.k, x.v, la, x.beta, x.S0, x.cu_seqlens)
    d = upload(x)
    o, ST = _run(dict(d, log_alpha=torch.from_numpy(la).cuda()), path, scalar_gate=True)
    torch.cuda.synchronize()
    assert_close(host(o), ref_o, "bf16", "o")
    assert_close(host(ST), ref_S, "bf16", "S_T")


def _expected_starts(strong, a, b, C):
    """Chunk starts of tokens a..b-1 by their definition: t starts a chunk
    when (t - A(t)) mod C == 0, A(t) the last anchor (a, or a strong token)
    at or before t."""
    out, anchor = [], a
    for t in range(a, b):
        if strong[t]:
            anchor = t
        if (t - anchor) % C == 0:
            out.append(t)
    return out


@pytest.mark.parametrize("scalar_gate", [False, True])
@pytest.mark.parametrize("dtype,dk,C", [("bf16", 64, 32), ("f32", 128, 16)])
def test_chunk_lists_follow_their_definition(dtype, dk, C, scalar_gate):
    """The planning kernel's lists (read back from the workspace: counts
    [N H] int32, then at the next 256-byte boundary the starts, pair (n, h)
    at h (T + 2 N) + cu[n] + 2 n) equal the definition, exactly.  C is the
    prefill's chunk length for the dtype and d_k."""
    import torch
    lengths = [300, 0, 1, 77, 520]
    H = 3
    x = _strong(lengths, H, dk, 64, dtype, seed=44, density=0.04)
    la = np.ascontiguousarray(x.log_alpha.min(axis=2)) if scalar_gate else x.log_alpha
    d = upload(x)
    if scalar_gate:
        d["log_alpha"] = torch.from_numpy(la).cuda()
    N, T = len(lengths), int(x.cu_seqlens[-1])
    flags = kda.KDA_PREFILL_ANY_DECAY | (kda.KDA_PREFILL_SCALAR_GATE if scalar_gate else 0)
    code = kda.KDA_DTYPE_BF16 if dtype == "bf16" else kda.KDA_DTYPE_F32
    ws_bytes = kda.kda_prefill_workspace_size_ex(N, T, H, dk, 64, code, flags)
    ws = torch.full((ws_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    _run(d, "chunked", scalar_gate=scalar_gate, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    off = (4 * N * H + 255) // 256 * 256
    counts = raw[: 4 * N * H].view(np.int32).reshape(N, H)
    starts = raw[off: off + 4 * H * (T + 2 * N)].view(np.int32)
    strong = (la < -5.0) if scalar_gate else (la < -5.0).any(axis=2)  # [T, H]
    cu = x.cu_seqlens
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            exp = _expected_starts(strong[:, h], a, b, C)
            base = h * (T + 2 * N) + a + 2 * n
            got = starts[base: base + counts[n, h] + 1]
            assert counts[n, h] == len(exp), (n, h, counts[n, h], len(exp))
            assert list(got[:-1]) == exp, (n, h)
            assert got[-1] == b, (n, h)


@pytest.mark.parametrize("la_range", [(0.001, 0.1), (0.0, 2.5)])
def test_chunked_any_decay_keeps_the_default_bits(la_range):
    """Gates within the default contract: no strong token, the same chunks,
    and the any-decay path gives exactly the default kernel's bits."""
    import torch
    x = inputs.make_prefill_inputs([300, 31, 0, 64, 650], 2, 128, 128, "bf16", seed=9, s0_std=1.0,
                                   log_alpha_range=la_range)
    d = upload(x)
    o_ref, S_ref = kda.prefill(**d)
    o, ST = _run(d, "chunked")
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(ST, S_ref)


@pytest.mark.parametrize("path", PATHS)
def test_any_decay_in_place_state(path):
    """S_T may be S0 itself (state updated in place); ordinary gates agree
    with the default chunked kernel to the tolerance."""
    import torch
    x = inputs.make_prefill_inputs([200, 31], 2, 128, 128, "bf16", seed=9, s0_std=1.0)
    d = upload(x)
    o_ref, S_ref = kda.prefill(**d)
    S = d["S0"].clone()
    o, ST = _run(dict(d, S0=S), path, S_T=S)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    assert_close(host(o), host(o_ref), "bf16", "o vs chunked")
    assert_close(host(S), host(S_ref), "bf16", "S_T vs chunked")


def test_any_decay_full_batch_sampled_heads():
    """The 32k-token batch of eight sequences, 32 heads, with -U(0, 5) gates
    and resets (the any-decay benchmark's inputs), chunked path; the oracle on
    three heads of every sequence."""
    import torch
    x = inputs.make_any_decay_workload()
    heads = [0, 17, 31]
    mask = np.zeros((x.N, x.H), bool)
    mask[:, heads] = True
    log(f"  oracle on heads {heads} of all {x.N} sequences")
    ref_o, ref_S = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens, pair_mask=mask)
    o, ST = _run(upload(x), "chunked")
    torch.cuda.synchronize()
    o, ST = host(o), host(ST)
    assert_close(o[:, heads], ref_o[:, heads], "bf16", "o (sampled heads)")
    assert_close(ST[:, heads], ref_S[:, heads], "bf16", "S_T (sampled heads)")


@pytest.mark.parametrize("path", PATHS)
def test_any_decay_all_sequences_empty(path):
    """T_tot = 0: no flag work, every list empty; S_T equals S0 exactly."""
    import torch
    x = inputs.make_prefill_inputs([0, 0, 0], 2, 64, 64, "bf16", seed=5, s0_std=1.0)
    d = upload(x)
    o, ST = _run(d, path)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(ST, d["S0"])
