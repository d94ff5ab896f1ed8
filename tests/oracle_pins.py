"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics that
do not re-use the oracle's own code path.

The update rule is the one printed in "Kimi Linear：让长上下文大模型真正实用的
线性注意力架构" (juejin.cn), section 三.5: S_t = (I - b_t k_t k_t^T) Diag(a_t)
S_{t-1} + b_t k_t v_t^T, per-channel a_t (section 三.1), read-out
o_t = S_t^T q_t after the update.

Each pin is a function ``pin_xxx(lib)`` that raises AssertionError when the
oracle build ``lib`` disagrees.  ``run_all`` runs every pin and returns the
names of those that failed; ``tests/test_oracle_mutants.py`` uses it to show
that planted mistakes in the oracle's C source are caught.
"""
from __future__ import annotations

import numpy as np

import oracle

_RTOL = 1e-10
_ATOL = 1e-12


def _close(a, b, what, rtol=_RTOL, atol=_ATOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= atol + rtol * scale, f"{what}: max abs err {err:.3e}"


def _random_case(rng, lengths, H, dk, dv, s0=True, la_hi=1.0):
    """Generic (not normalised) small inputs, exactly representable in fp32."""
    lengths = list(lengths)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    q = f(T, H, dk) / np.float32(np.sqrt(dk))
    k = f(T, H, dk) / np.float32(np.sqrt(dk))
    v = f(T, H, dv)
    la = (-la_hi * rng.random((T, H, dk))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) if s0 else None
    return q, k, v, la, beta, S0, cu


# --------------------------------------------------------------------------
# I0: brute-force expansion of the matrix product (independent formula)
# --------------------------------------------------------------------------
def _bruteforce(q, k, v, la, beta, S0, cu):
    """S_t = A_t...A_1 S0 + sum_s A_t...A_{s+1} b_s k_s v_s^T with explicit
    d_k x d_k transition matrices A_t = (I - b_t k_t k_t^T) Diag(a_t)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else S0[n, h].astype(np.float64)
            ts = list(range(cu[n], cu[n + 1]))
            A = []
            for t in ts:
                kt = k[t, h].astype(np.float64)[:, None]
                A.append((np.eye(dk) - float(beta[t, h]) * (kt @ kt.T))
                         @ np.diag(np.exp(la[t, h].astype(np.float64))))
            S = s0
            for a_idx, t in enumerate(ts):
                P = np.eye(dk)
                for j in range(a_idx, -1, -1):
                    P = P @ A[j]
                S = P @ s0
                for s_idx in range(a_idx + 1):
                    P = np.eye(dk)
                    for j in range(a_idx, s_idx, -1):
                        P = P @ A[j]
                    ks = k[ts[s_idx], h].astype(np.float64)[:, None]
                    vs = v[ts[s_idx], h].astype(np.float64)[None, :]
                    S = S + float(beta[ts[s_idx], h]) * (P @ ks @ vs)
                o[t, h] = S.T @ q[t, h].astype(np.float64)
            ST[n, h] = S
    return o, ST


def pin_bruteforce_product(lib):
    rng = np.random.default_rng(100)
    # d_k != d_v catches a transposed state; an empty sequence and H=2 catch
    # offset and head-stride mistakes.
    case = _random_case(rng, [5, 0, 8, 3], H=2, dk=5, dv=3)
    o, ST = oracle.prefill(*case, lib=lib)
    ob, STb = _bruteforce(*case)
    _close(o, ob, "o vs brute force")
    _close(ST, STb, "S_T vs brute force")


# --------------------------------------------------------------------------
# Special cases named on the pages
# --------------------------------------------------------------------------
def pin_deltanet_when_alpha_is_one(lib):
    """alpha == 1 (log alpha = 0): the ungated delta rule (DeltaNet, page
    section 三.5), S <- (I - b k k^T) S + b k v^T, applied as matrices."""
    rng = np.random.default_rng(101)
    q, k, v, la, beta, S0, cu = _random_case(rng, [20], H=1, dk=6, dv=4)
    la[:] = 0.0
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    S = S0[0, 0].copy()
    for t in range(20):
        kt = k[t, 0].astype(np.float64)[:, None]
        S = (np.eye(6) - beta[t, 0] * kt @ kt.T) @ S + beta[t, 0] * kt @ v[t, 0][None, :].astype(np.float64)
        _close(o[t, 0], S.T @ q[t, 0].astype(np.float64), f"o[{t}]")
    _close(ST[0, 0], S, "S_T")


def pin_gated_deltanet_scalar_gate(lib):
    """alpha_t[i] == a_t for every channel: Gated DeltaNet (one forgetting rate
    per head, page section 三.1), S_t = a_t (I - b k k^T) S_{t-1} + b k v^T,
    written as matrices; checks the oracle's scalar-gate entry points
    (prefill over two sequences and decode steps)."""
    rng = np.random.default_rng(102)
    lengths = [20, 7]
    q, k, v, la, beta, S0, cu = _random_case(rng, lengths, H=2, dk=4, dv=5)
    la2 = np.ascontiguousarray(la[:, :, 0])
    o, ST = oracle.gdn_prefill(q, k, v, la2, beta, S0, cu, lib=lib)
    for n in range(2):
        for h in range(2):
            S = S0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                a = np.exp(np.float64(la2[t, h]))
                kt = k[t, h].astype(np.float64)[:, None]
                S = a * ((np.eye(4) - beta[t, h] * kt @ kt.T) @ S) + beta[t, h] * kt @ v[t, h][None, :].astype(np.float64)
                _close(o[t, h], S.T @ q[t, h].astype(np.float64), f"o[{t},{h}]")
            _close(ST[n, h], S, f"S_T[{n},{h}]")
    # decode: the first 5 tokens of sequence 0 as steps of a batch of one
    S = S0[:1].copy()
    for t in range(5):
        od = oracle.gdn_decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], la2[t:t + 1], beta[t:t + 1], S, lib=lib)
        _close(od[0], o[t], f"decode o[{t}]")


def pin_exact_retrieval(lib):
    """||k_t|| = 1 and b_t = 1: one gradient step of size 1 on
    1/2||S^T k - v||^2 reaches the minimum, so k_t^T S_t = v_t^T exactly
    (page section 三.5, 'Attention as Learning').  With q_t = k_t the
    read-out after the update returns v_t."""
    rng = np.random.default_rng(103)
    T, dk, dv = 24, 16, 7
    k = (0.25 * rng.choice([-1.0, 1.0], size=(T, 1, dk))).astype(np.float32)  # ||k|| = 1 exactly
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    la = (-rng.random((T, 1, dk))).astype(np.float32)
    beta = np.ones((T, 1), np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    cu = np.array([0, T], np.int32)
    o, _ = oracle.prefill(k, k, v, la, beta, S0, cu, lib=lib)
    _close(o[:, 0], v[:, 0], "k_t^T S_t vs v_t")


def pin_beta_zero_closed_form(lib):
    """b == 0: the state only decays, S_t = Diag(exp(sum_{s<=t} log a_s)) S0
    and o_t = S_t^T q_t."""
    rng = np.random.default_rng(104)
    q, k, v, la, beta, S0, cu = _random_case(rng, [7, 0, 12], H=2, dk=5, dv=3)
    beta[:] = 0.0
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    for n in range(3):
        for h in range(2):
            g = np.zeros(5)
            for t in range(cu[n], cu[n + 1]):
                g += la[t, h].astype(np.float64)
                St = np.exp(g)[:, None] * S0[n, h]
                _close(o[t, h], St.T @ q[t, h].astype(np.float64), f"o[{t},{h}]")
            _close(ST[n, h], np.exp(g)[:, None] * S0[n, h], f"S_T[{n},{h}]")


def pin_beta_zero_alpha_one(lib):
    """b == 0 and a == 1: S stays S0 and o_t = S0^T q_t (a plain mat-vec)."""
    rng = np.random.default_rng(105)
    q, k, v, la, beta, S0, cu = _random_case(rng, [9], H=1, dk=6, dv=6)
    beta[:] = 0.0
    la[:] = 0.0
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    _close(o[:, 0], q[:, 0].astype(np.float64) @ S0[0, 0], "o")
    assert np.array_equal(ST, S0), "S_T must equal S0 exactly"


def pin_one_hot_key_value_table(lib):
    """One-hot keys k_t = e_{i_t}, b = 1, a = 1: each token overwrites row i_t
    of S with v_t, so S is a key-value table."""
    rng = np.random.default_rng(106)
    T, dk, dv = 30, 8, 5
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((T, 1, dk), np.float32)
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk)).astype(np.float32)
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    la = np.zeros((T, 1, dk), np.float32)
    beta = np.ones((T, 1), np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.prefill(q, k, v, la, beta, S0, np.array([0, T], np.int32), lib=lib)
    table = S0[0, 0].copy()
    for t in range(T):
        table[idx[t]] = v[t, 0]
        _close(o[t, 0], q[t, 0].astype(np.float64) @ table, f"o[{t}]")
    _close(ST[0, 0], table, "S_T")


def pin_scalar_recurrence(lib):
    """d_k = d_v = 1: s_t = a_t (1 - b_t k_t^2) s_{t-1} + b_t k_t v_t, o_t = q_t s_t."""
    rng = np.random.default_rng(107)
    T = 40
    q, k, v = (rng.standard_normal((T, 1, 1)).astype(np.float32) for _ in range(3))
    la = (-rng.random((T, 1, 1))).astype(np.float32)
    beta = rng.random((T, 1)).astype(np.float32)
    S0 = np.array([[[[0.7]]]])
    o, ST = oracle.prefill(q, k, v, la, beta, S0, np.array([0, T], np.int32), lib=lib)
    s = 0.7
    for t in range(T):
        a = np.exp(np.float64(la[t, 0, 0]))
        kk = np.float64(k[t, 0, 0])
        b = np.float64(beta[t, 0])
        s = a * (1.0 - b * kk * kk) * s + b * kk * np.float64(v[t, 0, 0])
        _close(o[t, 0, 0], np.float64(q[t, 0, 0]) * s, f"o[{t}]")
    _close(ST[0, 0, 0, 0], s, "S_T")


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def pin_linearity_in_state_and_values(lib):
    """For fixed q, k, gates and b, (S0, V) -> (O, S_T) is linear."""
    rng = np.random.default_rng(108)
    q, k, v, la, beta, S0, cu = _random_case(rng, [11, 6], H=2, dk=4, dv=3)
    o1, S1 = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    o2, S2 = oracle.prefill(q, k, v, la, beta, None, cu, lib=lib)
    o3, S3 = oracle.prefill(q, k, np.zeros_like(v), la, beta, S0, cu, lib=lib)
    _close(o1, o2 + o3, "o additivity")
    _close(S1, S2 + S3, "S_T additivity")
    o4, S4 = oracle.prefill(q, k, np.float32(2.0) * v, la, beta, 2.0 * S0, cu, lib=lib)
    _close(o4, 2.0 * o1, "o homogeneity")
    _close(S4, 2.0 * S1, "S_T homogeneity")


def pin_norm_bound(lib):
    """||k|| <= 1, b in [0,1], a <= 1: (I - b k k^T) and Diag(a) are
    contractions, so ||S_t||_2 <= ||S_{t-1}||_2 + b_t ||v_t||_2."""
    rng = np.random.default_rng(109)
    dk, dv = 6, 5
    S = np.ascontiguousarray(rng.standard_normal((1, 1, dk, dv)))
    for step in range(30):
        kk = rng.standard_normal((1, 1, dk))
        kk = (kk / np.linalg.norm(kk) * rng.random()).astype(np.float32)
        q = rng.standard_normal((1, 1, dk)).astype(np.float32)
        v = rng.standard_normal((1, 1, dv)).astype(np.float32)
        la = (-rng.random((1, 1, dk))).astype(np.float32)
        b = rng.random((1, 1)).astype(np.float32)
        before = np.linalg.norm(S[0, 0], 2)
        oracle.decode_step(q, kk, v, la, b, S, lib=lib)
        after = np.linalg.norm(S[0, 0], 2)
        assert after <= before + float(b[0, 0]) * np.linalg.norm(v) + 1e-12, f"step {step}"


def pin_varlen_equals_separate_sequences(lib):
    """No state crosses a cu_seqlens boundary: a packed batch equals its
    sequences run one by one, bit for bit."""
    rng = np.random.default_rng(110)
    q, k, v, la, beta, S0, cu = _random_case(rng, [4, 0, 9, 1], H=2, dk=3, dv=4)
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.prefill(q[a:b], k[a:b], v[a:b], la[a:b], beta[a:b], S0[n:n + 1],
                                np.array([0, b - a], np.int32), lib=lib)
        assert np.array_equal(on, o[a:b]) and np.array_equal(Sn, ST[n:n + 1]), f"sequence {n}"


def pin_decode_steps_equal_prefill(lib):
    rng = np.random.default_rng(111)
    q, k, v, la, beta, S0, cu = _random_case(rng, [13], H=3, dk=4, dv=2)
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    S = np.ascontiguousarray(S0.copy())
    for t in range(13):
        ot = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1],
                                beta[t:t + 1], S, lib=lib)
        assert np.array_equal(ot[0], o[t]), f"token {t}"
    assert np.array_equal(S, ST)


def pin_resume_from_state(lib):
    """prefill(T1) then prefill(T2, S0 = S_T1) == prefill(T1 + T2)."""
    rng = np.random.default_rng(112)
    q, k, v, la, beta, S0, cu = _random_case(rng, [17], H=2, dk=5, dv=5)
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    o1, S1 = oracle.prefill(q[:7], k[:7], v[:7], la[:7], beta[:7], S0, np.array([0, 7], np.int32), lib=lib)
    o2, S2 = oracle.prefill(q[7:], k[7:], v[7:], la[7:], beta[7:], S1, np.array([0, 10], np.int32), lib=lib)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(S2, ST)


def pin_zero_state_and_empty_sequences(lib):
    """S0 = NULL is the zero state; an empty sequence returns S0 unchanged;
    a pair mask computes exactly the selected pairs; the thread count does
    not change any bit."""
    rng = np.random.default_rng(113)
    q, k, v, la, beta, S0, cu = _random_case(rng, [6, 0, 5], H=2, dk=4, dv=4)
    o0, S_0 = oracle.prefill(q, k, v, la, beta, None, cu, lib=lib)
    oz, S_z = oracle.prefill(q, k, v, la, beta, np.zeros_like(S0), cu, lib=lib)
    assert np.array_equal(o0, oz) and np.array_equal(S_0, S_z)
    o1, S1 = oracle.prefill(q, k, v, la, beta, S0, cu, nthreads=1, lib=lib)
    assert np.array_equal(S1[1], S0[1]), "empty sequence must return S0"
    o5, S5 = oracle.prefill(q, k, v, la, beta, S0, cu, nthreads=5, lib=lib)
    assert np.array_equal(o1, o5) and np.array_equal(S1, S5)
    mask = np.zeros((3, 2), bool)
    mask[2, 1] = True
    om, Sm = oracle.prefill(q, k, v, la, beta, S0, cu, pair_mask=mask, lib=lib)
    assert np.array_equal(om[cu[2]:cu[3], 1], o1[cu[2]:cu[3], 1])
    assert np.array_equal(Sm[2, 1], S1[2, 1])
    assert np.all(np.isnan(Sm[0, 0]))


def pin_segments_compose(lib):
    """Linearity in (S0, V) over a split sequence: a later segment run from
    the zero state gives o0 and D; the same segment with V = 0 and S0 = I
    gives q^_t = M_t^T q_t as outputs and the transition M as final state;
    then o_t = o0_t + S_in^T q^_t and S_out = M S_in + D chain the segments
    back into the one-pass result (the decomposition of the segmented GPU
    prefill)."""
    rng = np.random.default_rng(114)
    d = 5
    q, k, v, la, beta, S0, cu = _random_case(rng, [23], H=2, dk=d, dv=d)
    o, ST = oracle.prefill(q, k, v, la, beta, S0, cu, lib=lib)
    cuts = [0, 6, 15, 23]
    eye = np.broadcast_to(np.eye(d), (1, 2, d, d)).copy()
    S_in = None
    for s in range(len(cuts) - 1):
        a, b = cuts[s], cuts[s + 1]
        sl = lambda x: np.ascontiguousarray(x[a:b])
        seg = np.array([0, b - a], np.int32)
        if s == 0:
            o_s, S_in = oracle.prefill(sl(q), sl(k), sl(v), sl(la), sl(beta), S0, seg, lib=lib)
        else:
            o0, D = oracle.prefill(sl(q), sl(k), sl(v), sl(la), sl(beta), None, seg, lib=lib)
            qh, M = oracle.prefill(sl(q), sl(k), np.zeros_like(sl(v)), sl(la), sl(beta), eye, seg, lib=lib)
            o_s = o0 + np.einsum("thi,hij->thj", qh, S_in[0])
            S_in = np.einsum("hij,hjk->hik", M[0], S_in[0])[None] + D
        _close(o_s, o[a:b], f"o of segment {s}")
    _close(S_in, ST, "S_T")


# --------------------------------------------------------------------------
# Backward pass: finite differences of the forward, and a closed form
# --------------------------------------------------------------------------
def _loss_grad_case(rng, lengths, H, dk, dv):
    q, k, v, la, beta, S0, cu = _random_case(rng, lengths, H, dk, dv, la_hi=0.5)
    Ro = rng.standard_normal((int(cu[-1]), H, dv))
    RS = rng.standard_normal((len(lengths), H, dk, dv))
    return q, k, v, la, beta, S0, cu, Ro, RS


def pin_backward_finite_differences(lib):
    """Each gradient of L = sum(o * Ro) + sum(S_T * RS) equals the central
    difference of the (separately pinned) forward.  The fp32 inputs are
    perturbed by h and the difference is divided by the step actually taken.
    Lengths include an empty sequence and one longer than the 64-token block
    the backward recomputes states in."""
    rng = np.random.default_rng(71)
    for lengths, H, dk, dv in (([4, 0, 3], 2, 3, 2), ([70], 1, 2, 2)):
        q, k, v, la, beta, S0, cu, Ro, RS = _loss_grad_case(rng, lengths, H, dk, dv)
        grads = oracle.prefill_backward(q, k, v, la, beta, S0, cu, Ro, RS, lib=lib)
        args = [q, k, v, la, beta]

        def loss(a, s0):
            o, ST = oracle.prefill(*a, s0, cu, lib=lib)
            return float((o * Ro).sum() + (ST * RS).sum())

        for ai, name in enumerate(("dq", "dk", "dv", "dlog_alpha", "dbeta")):
            x = args[ai]
            fd = np.zeros(x.shape)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += np.float32(2.0 ** -10)
                xm[idx] -= np.float32(2.0 ** -10)
                ap, am = list(args), list(args)
                ap[ai], am[ai] = xp, xm
                fd[idx] = (loss(ap, S0) - loss(am, S0)) / (float(xp[idx]) - float(xm[idx]))
            _close(grads[ai], fd, f"{name} vs finite differences {lengths}", rtol=2e-5, atol=1e-7)
        fd = np.zeros(S0.shape)
        for idx in np.ndindex(S0.shape):
            sp, sm = S0.copy(), S0.copy()
            sp[idx] += 1e-6
            sm[idx] -= 1e-6
            fd[idx] = (loss(args, sp) - loss(args, sm)) / 2e-6
        _close(grads[5], fd, f"dS0 vs finite differences {lengths}", rtol=1e-7, atol=1e-8)


def pin_gdn_backward_finite_differences(lib):
    """Gated DeltaNet (one forgetting rate per head, page section 三.1): every
    gradient of L = sum(o * Ro) + sum(S_T * RS) through ``gdn_prefill``
    equals the central difference of that (separately pinned) forward.  The
    gate gradient is taken with respect to the one [T, H] log gate, so a
    gate gradient that averages the channels, or keeps only one of them,
    fails here.  Two sequences and an empty one, H = 2, d_k != d_v."""
    rng = np.random.default_rng(73)
    lengths, H, dk, dv = [4, 0, 3], 2, 3, 2
    q, k, v, la, beta, S0, cu, Ro, RS = _loss_grad_case(rng, lengths, H, dk, dv)
    la2 = np.ascontiguousarray(la[:, :, 0])
    grads = oracle.gdn_prefill_backward(q, k, v, la2, beta, S0, cu, Ro, RS, lib=lib)
    shapes = [q.shape, k.shape, v.shape, la2.shape, beta.shape, S0.shape]
    for g, sh, name in zip(grads, shapes, ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")):
        assert np.asarray(g).shape == tuple(sh), f"{name}: shape {np.asarray(g).shape} vs {sh}"
    args = [q, k, v, la2, beta]

    def loss(a, s0):
        o, ST = oracle.gdn_prefill(*a, s0, cu, lib=lib)
        return float((o * Ro).sum() + (ST * RS).sum())

    for ai, name in enumerate(("dq", "dk", "dv", "dlog_alpha", "dbeta")):
        x = args[ai]
        fd = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += np.float32(2.0 ** -10)
            xm[idx] -= np.float32(2.0 ** -10)
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd[idx] = (loss(ap, S0) - loss(am, S0)) / (float(xp[idx]) - float(xm[idx]))
        _close(grads[ai], fd, f"gdn {name} vs finite differences", rtol=2e-5, atol=1e-7)
    fd = np.zeros(S0.shape)
    for idx in np.ndindex(S0.shape):
        sp, sm = S0.copy(), S0.copy()
        sp[idx] += 1e-6
        sm[idx] -= 1e-6
        fd[idx] = (loss(args, sp) - loss(args, sm)) / 2e-6
    _close(grads[5], fd, "gdn dS0 vs finite differences", rtol=1e-7, atol=1e-8)


def pin_backward_frozen_state_closed_form(lib):
    """beta = 0 and alpha = 1 freeze the state at S0, so o_t = S0^T q_t and the
    gradient reaching S_t is G_t = dS_T + sum over tau >= t of q_tau do_tau^T.
    Then dq_t = S0 do_t, dk = dv = 0, dbeta_t = k_t^T G_t (v_t - S0^T k_t),
    dlog_alpha_t[i] = sum_j G_t[i, j] S0[i, j] and dS0 = G at the first token."""
    rng = np.random.default_rng(72)
    q, k, v, la, beta, S0, cu, Ro, RS = _loss_grad_case(rng, [5, 3], 2, 4, 3)
    beta = np.zeros_like(beta)
    la = np.zeros_like(la)
    dq, dk, dv, dla, db, dS0 = oracle.prefill_backward(q, k, v, la, beta, S0, cu, Ro, RS, lib=lib)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(q.shape[1]):
            S = S0[n, h]
            G = RS[n, h].copy()
            for t in range(b - 1, a - 1, -1):
                G = G + np.outer(q[t, h], Ro[t, h])
                _close(dq[t, h], S @ Ro[t, h], "dq")
                _close(db[t, h], k[t, h] @ G @ (v[t, h] - S.T @ k[t, h]), "dbeta")
                _close(dla[t, h], (G * S).sum(axis=1), "dlog_alpha")
            _close(dS0[n, h], G, "dS0")
    _close(dk, np.zeros_like(dk), "dk")
    _close(dv, np.zeros_like(dv), "dv")


PINS = [
    pin_segments_compose,
    pin_bruteforce_product,
    pin_deltanet_when_alpha_is_one,
    pin_gated_deltanet_scalar_gate,
    pin_exact_retrieval,
    pin_beta_zero_closed_form,
    pin_beta_zero_alpha_one,
    pin_one_hot_key_value_table,
    pin_scalar_recurrence,
    pin_linearity_in_state_and_values,
    pin_norm_bound,
    pin_varlen_equals_separate_sequences,
    pin_decode_steps_equal_prefill,
    pin_resume_from_state,
    pin_zero_state_and_empty_sequences,
    pin_backward_finite_differences,
    pin_gdn_backward_finite_differences,
    pin_backward_frozen_state_closed_form,
]


def run_all(lib):
    """Run every pin against ``lib``; return the names of the pins that failed."""
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    return failed
