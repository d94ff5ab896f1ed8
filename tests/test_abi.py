"""The C ABI of libkda.so on the CPU: every symbol of include/kda.h is
exported, and every invalid-argument path returns its status before any HIP
call (no kernel is launched here)."""
import os
import re

import pytest

import gated_delta_rule_60_amd as kda
from gated_delta_rule_60_amd import _lib

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
BF16, F32 = kda.KDA_DTYPE_BF16, kda.KDA_DTYPE_F32


def _declared_functions():
    text = open(os.path.join(_ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("kda_prefill", "kda_decode_step", "kda_prefill_workspace_size",
                     "kda_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = kda.load()
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in kda.h but not exported"
        assert name in _lib.SIGNATURES, f"{name} has no binding in _lib.py"


def test_status_strings_and_version():
    assert kda.kda_version() == 6
    for s in (0, 1, 2, 3):
        assert kda.kda_status_string(s).startswith("KDA_")
    assert "unknown" in kda.kda_status_string(99)


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, o=FAKE, S_T=FAKE, workspace=None,
             workspace_bytes=0, v_split=0, stream=None)
    a.update(kw)
    return kda.kda_prefill_split(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARG, "N >= 1"),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG, "H >= 1"),
    (dict(T_tot=-1), kda.KDA_ERR_INVALID_ARG, "T_tot"),
    (dict(d_k=48), kda.KDA_ERR_UNSUPPORTED, "d_k and d_v"),
    (dict(d_v=256), kda.KDA_ERR_UNSUPPORTED, "d_k and d_v"),
    (dict(dtype=7), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(cu_seqlens=None), kda.KDA_ERR_INVALID_ARG, "cu_seqlens"),
    (dict(S_T=None), kda.KDA_ERR_INVALID_ARG, "S_T"),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG, "must not be NULL"),
    (dict(beta=None), kda.KDA_ERR_INVALID_ARG, "must not be NULL"),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG, "must not be NULL"),
    (dict(k=FAKE + 4), kda.KDA_ERR_INVALID_ARG, "aligned"),
    (dict(S0=FAKE + 8), kda.KDA_ERR_INVALID_ARG, "aligned"),
    (dict(v_split=3), kda.KDA_ERR_INVALID_ARG, "v_split"),
    (dict(v_split=8), kda.KDA_ERR_INVALID_ARG, "v_split"),  # 64 / 8 < 16
    (dict(T_tot=2**31), kda.KDA_ERR_INVALID_ARG, "int32"),
    (dict(T_tot=1, H=2**20 // 64 + 1), kda.KDA_ERR_INVALID_ARG, "2^20"),
    # a batch that may hold a segmented (> 1024-token) sequence needs a workspace
    (dict(T_tot=8192), kda.KDA_ERR_INVALID_ARG, "workspace smaller"),
    (dict(T_tot=8192, workspace_bytes=1 << 40), kda.KDA_ERR_INVALID_ARG, "workspace must not be NULL"),
    (dict(T_tot=8192, workspace=FAKE + 16, workspace_bytes=1 << 40), kda.KDA_ERR_INVALID_ARG, "256-byte"),
])
def test_prefill_rejects_invalid_arguments(kw, status, needle):
    assert _prefill(**kw) == status
    assert needle in kda.kda_last_error()


def test_prefill_entry_point_validates_too():
    rc = kda.kda_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 10, 1, 32, 100, BF16, FAKE,
                         FAKE, None, 0, None)
    assert rc == kda.KDA_ERR_UNSUPPORTED


def test_prefill_ex_rejects_unknown_flags():
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, o=FAKE, S_T=FAKE, workspace=None,
             workspace_bytes=0, v_split=0, stream=None)
    for unknown in (8, 16, 1 << 31):
        assert kda.kda_prefill_ex(flags=unknown, **a) == kda.KDA_ERR_INVALID_ARG
        assert "flags" in kda.kda_last_error()
    # known flags pass flag validation and fail later, on the bad v_split
    for f in (kda.KDA_PREFILL_SCALAR_GATE, kda.KDA_PREFILL_WIDE_DECAY, 3, kda.KDA_PREFILL_ANY_DECAY,
              kda.KDA_PREFILL_ANY_DECAY | kda.KDA_PREFILL_SCALAR_GATE):
        assert kda.kda_prefill_ex(flags=f, **dict(a, v_split=3)) == kda.KDA_ERR_INVALID_ARG
        assert "v_split" in kda.kda_last_error()


def test_gdn_entry_points_validate_the_per_head_gate():
    args = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1, T_tot=64, H=2,
                d_k=64, d_v=64, dtype=BF16, o=FAKE, S_T=FAKE, workspace=None, workspace_bytes=0,
                v_split=0, stream=None)
    # [T, H] fp32: 4-byte alignment is enough, 2 is not
    assert kda.gdn_prefill_split(log_alpha=FAKE + 2, **args) == kda.KDA_ERR_INVALID_ARG
    assert "4-byte" in kda.kda_last_error()
    assert kda.gdn_prefill_split(log_alpha=None, **args) == kda.KDA_ERR_INVALID_ARG
    assert kda.gdn_prefill_split(log_alpha=FAKE, **dict(args, d_k=48)) == kda.KDA_ERR_UNSUPPORTED
    assert kda.gdn_decode_step(FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, 4, 2, 64, 64, BF16, FAKE,
                               None) == kda.KDA_ERR_INVALID_ARG
    assert kda.gdn_decode_step(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 2, 64, 64, BF16, FAKE,
                               None) == kda.KDA_ERR_INVALID_ARG


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S=FAKE, N=4, H=2, d_k=128, d_v=128,
             dtype=F32, o=FAKE, stream=None)
    a.update(kw)
    return kda.kda_decode_step(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARG),
    (dict(H=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(d_k=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=2), kda.KDA_ERR_UNSUPPORTED),
    (dict(S=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(v=FAKE + 2), kda.KDA_ERR_INVALID_ARG),
])
def test_decode_rejects_invalid_arguments(kw, status):
    assert _decode(**kw) == status
    assert kda.kda_last_error() != ""


def test_workspace_and_default_split_queries():
    # no workspace unless a sequence can be long enough to run in segments
    # and the batch has too few (sequence, head) pairs to fill the GPU
    assert kda.kda_prefill_workspace_size(1, 1024, 32, 128, 128, BF16) == 0
    assert kda.kda_prefill_workspace_size(1, 4096, 32, 128, 128, BF16) > 0
    assert kda.kda_prefill_workspace_size(1, 100000, 4, 64, 128, BF16) == 0
    assert kda.kda_prefill_workspace_size(8, 32677, 32, 128, 128, BF16) == 0  # 256 pairs
    assert kda.kda_prefill_workspace_size(3, 32677, 42, 128, 128, BF16) > 0   # 126 pairs
    assert kda.kda_prefill_workspace_size(4, 32677, 32, 128, 128, BF16) == 0  # 128 pairs
    ws = kda.kda_prefill_workspace_size(1, 131072, 32, 128, 128, BF16)
    # the identity runs' outputs and M, D for N + min(T_tot // 1024, 3 N + T_tot // 32768)
    # segments (8 here; 4 are used), plus the plan
    segs = 1 + min(131072 // 1024, 3 + 131072 // 32768)
    assert segs == 8
    body = 131072 * 32 * 128 * 2 + 2 * segs * 32 * 128 * 128 * 4
    assert body <= ws <= body + 4096
    assert kda.kda_prefill_workspace_size(1, 131072, 32, 128, 128, F32) > ws
    assert kda.kda_prefill_workspace_size(2, 131072, 32, 128, 128, BF16) > ws
    assert kda.kda_prefill_workspace_size(0, 32677, 32, 128, 128, BF16) == 0
    for (N, H) in ((1, 32), (8, 32), (256, 32), (1, 2)):
        s = kda.kda_prefill_default_split(N, 4096, H, 128, 128, BF16)
        assert s in (1, 2, 4, 8)
    assert kda.kda_prefill_default_split(1, 10, 1, 48, 128, BF16) == 0
    assert kda.kda_prefill_default_split(1, 10, 1, 32, 32, BF16) in (1, 2)


def test_workspace_size_ex_with_flags():
    """Any decay: the chunk lists (counts [N H] int32 and H (T_tot + 2 N) int32
    starts, each rounded up to 256 bytes) and one flag byte per token and head;
    other flags: kda_prefill_workspace_size."""
    ANY, WIDE, SG = kda.KDA_PREFILL_ANY_DECAY, kda.KDA_PREFILL_WIDE_DECAY, kda.KDA_PREFILL_SCALAR_GATE
    for (N, T, H) in ((8, 32677, 32), (1, 131072, 32), (3, 0, 2), (70, 3000, 2)):
        lists = (4 * N * H + 255) // 256 * 256 + (4 * H * (T + 2 * N) + 255) // 256 * 256 + H * T
        for extra in (0, SG):
            assert kda.kda_prefill_workspace_size_ex(N, T, H, 128, 128, BF16, ANY | extra) == lists
            assert kda.kda_prefill_workspace_size_ex(N, T, H, 64, 32, F32, ANY | extra) == lists
        for flags in (0, SG, WIDE, WIDE | SG):
            assert (kda.kda_prefill_workspace_size_ex(N, T, H, 128, 128, BF16, flags)
                    == kda.kda_prefill_workspace_size(N, T, H, 128, 128, BF16))
    assert kda.kda_prefill_workspace_size_ex(1, 4096, 32, 128, 128, BF16, 0) > 0  # segmented
    assert kda.kda_prefill_workspace_size_ex(1, 64, 2, 128, 128, BF16, ANY | WIDE) == 0
    assert kda.kda_prefill_workspace_size_ex(1, 64, 2, 128, 128, BF16, 8) == 0
    assert kda.kda_prefill_workspace_size_ex(1, 64, 2, 48, 128, BF16, ANY) == 0
    assert kda.kda_prefill_workspace_size_ex(0, 64, 2, 128, 128, BF16, ANY) == 0
    assert kda.kda_prefill_workspace_size_ex(1, -1, 2, 128, 128, BF16, ANY) == 0


def _plan(N, T, H, d, cus, dtype=BF16):
    return kda.prefill_plan(N, T, H, d, d, dtype, compute_units=cus)


def test_prefill_plan_follows_the_compute_unit_count():
    # 256 compute units (MI355X): segments while 2 N H < 256; 128 columns split in two
    # while units * H * 2 <= 128, counting segments at their bound when segmented
    v, ws = _plan(1, 4096, 32, 128, 256)  # 5 units at most: 320 > 128
    assert (v, ws > 0) == (1, True)
    assert _plan(8, 32677, 32, 128, 256) == (1, 0)  # 256 pairs fill the device
    assert _plan(1, 1000, 32, 128, 256) == (2, 0)  # 64 <= 128, too short to segment
    assert _plan(2, 1000, 16, 128, 256) == (2, 0)
    assert _plan(4, 32677, 32, 128, 256) == (1, 0)  # 128 pairs: not segmented
    assert _plan(3, 32677, 42, 128, 256)[1] > 0  # 126 pairs: segmented
    # 32 compute units: the same sizes cross the rules at an eighth of the pairs
    assert _plan(1, 4096, 32, 128, 32) == (1, 0)  # 2 * 32 >= 32: one pass
    v, ws = _plan(1, 4096, 8, 128, 32)  # 16 < 32: segmented
    assert (v, ws > 0) == (1, True)
    assert _plan(1, 1000, 4, 128, 32) == (2, 0)  # 8 <= 16
    assert _plan(1, 1000, 32, 128, 32) == (1, 0)  # 64 > 16
    # 64 value columns never split; the workspace does not depend on the dtype's split
    assert _plan(1, 1000, 1, 64, 256) == (1, 0)
    # compute_units = 0 is the current device (here: none, so 256), as the two queries use
    for N, T, H in ((1, 4096, 32), (8, 32677, 32), (1, 1000, 32)):
        v, ws = _plan(N, T, H, 128, 0)
        assert v == kda.kda_prefill_default_split(N, T, H, 128, 128, BF16)
        assert ws == kda.kda_prefill_workspace_size(N, T, H, 128, 128, BF16)
        assert (v, ws) == _plan(N, T, H, 128, 256)


@pytest.mark.parametrize("args,status", [
    ((0, 10, 1, 128, 128, BF16, 256), kda.KDA_ERR_INVALID_ARG),
    ((1, 10, 1, 128, 128, BF16, -1), kda.KDA_ERR_INVALID_ARG),
    ((1, 10, 1, 48, 128, BF16, 256), kda.KDA_ERR_UNSUPPORTED),
    ((1, 10, 1, 128, 128, 9, 256), kda.KDA_ERR_UNSUPPORTED),
])
def test_prefill_plan_validation(args, status):
    import ctypes
    v, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    assert kda.kda_prefill_plan(*args, ctypes.byref(v), ctypes.byref(ws)) == status
    assert kda.kda_last_error() != ""
    assert kda.kda_prefill_plan(1, 10, 1, 128, 128, BF16, 256, None, ctypes.byref(ws)) == kda.KDA_ERR_INVALID_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def _backward(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, d_o=FAKE, d_S_T=None, d_q=FAKE, d_k_out=FAKE,
             d_v_out=FAKE, d_log_alpha=FAKE, d_beta=FAKE, d_S0=FAKE, workspace=0x100000,
             workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    return kda.kda_prefill_backward(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARG, "N >= 1"),
    (dict(T_tot=-1), kda.KDA_ERR_INVALID_ARG, "T_tot"),
    (dict(d_k=48), kda.KDA_ERR_UNSUPPORTED, "d_k and d_v"),
    (dict(dtype=5), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(d_S0=None), kda.KDA_ERR_INVALID_ARG, "d_S0"),
    (dict(d_o=None), kda.KDA_ERR_INVALID_ARG, "d_o"),
    (dict(d_beta=None), kda.KDA_ERR_INVALID_ARG, "gradient"),
    (dict(d_q=FAKE + 4), kda.KDA_ERR_INVALID_ARG, "16-byte aligned"),
    (dict(d_beta=FAKE + 2), kda.KDA_ERR_INVALID_ARG, "4-byte aligned"),
    (dict(workspace_bytes=16), kda.KDA_ERR_INVALID_ARG, "workspace smaller"),
    (dict(workspace=None), kda.KDA_ERR_INVALID_ARG, "workspace must not be NULL"),
    (dict(workspace=0x100010), kda.KDA_ERR_INVALID_ARG, "256-byte aligned"),
])
def test_backward_validation(kw, status, needle):
    assert _backward(**kw) == status
    assert needle in kda.kda_last_error()


def test_backward_workspace_size():
    n, t, h, dk, dv = 3, 1000, 4, 64, 32
    # chunked (default): the entering state and W0 of at most T/C + N + 1 chunks per
    # head in the storage type (C = 32; 16 for fp32 with d_k >= 64)
    for dtype, C, es in ((BF16, 32, 2), (F32, 16, 4)):
        slots = (t // C + n + 1) * h
        want = (slots * dk * dv * es + 255) // 256 * 256 + slots * C * dv * es
        assert kda.kda_prefill_backward_workspace_size(n, t, h, dk, dv, dtype) == want
        assert kda.kda_prefill_backward_workspace_size_ex(n, t, h, dk, dv, dtype, 0) == want
        assert kda.kda_prefill_backward_workspace_size_ex(n, t, h, dk, dv, dtype, kda.KDA_PREFILL_SCALAR_GATE) == want
    assert kda.kda_prefill_backward_workspace_size(n, t, h, 32, dv, F32) == \
        ((t // 32 + n + 1) * h * 32 * dv * 4 + 255) // 256 * 256 + (t // 32 + n + 1) * h * 32 * dv * 4
    # token-recurrent: fp32 checkpoints for T/16 + N + 1 blocks per head (256-byte rounded)
    # plus one fp32 row per token-head
    ck = (t // 16 + n + 1) * h * dk * dv * 4
    assert kda.kda_prefill_backward_workspace_size_ex(n, t, h, dk, dv, BF16, kda.KDA_PREFILL_ANY_DECAY) == \
        (ck + 255) // 256 * 256 + t * h * dv * 4
    assert kda.kda_prefill_backward_workspace_size(0, t, h, dk, dv, BF16) == 0
    assert kda.kda_prefill_backward_workspace_size(n, t, h, 48, dv, BF16) == 0


def test_backward_ex_rejects_unknown_flags():
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, d_o=FAKE, d_S_T=None, d_q=FAKE, d_k_out=FAKE,
             d_v_out=FAKE, d_log_alpha=FAKE, d_beta=FAKE, d_S0=FAKE, workspace=0x100000,
             workspace_bytes=1 << 40, stream=None)
    for bad in (kda.KDA_PREFILL_WIDE_DECAY, 8, 1 << 31):
        assert kda.kda_prefill_backward_ex(flags=bad, **a) == kda.KDA_ERR_INVALID_ARG
        assert "flags" in kda.kda_last_error()
    # known flags pass flag validation and fail later, on the small workspace
    for f in (0, kda.KDA_PREFILL_ANY_DECAY, kda.KDA_PREFILL_SCALAR_GATE | kda.KDA_PREFILL_ANY_DECAY):
        assert kda.kda_prefill_backward_ex(flags=f, **dict(a, workspace_bytes=16)) == kda.KDA_ERR_INVALID_ARG
        assert "workspace smaller" in kda.kda_last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(log_alpha=FAKE + 2), "4-byte aligned"),
    (dict(d_log_alpha=FAKE + 2), "4-byte aligned"),
    (dict(d_q=FAKE + 4), "16-byte aligned"),
])
def test_gdn_backward_validation(kw, needle):
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE + 4, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, d_o=FAKE, d_S_T=None, d_q=FAKE, d_k_out=FAKE,
             d_v_out=FAKE, d_log_alpha=FAKE + 4, d_beta=FAKE, d_S0=FAKE, workspace=0x100000,
             workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    assert kda.gdn_prefill_backward(**a) == kda.KDA_ERR_INVALID_ARG
    assert needle in kda.kda_last_error()


def test_prefill_any_decay_excludes_wide_decay():
    a = dict(q=FAKE, k=FAKE, v=FAKE, log_alpha=FAKE, beta=FAKE, S0=None, cu_seqlens=FAKE, N=1,
             T_tot=64, H=2, d_k=64, d_v=64, dtype=BF16, o=FAKE, S_T=FAKE, workspace=None,
             workspace_bytes=0, v_split=0,
             flags=kda.KDA_PREFILL_WIDE_DECAY | kda.KDA_PREFILL_ANY_DECAY, stream=None)
    assert kda.kda_prefill_ex(**a) == kda.KDA_ERR_INVALID_ARG
    assert "exclude each other" in kda.kda_last_error()
