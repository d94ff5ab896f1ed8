"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of oracle/kda_oracle.c with one plausible mistake (a
dropped term, a wrong sign, a wrong index, a transposed operand, the read-out
taken before the update).  It is compiled with gcc into a temporary
directory and the pin suite runs against it in a child process, so a mutant
that crashes counts as caught.  CPU only; the real oracle is not modified.
"""
import json
import os
import subprocess
import sys

import pytest

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_SRC = os.path.join(_ROOT, "oracle", "kda_oracle.c")

# (name, exact text in the source, replacement)
MUTANTS = [
    ("decay_dropped", "S[(size_t)i * dv + j] *= a;", "S[(size_t)i * dv + j] *= 1.0;"),
    ("decay_sign", "exp((double)lat[i])", "exp(-(double)lat[i])"),
    ("decay_on_value_columns", "const double a = exp((double)lat[i]);\n"
     "            for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;",
     "for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= "
     "exp((double)lat[j < dk ? j : 0]);"),
    ("error_sign", "u[j] = bt * ((double)vt[j] - u[j]);", "u[j] = bt * ((double)vt[j] + u[j]);"),
    ("beta_dropped", "u[j] = bt * ((double)vt[j] - u[j]);", "u[j] = ((double)vt[j] - u[j]);"),
    ("beta_wrong_head", "(double)J->beta[(size_t)t * H + h]", "(double)J->beta[(size_t)t * H]"),
    ("prediction_uses_query", "u[j] += ki * S[(size_t)i * dv + j];",
     "u[j] += (double)qt[i] * S[(size_t)i * dv + j];"),
    ("readout_uses_key", "const double qi = (double)qt[i];", "const double qi = (double)kt[i];"),
    ("state_transposed_in_prediction", "u[j] += ki * S[(size_t)i * dv + j];",
     "u[j] += ki * S[((size_t)j * dk + i) % ((size_t)dk * dv)];"),
    ("initial_state_ignored", "if (J->S0) {", "if (0) {"),
    ("first_token_skipped", "for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t)",
     "for (int64_t t = J->cu[n] + (J->cu[n + 1] > J->cu[n]); t < J->cu[n + 1]; ++t)"),
    ("rank1_update_dropped", "S[(size_t)i * dv + j] += ki * u[j];",
     "S[(size_t)i * dv + j] += 0.0 * ki * u[j];"),
    # backward pass
    ("bwd_readout_grad_uses_pre_update_state", "acc += dSp[(size_t)i * dv + j] * dot[j];",
     "acc += S[(size_t)i * dv + j] * dot[j];"),
    ("bwd_readout_grad_not_accumulated", "G[(size_t)i * dv + j] += (double)qt[i] * dot[j];",
     "G[(size_t)i * dv + j] += 0.0 * (double)qt[i] * dot[j];"),
    ("bwd_beta_grad_uses_scaled_error", "db += de[j] * w[j];", "db += de[j] * bt * w[j];"),
    ("bwd_key_grad_prediction_term_dropped", "J->dk_[tk + i] = tmp[i] + acc;", "J->dk_[tk + i] = tmp[i];"),
    ("bwd_decay_grad_uses_decayed_state", "da += g * Sp[(size_t)i * dv + j];",
     "da += g * S[(size_t)i * dv + j];"),
    ("bwd_state_grad_not_decayed", "G[(size_t)i * dv + j] = a * g;", "G[(size_t)i * dv + j] = g;"),
    ("bwd_value_grad_beta_dropped", "J->dv_[tv + j] = bt * de[j];", "J->dv_[tv + j] = de[j];"),
    ("bwd_prediction_grad_sign", "du[j] = -bt * de[j];", "du[j] = bt * de[j];"),
    ("bwd_key_grad_transposed_state", "acc += S[(size_t)i * dv + j] * du[j];",
     "acc += S[((size_t)j * dk + i) % ((size_t)dk * dv)] * du[j];"),
    ("bwd_states_one_token_late",
     "memcpy(states + (size_t)(t - tb) * SS, S, sizeof(double) * SS);\n            forward_token(J, t, h, S, u);",
     "forward_token(J, t, h, S, u);\n            memcpy(states + (size_t)(t - tb) * SS, S, sizeof(double) * SS);"),
    ("bwd_final_state_grad_ignored", "if (J->dST) memcpy(G,", "if (0) memcpy(G,"),
]

_CHILD = r"""
import json, sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle, oracle_pins
lib = oracle.bind(sys.argv[3])
print(json.dumps(oracle_pins.run_all(lib)))
"""


def _readout_before_update(src):
    """Move step 5 (read-out) in front of step 4 (rank-1 correction)."""
    a = src.index("        /* 4. rank-1 correction")
    b = src.index("        /* 5. read-out")
    c = src.index("    }\n    memcpy(J->S_T + sbase")
    return src[:a] + src[b:c] + src[a:b] + src[c:]


@pytest.mark.parametrize("name,old,new", MUTANTS + [("readout_before_update", None, None)],
                         ids=[m[0] for m in MUTANTS] + ["readout_before_update"])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(_SRC).read()
    if old is None:
        mutated = _readout_before_update(src)
    else:
        assert src.count(old) >= 1, f"mutation anchor for {name} not found in the oracle"
        mutated = src.replace(old, new, 1)
    assert mutated != src
    c_path = tmp_path / "kda_oracle.c"
    c_path.write_text(mutated)
    (tmp_path / "kda_oracle.h").write_text(open(_SRC[:-2] + ".h").read())
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so),
                    str(c_path), "-lm"], check=True)
    r = subprocess.run([sys.executable, "-c", _CHILD, _ROOT, os.path.join(_ROOT, "tests"),
                        str(so)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # the mutant crashed the pin run: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"


# Mistakes planted in the oracle's Python layer (oracle/__init__.py): the
# Gated DeltaNet backward sums the per-channel gate gradient over the key
# channels, the chain rule of repeating one gate per head over them.
PY_MUTANTS = [
    ("gdn_gate_grad_mean_over_channels", "dla.sum(axis=2)", "dla.mean(axis=2)"),
    ("gdn_gate_grad_channel_zero_only", "dla.sum(axis=2)", "dla[:, :, 0]"),
    ("gdn_gate_grad_last_channel_only", "dla.sum(axis=2)", "dla[:, :, -1]"),
]

_PY_CHILD = r"""
import json, sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle, oracle_pins
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
lib = oracle.bind(sys.argv[3])
print(json.dumps(oracle_pins.run_all(lib)))
"""


_PY_CONTROL = ("unmodified_copy", "dla.sum(axis=2)", "dla.sum(axis=2)")


@pytest.mark.parametrize("name,old,new", PY_MUTANTS + [_PY_CONTROL], ids=[m[0] for m in PY_MUTANTS + [_PY_CONTROL]])
def test_python_mutant_is_caught(tmp_path, name, old, new):
    import oracle

    pkg = os.path.join(_ROOT, "oracle")
    src = open(os.path.join(pkg, "__init__.py")).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found in the oracle"
    mutated = src.replace(old, new, 1)
    assert (mutated != src) == (old != new)
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "__init__.py").write_text(mutated)
    (tmp_path / "oracle" / "build.py").write_text(open(os.path.join(pkg, "build.py")).read())
    so = oracle.library_path()
    if not os.path.exists(so):
        oracle.build_oracle()
    r = subprocess.run([sys.executable, "-c", _PY_CHILD, str(tmp_path), os.path.join(_ROOT, "tests"), so],
                       capture_output=True, text=True, timeout=300)
    if old == new:  # control: the unmodified copy passes every pin in the child
        assert r.returncode == 0, r.stderr
        assert json.loads(r.stdout.strip().splitlines()[-1]) == []
        return
    if r.returncode != 0:
        return  # the mutant crashed the pin run: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert "pin_gdn_backward_finite_differences" in failed, f"mutant {name} passed the GDN backward pin"
