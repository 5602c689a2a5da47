"""Plant plausible mistakes in copies of the oracle (on the CPU, in a temp
directory) and require that each one fails at least one pin.  This shows the
pins constrain every step of the oracle: a dropped term, a wrong sign or
index, a swapped operand, a reordered step."""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS

_SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")
_HDR = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.h")

_DECAY_AFTER_READ = (
    "    for (int64_t i = 0; i < Dk; ++i) {\n"
    "      const double e2 = exp(gt[i]);\n"
    "      for (int64_t j = 0; j < Dv; ++j) S[i * Dv + j] *= e2;\n"
    "    }\n"
    "    /* 3. write the beta-scaled correction along k */")
_READ_BEFORE_WRITE = (
    "    for (int64_t j = 0; j < Dv; ++j) {\n"
    "      double a = 0.0;\n"
    "      for (int64_t i = 0; i < Dk; ++i) a += S[i * Dv + j] * qt[i];\n"
    "      ot[j] = a;\n"
    "    }\n"
    "    /* 3. write the beta-scaled correction along k */")

# name -> list of (old, new) textual substitutions
MUTANTS = {
    "decay_on_columns": [("row[j] *= e;", "row[j] *= exp(gt[j % Dk]);")],
    "decay_dropped": [("row[j] *= e;", "(void)e;")],
    "decay_index_shift": [("const double e = exp(gt[i]);\n      double *row",
                           "const double e = exp(gt[i > 0 ? i - 1 : 0]);\n"
                           "      double *row")],
    "decay_after_prediction": [("row[j] *= e;", "(void)e; (void)row;"),
                               ("    /* 3. write the beta-scaled correction "
                                "along k */", _DECAY_AFTER_READ)],
    "beta_dropped": [("u[j] = bt * (vt[j] - u[j]);", "u[j] = vt[j] - u[j];")],
    "residual_sign": [("u[j] = bt * (vt[j] - u[j]);",
                       "u[j] = bt * (vt[j] + u[j]);")],
    "beta_index_shift": [("beta[t * tok_stride_b]",
                          "beta[(t > 0 ? t - 1 : 0) * tok_stride_b]")],
    "predict_with_q": [("u[j] += row[j] * ki;", "u[j] += row[j] * qt[i];")],
    "write_along_q": [("row[j] += ki * u[j];", "row[j] += qt[i] * u[j];")],
    "readout_with_k": [("ot[j] += row[j] * qi;", "ot[j] += row[j] * kt[i];")],
    "readout_before_write": [
        ("for (int64_t j = 0; j < Dv; ++j) ot[j] = 0.0;", ";"),
        ("ot[j] += row[j] * qi;", "(void)row; (void)qi;"),
        ("    /* 3. write the beta-scaled correction along k */",
         _READ_BEFORE_WRITE)],
    "scale_dropped": [("for (int64_t j = 0; j < Dv; ++j) ot[j] *= scale;",
                       "(void)scale;")],
    "conv_taps_reversed": [("acc += w[c * W + j] * xv;",
                            "acc += w[c * W + (W - 1 - j)] * xv;")],
    "conv_history_off_by_one": [("const int64_t tau = T - (W - 1) + m;",
                                 "const int64_t tau = T - (W - 1) + m - 1;")],
    "l2_eps_outside_sqrt": [("1.0 / sqrt(ss + eps)",
                             "1.0 / (sqrt(ss) + eps)")],
    "l2_eps_dropped": [("1.0 / sqrt(ss + eps)", "1.0 / sqrt(ss)")],
    # the gradient
    "bwd_prediction_term_dropped": [("        dkt[i] += a;\n", "        (void)a;\n")],
    "bwd_du_sign": [("du[j] = -bt * ddel[j];", "du[j] = bt * ddel[j];")],
    "bwd_dg_undecayed_state": [("a += dS[i * Dv + j] * Sp[i * Dv + j];",
                                "a += dS[i * Dv + j] * P[i * Dv + j];")],
    "bwd_decay_not_propagated": [("          dS[i * Dv + j] *= e;\n",
                                  "          (void)e;\n")],
    "bwd_dq_from_decayed_state": [("a += (Sp[i * Dv + j] + kt[i] * del[j]) * dot[j];",
                                   "a += Sp[i * Dv + j] * dot[j];")],
    "bwd_block_recompute_short": [("for (int64_t t = t0; t + 1 < t1; ++t)",
                                   "for (int64_t t = t0; t + 2 < t1; ++t)")],
    "bwd_dbeta_residual_sign": [("db += ddel[j] * (vt[j] - u[j]);",
                                 "db += ddel[j] * (vt[j] + u[j]);")],
}


# mistakes in the Python composition of the conv prologue (oracle/__init__.py)
PY_MUTANTS = {
    "py_l2_on_v": [("if l2norm_qk and i < 2:", "if l2norm_qk:")],
    "py_heads_as_d_by_h": [("y = y.reshape(B, T, H, D)",
                            "y = y.reshape(B, T, D, H).transpose(0, 1, 3, 2)")],
    "py_history_ignored": [("None if hist is None else hist[i]", "None")],
    "py_l2_only_q": [("if l2norm_qk and i < 2:", "if l2norm_qk and i < 1:")],
}


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="kda_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _failures(orc):
    bad = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            bad.append(pin.__name__)
    return bad


def test_real_oracle_passes_all(orc):
    assert _failures(orc) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    text = open(_SRC).read()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, (name, old)
        text = text.replace(old, new)
    d = os.path.join(tmpdir_mod, name)
    os.makedirs(d)
    shutil.copy(_HDR, d)
    src = os.path.join(d, "kda_oracle.c")
    with open(src, "w") as f:
        f.write(text)
    lib = oracle.build(src, os.path.join(d, "lib.so"))
    failed = _failures(oracle.Oracle(lib))
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(name, orc):
    """The same for the prologue composition in the oracle's Python layer:
    the mutated module runs on the real compiled library."""
    import types
    path = oracle.__file__
    text = open(path).read()
    for old, new in PY_MUTANTS[name]:
        assert text.count(old) == 1, (name, old)
        text = text.replace(old, new)
    mod = types.ModuleType("oracle_mutant_" + name)
    mod.__file__ = path
    exec(compile(text, path, "exec"), mod.__dict__)
    failed = _failures(mod.Oracle(oracle._LIB))
    assert failed, f"mutant {name} passed every pin"
