"""The oracle's pins must catch plausible mistakes (CPU only).

Each case copies oracle/gla_oracle.c, plants one mistake by text substitution,
builds the copy with gcc into a temporary directory and runs the pin suite
(tests/test_oracle.py) against it in a subprocess.  The suite has to fail for
every mutant; the unmodified source has to pass.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gla_oracle.c")

MUTANTS = {
    "decay_after_write": ("row[j] = alpha[i] * row[j] + kt[i] * vt[j];",
                          "row[j] = alpha[i] * (row[j] + kt[i] * vt[j]);"),
    "gate_sign": ("alpha[i] = exp(gt[i]);", "alpha[i] = exp(-gt[i]);"),
    "current_token_dropped": ("row[j] = alpha[i] * row[j] + kt[i] * vt[j];",
                              "row[j] = alpha[i] * row[j] + (t > 0 ? kt[i] * vt[j] : 0.0);"),
    "state_transposed_in_read": ("acc += qt[i] * S[(long)i * d_v + j];",
                                 "acc += qt[i] * S[(long)j * d_v + i];"),
    "gate_on_value_dims": ("row[j] = alpha[i] * row[j] + kt[i] * vt[j];",
                           "row[j] = alpha[j % d_k] * row[j] + kt[i] * vt[j];"),
    "tb_row_major": ("return row * grid_w + col;\n    }\n    case 3",
                     "return col * grid_h + row;\n    }\n    case 3"),
    "rl_row_mirror": ("case 1: return n_tok - 1 - t;",
                      "case 1: return (t / grid_w) * grid_w + (grid_w - 1 - t % grid_w);"),
    "query_reads_old_state": ("for (int i = 0; i < d_k; ++i) alpha[i] = exp(gt[i]);",
                              "for (int i = 0; i < d_k; ++i) alpha[i] = exp(gt[i]);\n"
                              "                for (int j = 0; j < d_v; ++j) { double a0 = 0.0;"
                              " for (int i = 0; i < d_k; ++i) a0 += qt[i] * S[(long)i * d_v + j];"
                              " os[n * d_v + j] = a0; }"),
}


def run_pins(lib_path):
    env = dict(os.environ, GLA_ORACLE_LIB_OVERRIDE=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mut = src.replace(old, new, 1)
    if name == "query_reads_old_state":
        # the mutant writes the output before the update; drop the correct write after it
        mut = mut.replace("ot[j] = acc;", "(void)acc; (void)ot;", 1)
    path = tmp_path / f"{name}.c"
    path.write_text(mut)
    return oracle.build_from(str(path), str(tmp_path / f"{name}.so"))


def test_unmodified_oracle_passes(tmp_path):
    lib = oracle.build_from(SRC, str(tmp_path / "clean.so"))
    rc, out = run_pins(lib)
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = build_mutant(tmp_path, name, old, new)
    rc, out = run_pins(lib)
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"


# Mistakes planted in the backward pass; the backward pins (tests/test_oracle_bwd.py) must fail.
BWD_MUTANTS = {
    "bwd_dq_from_old_state": ("acc += S[(long)i * d_v + j] * dos[n * d_v + j];",
                              "acc += prev[t * kv + (long)i * d_v + j] * dos[n * d_v + j];"),
    "bwd_extra_decay": ("G[(long)i * d_v + j] += qs[n * d_k + i] * dos[n * d_v + j];",
                        "G[(long)i * d_v + j] = exp(gs[n * d_k + i]) * G[(long)i * d_v + j]"
                        " + qs[n * d_k + i] * dos[n * d_v + j];"),
    "bwd_gate_grad_without_alpha": ("dgs[n * d_k + i] = exp(gs[n * d_k + i]) * da;",
                                    "dgs[n * d_k + i] = da;"),
    "bwd_dk_transposed_state": ("acc += G[(long)i * d_v + j] * vs[n * d_v + j];",
                                "acc += G[(long)(j % d_k) * d_v + (i % d_v)] * vs[n * d_v + j];"),
    "bwd_dv_uses_query": ("acc += ks[n * d_k + i] * G[(long)i * d_v + j];",
                          "acc += qs[n * d_k + i] * G[(long)i * d_v + j];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(tmp_path, name):
    old, new = BWD_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new, 1))
    lib = oracle.build_from(str(path), str(tmp_path / f"{name}.so"))
    env = dict(os.environ, GLA_ORACLE_LIB_OVERRIDE=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_bwd.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every backward pin:\n{r.stdout[-2000:]}"


def test_unmodified_backward_passes(tmp_path):
    lib = oracle.build_from(SRC, str(tmp_path / "clean_bwd.so"))
    env = dict(os.environ, GLA_ORACLE_LIB_OVERRIDE=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_bwd.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
