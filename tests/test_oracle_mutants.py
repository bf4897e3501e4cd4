"""Plant plausible mistakes in the oracle (on the CPU, in a temporary copy of
its source) and check that the pins catch every one of them.  This is what
makes the pins a real check of the oracle rather than a restatement of it.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "mdn_oracle.c")

# (name, text in the oracle, replacement).  Each text must occur exactly once.
MUTANTS = [
    ("residual drops alpha",
     "vt[c] = vv[c] - a * vt[c];", "vt[c] = vv[c] - vt[c];"),
    ("residual sign",
     "vt[c] = vv[c] - a * vt[c];", "vt[c] = vv[c] + a * vt[c];"),
    ("momentum write sign",
     "M[x] = m * M[x] - e * kt[i] * vt[c];", "M[x] = m * M[x] + e * kt[i] * vt[c];"),
    ("momentum retention dropped",
     "M[x] = m * M[x] - e * kt[i] * vt[c];", "M[x] = - e * kt[i] * vt[c];"),
    ("eta dropped",
     "M[x] = m * M[x] - e * kt[i] * vt[c];", "M[x] = m * M[x] - kt[i] * vt[c];"),
    ("memory step sign",
     "S[x] = a * S[x] - s * M[x];", "S[x] = a * S[x] + s * M[x];"),
    ("memory decay dropped",
     "S[x] = a * S[x] - s * M[x];", "S[x] = S[x] - s * M[x];"),
    ("memory reads old momentum",
     "            M[x] = m * M[x] - e * kt[i] * vt[c];\n"
     "            S[x] = a * S[x] - s * M[x];",
     "            S[x] = a * S[x] - s * M[x];\n"
     "            M[x] = m * M[x] - e * kt[i] * vt[c];"),
    ("read-out uses key",
     "o[c] += S[(size_t)i * nc + c] * qt[i];", "o[c] += S[(size_t)i * nc + c] * kt[i];"),
    ("residual reads the momentum",
     "vt[c] += S[(size_t)i * nc + c] * kt[i];", "vt[c] += M[(size_t)i * nc + c] * kt[i];"),
    ("gates swapped",
     "const double a = alpha[g];\n        const double m = mu[g];",
     "const double a = mu[g];\n        const double m = alpha[g];"),
    ("beta ignored",
     "const double s = beta ? beta[g] : 1.0;", "const double s = 1.0;"),
    ("initial momentum ignored",
     "M[(size_t)i * nc + c] = M0 ? M0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;",
     "M[(size_t)i * nc + c] = 0.0;"),
    ("final states swapped",
     "if (ST) ST[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = S[(size_t)i * nc + c];",
     "if (ST) ST[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = M[(size_t)i * nc + c];"),
    ("value column offset dropped",
     "const double* vv = v + IDX_TOK(b, t, h, c0, T, H, Dv);",
     "const double* vv = v + IDX_TOK(b, t, h, 0, T, H, Dv);"),
    ("brute force: Gamma row shift off by one",
     "if (j < i) x = G[(size_t)(i - 1) * n + j];", "if (j < i) x = G[(size_t)i * n + j];"),
    ("brute force: carry uses old momentum sign",
     "Mn[x] = mbar[n] * M[x] - wm;", "Mn[x] = mbar[n] * M[x] + wm;"),
    ("residual output reports the read-out",
     "for (int c = 0; c < nc; ++c) vo[c] = vt[c];", "for (int c = 0; c < nc; ++c) vo[c] = o[c];"),
    ("backward: read-out gradient uses the key",
     "Sh[x] += qt[i] * dot[c];", "Sh[x] += kt[i] * dot[c];"),
    ("backward: memory step drops beta",
     "P[x] = Mh[x] - s * Sh[x];", "P[x] = Mh[x] - Sh[x];"),
    ("backward: memory gradient not decayed",
     "Sh[x] = a * Sh[x] - a * kt[i] * dvt[c];", "Sh[x] = Sh[x] - a * kt[i] * dvt[c];"),
    ("backward: residual gradient sign",
     "for (int c = 0; c < nc; ++c) dvt[c] *= -e;", "for (int c = 0; c < nc; ++c) dvt[c] *= e;"),
    ("backward: momentum gradient skips the memory step",
     "Mh[x] = m * P[x];", "Mh[x] = m * Mh[x];"),
    ("backward: dalpha misses the residual term",
     "ga -= kt[i] * acc;", "ga -= 0.0 * kt[i] * acc;"),
    ("backward: deta sign", "ge -= kt[i] * acc;", "ge += kt[i] * acc;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = oracle.build(str(mutated), str(tmp_path / "libmutant.so"))
    lib = oracle.load(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError,
                __import__("numpy").linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"


# the gate parameterisation is numpy code in oracle/__init__.py: mutate the
# function's own source text and run the pins against the mutated copy
GATE_MUTANTS = [
    ("eta offset dropped", "eta = 1.0 + np.tanh(", "eta = np.tanh("),
    ("eta temperature multiplies", "np.tanh(z(z_eta) / tau)", "np.tanh(z(z_eta) * tau)"),
    ("cos and sin swapped", "alpha_max = np.cos(theta) ** 2", "alpha_max = np.sin(theta) ** 2"),
    ("softplus shift sign", "np.logaddexp(0.0, x + b)", "np.logaddexp(0.0, x - b)"),
    ("decay scale dropped", "f = lambda x: -a * np.logaddexp", "f = lambda x: -np.logaddexp"),
    ("alpha_max dropped", "alpha = np.exp(f(z(z_alpha)) + np.log(alpha_max))",
     "alpha = np.exp(f(z(z_alpha)))"),
    ("sigmoid sign", "sig = 1.0 / (1.0 + np.exp(-z(z_beta)))",
     "sig = 1.0 / (1.0 + np.exp(z(z_beta)))"),
    ("beta_max dropped", "beta = sig * beta_max", "beta = sig"),
    ("momentum floor as a ceiling", "np.maximum(f(z(z_mu)), log_mu_min)",
     "np.minimum(f(z(z_mu)), log_mu_min)"),
]


@pytest.mark.parametrize("name,old,new", GATE_MUTANTS, ids=[m[0] for m in GATE_MUTANTS])
def test_gate_pin_catches_mutant(name, old, new, monkeypatch):
    import inspect
    import textwrap

    import numpy as np
    from oracle_pins import pin_gate_parameterisation

    src = textwrap.dedent(inspect.getsource(oracle.gates_from_logits))
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    ns = {"np": np}
    exec(compile(src.replace(old, new), "<gate mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "gates_from_logits", ns["gates_from_logits"])
    with pytest.raises(AssertionError):
        pin_gate_parameterisation(None)


LAYER_MUTANTS = [
    ("prologue", "correction sign", "q = q - np.asarray(d", "q = q + np.asarray(d"),
    ("prologue", "eps dropped from the query norm", "nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)",
     "nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True))"),
    ("prologue", "keys not normalised", "return q / nq, k / nk", "return q / nq, k"),
    ("epilogue", "sum instead of mean", "rms = np.sqrt(np.mean(o * o", "rms = np.sqrt(np.sum(o * o"),
    ("epilogue", "gate sign", "y = (1.0 / (1.0 + np.exp(-g)))", "y = (1.0 / (1.0 + np.exp(g)))"),
    ("epilogue", "weight ignored", "y = y * np.asarray(w, dtype=np.float64)", "y = y"),
]


@pytest.mark.parametrize("fn,name,old,new", LAYER_MUTANTS, ids=[m[1] for m in LAYER_MUTANTS])
def test_layer_pin_catches_mutant(fn, name, old, new, monkeypatch):
    import inspect
    import textwrap

    import numpy as np
    from oracle_pins import pin_layer_prologue_epilogue

    f = oracle.qk_prologue if fn == "prologue" else oracle.output_epilogue
    src = textwrap.dedent(inspect.getsource(f))
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    ns = {"np": np}
    exec(compile(src.replace(old, new), "<layer mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "qk_prologue" if fn == "prologue" else "output_epilogue",
                        ns["qk_prologue" if fn == "prologue" else "output_epilogue"])
    with pytest.raises(AssertionError):
        pin_layer_prologue_epilogue(None)
