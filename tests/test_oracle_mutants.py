"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case plants one mistake in a copy of oracle/sru_oracle.c (a flipped sign,
a dropped term, a wrong parameter or index, the wrong rounding or
normalisation), builds it on the CPU, points the oracle module at the mutant
library and runs the pin suite (tests/test_oracle_pins.py) in a subprocess.
The compositions written in Python (oracle/__init__.py: the SRU++ attention's
residual, context order, rounding points and layer-norm placement) get the
same treatment: a mutated copy of the module is loaded in place of the real
one, over an unchanged build of the C library.
At least one pin must fail for every mutant.  Nothing here touches the GPU
or the HIP library.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sru_oracle.c")

# (name, text in sru_oracle.c, the planted mistake)
MUTANTS = [
    ("sigmoid sign",
     "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    ("bf16 ties away from zero",
     "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    ("Eq. 2 with the reset gate's v",
     "double f = oracle_sigmoid(uf[t] + vf * seen + bf);          /* Eq. 2 */",
     "double f = oracle_sigmoid(uf[t] + vr * seen + bf);          /* Eq. 2 */"),
    ("Eq. 4 with f and 1 - f swapped",
     "state = f * prev + (1.0 - f) * ux[t];", "state = (1.0 - f) * prev + f * ux[t];"),
    ("Eq. 5 without alpha",
     "h[t] = r * state + (1.0 - r) * alpha * x[t];", "h[t] = r * state + (1.0 - r) * x[t];"),
    ("state adjoint without the reset-gate term",
     "gc = linear ? dc * f : dc * f + dzf * vf + dzr * vr;",
     "gc = linear ? dc * f : dc * f + dzf * vf;"),
    ("linear-mode gates that see the state in the backward",
     "double seen = linear ? 0.0 : prev;\n        double f = oracle_sigmoid(uf[t] + vf * seen + bf);\n",
     "double seen = prev;\n        double f = oracle_sigmoid(uf[t] + vf * seen + bf);\n"),
    ("linear-mode state adjoint with the gate terms",
     "gc = linear ? dc * f : dc * f + dzf * vf + dzr * vr;",
     "gc = dc * f + dzf * vf + dzr * vr;"),
    ("highway gradient without alpha",
     "dx_hw[t] = dh[t] * (1.0 - r) * alpha;", "dx_hw[t] = dh[t] * (1.0 - r);"),
    ("candidate gradient with f for 1 - f",
     "dux[t] = dc * (1.0 - f);", "dux[t] = dc * f;"),
    ("projection with the weight row reversed",
     "s += arow[q] * (double)w[q];", "s += arow[q] * (double)w[K - 1 - q];"),
    ("backward-data with the weight row reversed",
     "o[q] += g[n] * (double)w[q];", "o[q] += g[n] * (double)w[K - 1 - q];"),
    ("weight gradient ignoring the rounding of X",
     "const double xv = round_x ? (double)sru_oracle_round_bf16(x[q]) : (double)x[q];",
     "const double xv = (double)x[q];"),
    ("attention without the 1/sqrt(d') scale",
     "const double scale = 1.0 / sqrt((double)dp);\n#pragma omp parallel\n    {\n        double *p = (double *)malloc(sizeof(double) * (size_t)Lk);\n#pragma omp for",
     "const double scale = 1.0;\n#pragma omp parallel\n    {\n        double *p = (double *)malloc(sizeof(double) * (size_t)Lk);\n#pragma omp for"),
    ("causal mask one key short",
     "* dp;\n            const int64_t nk = causal ? Lm + t + 1 : Lk;",
     "* dp;\n            const int64_t nk = causal ? Lm + t + (t > 0) : Lk;"),
    ("attention backward without the 1/sqrt(d') scale",
     "const double scale = 1.0 / sqrt((double)dp);\n    for (int64_t i = 0;",
     "const double scale = 1.0;\n    for (int64_t i = 0;"),
    ("attention backward with the causal mask one key short",
     "* dp;\n                const int64_t nk = causal ? Lm + t + 1 : Lk;",
     "* dp;\n                const int64_t nk = causal ? Lm + t + (t > 0) : Lk;"),
    ("layer norm with the unbiased variance",
     "var /= (double)w;\n        const double inv = 1.0 / sqrt(var + eps);\n        for (int64_t e = 0; e < w; ++e)\n            y[i * w + e]",
     "var /= (double)(w > 1 ? w - 1 : 1);\n        const double inv = 1.0 / sqrt(var + eps);\n        for (int64_t e = 0; e < w; ++e)\n            y[i * w + e]"),
    ("softmax backward without the weighted mean of the value gradients",
     "const double ds = p[j] * (g[j] - D) * scale;", "const double ds = p[j] * g[j] * scale;"),
    ("value gradient without the attention weight",
     "dv[e] += p[j] * da[e];", "dv[e] += da[e];"),
    ("layer norm backward without the mean term",
     "dx[i * w + e] = (g[e] * gamma[e] - m1 - xh[e] * m2) * inv;",
     "dx[i * w + e] = (g[e] * gamma[e] - xh[e] * m2) * inv;"),
]

# (name, text in oracle/__init__.py, the planted mistake)
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = [
    ("attention residual with the wrong sign",
     "R = Q + alpha * A.reshape(L * B, dp)", "R = Q - alpha * A.reshape(L * B, dp)"),
    ("context rows after the segment's own rows",
     "        Kc = np.concatenate([np.asarray(Kmem, np.float64), Kc])\n"
     "        Vc = np.concatenate([np.asarray(Vmem, np.float64), Vc])",
     "        Kc = np.concatenate([Kc, np.asarray(Kmem, np.float64)])\n"
     "        Vc = np.concatenate([Vc, np.asarray(Vmem, np.float64)])"),
    ("keys and values from the unrounded Q",
     "Qt = _maybe_bf16(Q, round_ops)", "Qt = Q"),
    ("values from the key weights",
     "Vc = matmul(Qt, Wv, b_nk=True)", "Vc = matmul(Qt, Wk, b_nk=True)"),
    ("layer norm after the output projection",
     "    if ln is not None:\n"
     "        R = layernorm(R, ln[0], ln[1], ln[2])\n"
     "    U = matmul(_maybe_bf16(R, round_ops), Wo, b_nk=True)",
     "    U = matmul(_maybe_bf16(R, round_ops), Wo, b_nk=True)\n"
     "    if ln is not None:\n"
     "        U = layernorm(U, np.resize(ln[0], U.shape[1]), np.resize(ln[1], U.shape[1]), ln[2])"),
    ("alpha's gradient taken against R instead of A",
     "dalpha = float(np.sum(dS * A))", "dalpha = float(np.sum(dS * R))"),
    ("no residual path from the normalised sum back to Q",
     "dQ = dS + dQa.reshape(L * B, dp)", "dQ = dQa.reshape(L * B, dp)"),
    ("the context rows take the key and value gradients",
     "dKs = dK[mem_len:].reshape(L * B, dp)", "dKs = dK[:L].reshape(L * B, dp)"),
    ("layer norm of Q before the attention term is added",
     "    R = Q + alpha * A.reshape(L * B, dp)\n"
     "    if ln is not None:\n"
     "        R = layernorm(R, ln[0], ln[1], ln[2])",
     "    R = Q\n"
     "    if ln is not None:\n"
     "        R = layernorm(R, ln[0], ln[1], ln[2])\n"
     "    R = R + alpha * A.reshape(L * B, dp)"),
]

RUNNER = """
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._LIB_PATH = {lib!r}
oracle._lib = None
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {pins!r}]))
"""


# As RUNNER, with the oracle module itself replaced by a copy loaded from a
# scratch package directory before the pins import it.
RUNNER_PY = """
import importlib.util
import sys
sys.path.insert(0, {root!r})
spec = importlib.util.spec_from_file_location("oracle", {init!r},
                                              submodule_search_locations=[{pkg!r}])
mod = importlib.util.module_from_spec(spec)
sys.modules["oracle"] = mod
spec.loader.exec_module(mod)
mod._LIB_PATH = {lib!r}
mod._lib = None
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {pins!r}]))
"""


def run_pins(tmp_path, source, py_source=None):
    """Build `source` as the oracle library and run the pin suite against it
    (with `py_source` as the oracle module, when given)."""
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    c = tmp_path / "sru_oracle_copy.c"
    c.write_text(source)
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(c),
                    "-o", str(lib), "-lm"], check=True)
    pins = os.path.join(ROOT, "tests", "test_oracle_pins.py")
    if py_source is None:
        code = RUNNER.format(root=ROOT, lib=str(lib), pins=pins)
    else:
        pkg = tmp_path / "oracle_copy"
        pkg.mkdir()
        (pkg / "__init__.py").write_text(py_source)
        shutil.copy(os.path.join(ROOT, "oracle", "build.py"), pkg / "build.py")
        code = RUNNER_PY.format(root=ROOT, init=str(pkg / "__init__.py"), pkg=str(pkg),
                                lib=str(lib), pins=pins)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                          text=True, timeout=600, env=dict(os.environ, OMP_NUM_THREADS="4"))


def test_unchanged_copy_passes_every_pin(tmp_path):
    """Control: the harness itself runs the pins against a copy cleanly."""
    r = run_pins(tmp_path, open(SRC).read())
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    r = run_pins(tmp_path, src.replace(old, new))
    # pytest's exit status 1 with a failed pin (not an import or collection error)
    assert r.returncode == 1 and " failed" in r.stdout, (
        f"no pin caught '{name}' (exit {r.returncode})\n" + r.stdout[-2000:] + r.stderr[-2000:])


def test_unchanged_module_copy_passes_every_pin(tmp_path):
    """Control for the Python mutants: an unchanged copy of the module."""
    r = run_pins(tmp_path, open(SRC).read(), open(PY_SRC).read())
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_planted_mistake_in_the_python_compositions(tmp_path, name, old, new):
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    r = run_pins(tmp_path, open(SRC).read(), src.replace(old, new))
    assert r.returncode == 1 and " failed" in r.stdout, (
        f"no pin caught '{name}' (exit {r.returncode})\n" + r.stdout[-2000:] + r.stderr[-2000:])
