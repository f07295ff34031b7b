"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case plants one mistake in a copy of oracle/sru_oracle.c (a flipped sign,
a dropped term, a wrong parameter or index, the wrong rounding or
normalisation), builds it on the CPU, points the oracle module at the mutant
library and runs the pin suite (tests/test_oracle_pins.py) in a subprocess.
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
     "double f = oracle_sigmoid(uf[t] + vf * prev + bf);          /* Eq. 2 */",
     "double f = oracle_sigmoid(uf[t] + vr * prev + bf);          /* Eq. 2 */"),
    ("Eq. 4 with f and 1 - f swapped",
     "state = f * prev + (1.0 - f) * ux[t];", "state = (1.0 - f) * prev + f * ux[t];"),
    ("Eq. 5 without alpha",
     "h[t] = r * state + (1.0 - r) * alpha * x[t];", "h[t] = r * state + (1.0 - r) * x[t];"),
    ("state adjoint without the reset-gate term",
     "gc = dc * f + dzf * vf + dzr * vr;", "gc = dc * f + dzf * vf;"),
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
     "const double scale = 1.0 / sqrt((double)dp);", "const double scale = 1.0;"),
    ("causal mask one key short",
     "const int64_t nk = causal ? Lm + t + 1 : Lk;",
     "const int64_t nk = causal ? Lm + t + (t > 0) : Lk;"),
    ("layer norm with the unbiased variance",
     "var /= (double)w;", "var /= (double)(w > 1 ? w - 1 : 1);"),
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


def run_pins(tmp_path, source):
    """Build `source` as the oracle library and run the pin suite against it."""
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    c = tmp_path / "sru_oracle_copy.c"
    c.write_text(source)
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(c),
                    "-o", str(lib), "-lm"], check=True)
    code = RUNNER.format(root=ROOT, lib=str(lib),
                         pins=os.path.join(ROOT, "tests", "test_oracle_pins.py"))
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
