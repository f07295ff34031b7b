"""Sanitizer builds of the host code (CPU only; nothing here touches a GPU).

* The CPU oracle (oracle/sru_oracle.c) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, and the whole oracle pin suite
  (tests/test_oracle_pins.py) run against it.
* libsru with its host code (the C entry points' argument validation,
  workspace sizing and the binding's marshalling) built with clang's
  AddressSanitizer and UndefinedBehaviorSanitizer, device code unchanged,
  and tests/test_abi_host.py run against it (those checks launch nothing).
Each run is a subprocess with the sanitizer runtime preloaded; any report
fails the test.  Skipped where LD_PRELOAD is already in use (nothing of the
caller's is overridden) or the runtime is missing.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _env(preload):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("LD_PRELOAD is already set; the sanitizer runtime is not forced over it")
    return dict(os.environ, LD_PRELOAD=preload, OMP_NUM_THREADS="4", **SAN_OPTS)


def _check(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]


def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "sru_oracle.c"),
                    "-o", str(lib), "-lm"], check=True)
    code = ("import sys\nsys.path.insert(0, %r)\nimport oracle\noracle._LIB_PATH = %r\n"
            "oracle._lib = None\nimport pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, str(lib), os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=900, env=_env(asan))
    _check(r)
    assert " passed" in r.stdout


def test_abi_host_checks_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from parallelizable_recurrent_units_amd import build
    objs = []
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    procs = []
    for src in build.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            ["hipcc", *build.CFLAGS, *host_san, "-g", "-c", os.path.join(build.CSRC, src),
             "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-3000:]
    lib = str(tmp_path / "libsru_san.so")
    subprocess.run(["hipcc", f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *host_san, *objs,
                    "-o", lib], check=True)
    code = ("import sys\nsys.path.insert(0, %r)\n"
            "from parallelizable_recurrent_units_amd import _binding\n"
            "_binding.load_library(%r)\nimport pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi_host.py")))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=900, env=_env(rt[-1]))
    _check(r)
    assert " passed" in r.stdout
