"""The boundary from C: include/sru.h compiles as C99 with every warning an
error, and a C program links libsru.so and calls entry points that need no
GPU (a status string, a workspace size, argument validation with its error
text)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "parallelizable_recurrent_units_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "sru.h"

int main(void)
{
    sru_shape s = {64, 128, 512, 1, 1.0f};
    sru_shape bad = {0, 1, 1, 0, 1.0f};
    size_t ws;
    if (strcmp(sru_status_string(SRU_ERR_WORKSPACE), "SRU_ERR_WORKSPACE") != 0) return 1;
    ws = sru_workspace_size(&s, SRU_WS_BACKWARD, 0);
    if (ws == 0 || ws % 256 != 0) return 2;
    if (sru_forward(&bad, NULL, SRU_F32, NULL, SRU_F32, NULL, NULL, NULL, NULL, SRU_F32, NULL,
                    NULL, NULL) != SRU_ERR_INVALID_ARG)
        return 3;
    if (strstr(sru_last_error(), "L, B, d") == NULL) return 4;
    printf("%lu\n", (unsigned long)ws);
    return 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    assert os.path.exists(os.path.join(PKG, "libsru.so")), "build libsru.so first"
    src = tmp_path / "use_sru.c"
    exe = tmp_path / "use_sru"
    src.write_text(PROGRAM)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-L", PKG, "-lsru",
           f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    # the backward workspace of L=64 B=128 d=512 bidirectional, as sized in Python
    from parallelizable_recurrent_units_amd import SRU_WS_BACKWARD, SruShape, sru_workspace_size
    assert int(r.stdout.strip()) == sru_workspace_size(SruShape(64, 128, 512, True, 1.0),
                                                       SRU_WS_BACKWARD)
