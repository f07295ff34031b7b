"""The stored oracle digest for the small fp32 workload still reproduces (CPU)."""
import json
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_config1_oracle_digest_unchanged():
    from tests.golden.make_golden import compute
    with open(os.path.join(HERE, "golden", "config1_oracle.json")) as f:
        stored = json.load(f)
    now = compute()
    assert now["inputs_sha256"] == stored["inputs_sha256"]
    for a, b in zip(now["samples"], stored["samples"]):
        for k in ("U_f", "h", "c"):
            assert a[k] == pytest.approx(b[k], rel=1e-13, abs=1e-15)
    assert now["h_sum"] == pytest.approx(stored["h_sum"], rel=1e-12)
    assert now["c_last_sum"] == pytest.approx(stored["c_last_sum"], rel=1e-12)
