"""The oracle against the closed-form fixtures in tests/golden/ (cases whose
exact results follow by hand from the definitions; see
tests/golden/make_closed_forms.py for each derivation and its source)."""

import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))["cases"]


def test_golden_sconv():
    for c in [c for c in CASES if c["kind"] == "sconv"]:
        y, st = oracle.sconv_sequence(np.array(c["x"]), np.array(c["w"]), np.array(c["state"]))
        assert np.array_equal(y, np.array(c["y"])), c["cite"]
        assert np.array_equal(st, np.array(c["new_state"])), c["cite"]


def test_golden_attention():
    cases = [c for c in CASES if c["kind"] == "attention"]
    assert len(cases) == 3
    for c in cases:
        q, K, V = np.array(c["q"]), np.array(c["k"]), np.array(c["v"])
        out, lse = oracle.relattn_prefill(q, K, V, np.array(c["bias"]), c["window"], 1)
        np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-12,
                                   err_msg=c["cite"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-12,
                                   err_msg=c["cite"])
