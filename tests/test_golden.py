"""The oracle's operators against hand-derived closed-form cases stored in
tests/golden/closed_forms.json (each case carries its derivation; none was
produced by the oracle)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
CASES = json.load(open(GOLDEN))


@pytest.mark.parametrize("c", CASES["rmsnorm"])
def test_rmsnorm(c):
    y = oracle.rmsnorm(np.array(c["x"]), np.array(c["g"], dtype=np.float32), c["eps"])
    np.testing.assert_allclose(y, c["y"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("c", CASES["rope"])
def test_rope(c):
    y = oracle.rope(np.array(c["v"]), 1, c["head_dim"], c["pos"], c["theta"])
    np.testing.assert_allclose(y, c["y"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("c", CASES["softmax"])
def test_softmax(c):
    np.testing.assert_allclose(oracle.softmax(np.array(c["s"])), c["p"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("c", CASES["attention"])
def test_attention(c):
    o = oracle.attend(np.array(c["q"]), np.array(c["K"], dtype=np.float32), np.array(c["V"], dtype=np.float32))
    np.testing.assert_allclose(o, c["o"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("c", CASES["silu"])
def test_silu(c):
    assert oracle.silu(c["z"]) == pytest.approx(c["y"], rel=0, abs=1e-15)


@pytest.mark.parametrize("c", CASES["bf16"])
def test_bf16_ties(c):
    assert oracle.bf16_from_f64(c["x"]) == c["bits"]
