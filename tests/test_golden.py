"""The worked example in tests/golden/ (CPU only).

worked_example.json was written from the oracle by make_worked_example.py. The
test recomputes it (any later change to the oracle's arithmetic shows here) and
checks the forward part against the example worked by hand: head 0 of the
token has q = (1, 2, 0, ...), its valid slots hold rows 2, 0, 3 =
(0, 1, 3, 3), (2, 0, 0, 1), (-1, 0, 1, 4) in the first four columns, so with
scale 0.5 its logits are 1, 1 and -1/2, and with its sink 1/2 the softmax
denominator is 2e + e^-1/2 + e^1/2.
"""
import json
import math
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

import importlib.util  # noqa: E402

_spec = importlib.util.spec_from_file_location("make_worked_example", os.path.join(HERE, "make_worked_example.py"))
_mod = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_mod)


def load():
    with open(os.path.join(HERE, "worked_example.json")) as fh:
        return json.load(fh)


def test_worked_example_forward_by_hand():
    g = load()
    z = 2 * math.e + math.exp(-0.5) + math.exp(0.5)
    assert abs(g["lse"][0] - math.log(z)) < 1e-12
    rows = {2: [0, 1, 3, 3], 0: [2, 0, 0, 1], 3: [-1, 0, 1, 4]}
    w = {2: math.e / z, 0: math.e / z, 3: math.exp(-0.5) / z}
    want = [sum(w[r] * rows[r][d] for r in rows) for d in range(4)]
    np.testing.assert_allclose(g["o_cols_0_3"][0], want, rtol=0, atol=1e-12)


def test_worked_example_matches_oracle():
    g = load()
    q, kv, topk, sink, dout, scale = _mod.case()
    f = oracle.forward(q, kv, topk, sink, scale)
    b = oracle.backward(q, kv, dout, f["o"], f["lse"], topk, sink, scale)
    np.testing.assert_allclose(f["o"][0][:, :4], g["o_cols_0_3"], rtol=0, atol=1e-12)
    assert np.all(f["o"][0][:, 4:] == 0)
    np.testing.assert_allclose(f["lse"][0], g["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["dq"][0][:, :4], g["dq_cols_0_3"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["dkv"][:, :4], g["dkv_cols_0_3"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["d_sink"], g["d_sink"], rtol=0, atol=1e-12)
    assert np.all(b["dkv"][1] == 0)  # row 1 is in the pool but no slot holds it
