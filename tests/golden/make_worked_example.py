"""Write tests/golden/worked_example.json from the oracle (the only module this script calls).

The case is small and exact in bf16: T=1, H=2, a 4-row pool, top-k [2, -1, 0, 3]
(one invalid slot), a sink, scale 0.5. q and the pool rows are sparse
small-integer vectors, so every logit is an exact small number and the fixture
can be checked by hand against the operation's definition (the contract of the
sparse MLA training backward page: softmax over the valid gathered rows, K == V,
sink in the denominator only, lse sink-inclusive, natural log). dO is a fixed
small-integer tensor for the backward part.

    python tests/golden/make_worked_example.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from sparse_attention_top_amd import synth  # noqa: E402


def case():
    D = 512
    q = np.zeros((1, 2, D), np.float32)
    q[0, 0, 0], q[0, 0, 1] = 1.0, 2.0
    q[0, 1, 0], q[0, 1, 2] = -1.0, 1.0
    kv = np.zeros((4, D), np.float32)
    kv[0, 0], kv[0, 1] = 2.0, 0.0
    kv[1, 0] = 5.0            # never referenced
    kv[2, 1], kv[2, 2] = 1.0, 3.0
    kv[3, 0], kv[3, 2] = -1.0, 1.0
    kv[:, 3] = [1.0, 2.0, 3.0, 4.0]
    topk = np.array([[2, -1, 0, 3]], np.int32)
    sink = np.array([0.5, -1.0], np.float32)
    dout = np.zeros((1, 2, D), np.float32)
    dout[0, 0, 0], dout[0, 0, 3] = 1.0, -2.0
    dout[0, 1, 1], dout[0, 1, 2] = 3.0, 1.0
    return (synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(kv), topk, sink, synth.f32_to_bf16_bits(dout), 0.5)


def main():
    q, kv, topk, sink, dout, scale = case()
    f = oracle.forward(q, kv, topk, sink, scale)
    b = oracle.backward(q, kv, dout, f["o"], f["lse"], topk, sink, scale)
    nz = [0, 1, 2, 3]  # the only columns any input touches; the rest are 0
    out = {
        "source": "written by tests/golden/make_worked_example.py from the oracle",
        "scale": scale, "topk": topk.tolist(), "sink": sink.tolist(),
        "o_cols_0_3": f["o"][0][:, nz].tolist(), "lse": f["lse"][0].tolist(),
        "dq_cols_0_3": b["dq"][0][:, nz].tolist(), "dkv_cols_0_3": b["dkv"][:, nz].tolist(),
        "d_sink": b["d_sink"].tolist(),
    }
    with open(os.path.join(HERE, "worked_example.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
