"""Pins of the backward oracle to things other than itself (CPU only).

(a) torch's automatic differentiation through a dense per-slot formulation of
the forward built from library routines (``index_select`` of the slot rows,
``matmul``, ``softmax`` / ``logsumexp`` with the sink as one extra logit
column), in float64; (b) central finite differences of the forward oracle
(itself pinned in test_oracle_pins.py) for the sink gradient; (c) closed forms
and invariants: one valid slot without a sink gives dq = 0 and dkv = the sum of
dO over heads; rows no slot holds get dkv = 0; every gradient is linear in dO.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_top_amd import synth

D = 512


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def case(seed, T=5, H=3, num_kv=24, topk=10, p_invalid=0.25, sink=True, dup=False):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((T, H, D)))
    kv = bf16(rng.standard_normal((num_kv, D)))
    dout = bf16(rng.standard_normal((T, H, D)))
    idx = np.empty((T, topk), np.int32)
    for t in range(T):
        rows = rng.choice(num_kv, topk, replace=dup).astype(np.int64)
        bad = rng.random(topk) < p_invalid
        rows[bad] = rng.choice(np.array([-1, num_kv, num_kv + 7, -(2**31)], np.int64), bad.sum())
        idx[t] = rows.astype(np.int32)
    s = rng.standard_normal(H).astype(np.float32) if sink else None
    return q, kv, dout, idx, s


def autograd_reference(q, kv, dout, idx, sink, scale):
    """Forward and gradients by torch autograd (float64), one token at a time."""
    T, H, _ = q.shape
    num_kv = kv.shape[0]
    Q = torch.tensor(f64(q), requires_grad=True)
    K = torch.tensor(f64(kv), requires_grad=True)
    S = torch.tensor(sink.astype(np.float64), requires_grad=True) if sink is not None else None
    dO = torch.tensor(f64(dout))
    o = torch.zeros((T, H, D), dtype=torch.float64)
    lse = torch.full((T, H), -np.inf, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    outs = []
    for t in range(T):
        r = idx[t].astype(np.int64)
        r = r[(r >= 0) & (r < num_kv)]
        if r.size == 0 and S is None:
            outs.append((None, None))
            continue
        Kt = K.index_select(0, torch.from_numpy(r))              # [n, D], one row per valid slot
        logits = scale * (Q[t] @ Kt.T)                           # [H, n]
        if S is not None:
            logits = torch.cat([logits, S[:, None]], dim=1)      # the sink: one more logit, no value row
        p = torch.softmax(logits, dim=1)
        ot = p[:, : r.size] @ Kt                                 # [H, D]
        lt = torch.logsumexp(logits, dim=1)
        loss = loss + (ot * dO[t]).sum()
        outs.append((ot.detach(), lt.detach()))
    loss.backward()
    for t, (ot, lt) in enumerate(outs):
        if ot is not None:
            o[t] = ot
            lse[t] = lt
    dq = Q.grad.numpy() if Q.grad is not None else np.zeros(Q.shape)
    dkv = K.grad.numpy() if K.grad is not None else np.zeros(K.shape)
    ds = S.grad.numpy() if S is not None and S.grad is not None else (np.zeros(S.shape) if S is not None else None)
    return o.numpy(), lse.numpy(), dq, dkv, ds


@pytest.mark.parametrize("seed,sink,dup", [(1, True, False), (2, False, False), (3, True, True), (4, False, True)])
def test_backward_matches_autograd(seed, sink, dup):
    q, kv, dout, idx, s = case(seed, sink=sink, dup=dup)
    scale = synth.DEFAULT_SCALE
    o, lse, dq, dkv, ds = autograd_reference(q, kv, dout, idx, s, scale)
    r = oracle.backward(q, kv, dout, o, lse, idx, s, scale)
    np.testing.assert_allclose(r["dq"], dq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["dkv"], dkv, rtol=1e-9, atol=1e-12)
    if sink:
        np.testing.assert_allclose(r["d_sink"], ds, rtol=1e-9, atol=1e-12)
    else:
        assert r["d_sink"] is None


def test_backward_matches_autograd_tiny_config():
    inp = synth.make_inputs("tiny")
    rng = np.random.default_rng(7)
    dout = bf16(rng.standard_normal(inp["q"].shape))
    o, lse, dq, dkv, ds = autograd_reference(inp["q"], inp["kv"], dout, inp["topk"], inp["sink"], inp["scale"])
    r = oracle.backward(inp["q"], inp["kv"], dout, o, lse, inp["topk"], inp["sink"], inp["scale"])
    np.testing.assert_allclose(r["dq"], dq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["dkv"], dkv, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["d_sink"], ds, rtol=1e-9, atol=1e-12)


def test_sink_gradient_matches_finite_differences_of_forward_oracle():
    """d_sink[h] = dL/dsink[h] with L = sum(o * dO), o from the forward oracle."""
    q, kv, dout, idx, s = case(11, T=6, H=4)
    scale = 0.05
    f = oracle.forward(q, kv, idx, s, scale)
    r = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, scale)
    g = f64(dout)
    for h in range(4):
        sp, sm = s.copy(), s.copy()
        sp[h] = np.float32(s[h] + np.float32(1e-3))
        sm[h] = np.float32(s[h] - np.float32(1e-3))
        lp = (oracle.forward(q, kv, idx, sp, scale)["o"] * g).sum()
        lm = (oracle.forward(q, kv, idx, sm, scale)["o"] * g).sum()
        fd = (lp - lm) / (float(sp[h]) - float(sm[h]))
        assert abs(fd - r["d_sink"][h]) <= 1e-6 * max(1.0, abs(fd)), (h, fd, r["d_sink"][h])


def test_single_slot_closed_form():
    """One valid slot, no sink: P = 1 and o = that row, so dS = 0: dq = 0 and
    dkv[row] = sum over heads of dO."""
    q, kv, dout, idx, _ = case(21, T=3, H=4, topk=6, p_invalid=0.0)
    idx[:] = -1
    idx[0, 3], idx[1, 0], idx[2, 5] = 7, 9, 7
    f = oracle.forward(q, kv, idx, None, 0.3)
    r = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, None, 0.3)
    assert np.all(r["dq"] == 0.0)
    g = f64(dout)
    want7 = np.zeros(D)
    for t in (0, 2):
        for h in range(4):
            want7 = want7 + g[t, h]
    want9 = np.zeros(D)
    for h in range(4):
        want9 = want9 + g[1, h]
    np.testing.assert_allclose(r["dkv"][7], want7, rtol=1e-15, atol=0)
    np.testing.assert_allclose(r["dkv"][9], want9, rtol=1e-15, atol=0)
    others = [i for i in range(kv.shape[0]) if i not in (7, 9)]
    assert np.all(r["dkv"][others] == 0.0)


def test_unreferenced_rows_and_linearity_in_dout():
    q, kv, dout, idx, s = case(31, num_kv=40)
    f = oracle.forward(q, kv, idx, s, 0.1)
    r1 = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, 0.1)
    referenced = np.unique(idx[(idx >= 0) & (idx < 40)])
    unref = np.setdiff1d(np.arange(40), referenced)
    assert unref.size > 0 and np.all(r1["dkv"][unref] == 0.0)
    dout2 = bf16(2.0 * f64(dout))  # exact doubling of every bf16 value
    r2 = oracle.backward(q, kv, dout2, f["o"], f["lse"], idx, s, 0.1)
    for k in ("dq", "dkv", "d_sink"):
        assert np.array_equal(r2[k], 2.0 * r1[k]), k


def test_magnitudes_bound_the_gradients():
    """|gradient| <= sum of |terms|, with equality where every term has one sign
    (P dO terms of a row held by one slot of one head: H = 1, one token)."""
    q, kv, dout, idx, s = case(51, num_kv=30)
    f = oracle.forward(q, kv, idx, s, 0.2)
    r = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, 0.2, want_mag=True)
    for k in ("dq", "dkv", "d_sink"):
        assert np.all(np.abs(r[k]) <= r[k + "_mag"] * (1 + 1e-12) + 1e-300), k
    plain = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, 0.2)
    for k in ("dq", "dkv", "d_sink"):
        assert np.array_equal(plain[k], r[k]), k
    q1, kv1, dout1, idx1, _ = case(52, T=1, H=1, topk=4, p_invalid=0.0)
    idx1[0] = [3, -1, -1, -1]
    f1 = oracle.forward(q1, kv1, idx1, None, 0.2)
    r1 = oracle.backward(q1, kv1, dout1, f1["o"], f1["lse"], idx1, None, 0.2, want_mag=True)
    np.testing.assert_allclose(r1["dkv_mag"][3], np.abs(r1["dkv"][3]), rtol=1e-15)


def test_selected_tokens_and_rows_match_full_evaluation():
    q, kv, dout, idx, s = case(41, T=7, num_kv=30)
    f = oracle.forward(q, kv, idx, s, 0.2)
    full = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, 0.2)
    part = oracle.backward(q, kv, dout, f["o"], f["lse"], idx, s, 0.2, tokens=[5, 1], rows=[29, 3, 0])
    assert np.array_equal(part["dq"], full["dq"][[5, 1]])
    assert np.array_equal(part["dkv"], full["dkv"][[29, 3, 0]])


@pytest.mark.parametrize("seed", [41, 42])
def test_fp8_pool_equals_bf16_pool_of_the_same_values(seed):
    """An fp8 pool with a power-of-two dequant scale holds values that bf16 represents exactly (an E4M3 code value
    has at most four significant bits): the fp8 form must give, bit for bit, the bf16 form's gradients on the pool of
    those values (decoded here by torch's float8_e4m3fn, to which the forward oracle's decoding is pinned)."""
    rng = np.random.default_rng(seed)
    q, _, dout, idx, s = case(seed, T=4, H=3, num_kv=20, topk=9)
    codes = rng.integers(0, 256, (20, D)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, 0x3C, codes)  # no NaN codes
    kv_scale = 2.0 ** -4
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy() * np.float32(kv_scale)
    kv_bf16 = bf16(vals)
    assert np.array_equal(f64(kv_bf16), vals.astype(np.float64))  # exact in bf16
    fwd = oracle.forward(q, kv_bf16, idx, s, synth.DEFAULT_SCALE, want_bf16=False)
    a = oracle.backward(q, kv_bf16, dout, fwd["o"], fwd["lse"], idx, s, synth.DEFAULT_SCALE)
    b = oracle.backward(q, codes, dout, fwd["o"], fwd["lse"], idx, s, synth.DEFAULT_SCALE, kv_scale=kv_scale)
    for k in ("dq", "dkv", "d_sink"):
        assert np.array_equal(a[k], b[k]), k
