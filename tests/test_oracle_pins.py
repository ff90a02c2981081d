"""Pins of the CPU oracle to things other than itself (CPU only).

The pages print no worked example with values, so the oracle is pinned by
(a) a brute-force evaluation through library routines -- dense masked
attention (``torch.nn.functional.scaled_dot_product_attention`` in float64)
plus ``scipy.special.logsumexp`` for the log-sum-exp, with the sink as one
extra key of zero value; (b) closed forms; and (c) invariants of the
operation stated on the pages (slot-order independence, sink = -inf equals no
sink, all-invalid rows, poisoned unused rows, out-of-range slots).
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from sparse_attention_top_amd import synth

D = 512
INT32_MIN = -(2**31)
INT32_MAX = 2**31 - 1


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def f32(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def random_case(seed, T=6, H=5, num_kv=40, topk=24, p_invalid=0.3, sink=True):
    """Random rows without repeated valid indices; invalid slots use assorted out-of-range values."""
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((T, H, D)))
    kv = bf16(rng.standard_normal((num_kv, D)))
    idx = np.empty((T, topk), np.int32)
    bad_vals = np.array([-1, -2, INT32_MIN, num_kv, num_kv + 1, INT32_MAX], np.int64)
    for t in range(T):
        rows = rng.choice(num_kv, topk, replace=False)
        inval = rng.random(topk) < p_invalid
        rows = np.where(inval, rng.choice(bad_vals, topk), rows)
        idx[t] = rows.astype(np.int32)
    s = rng.standard_normal(H).astype(np.float32) if sink else None
    return q, kv, idx, s


def brute_force(q, kv, idx, sink, scale):
    """Dense masked attention over all rows, by library routines (float64)."""
    T, H, _ = q.shape
    num_kv = kv.shape[0]
    K = torch.from_numpy(np.vstack([f32(kv), np.zeros((1, D))]))  # extra zero-value key = sink
    o = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        valid = np.zeros(num_kv + 1, bool)
        r = idx[t].astype(np.int64)
        valid[r[(r >= 0) & (r < num_kv)]] = True
        mask = np.where(valid, 0.0, -np.inf)[None, :].repeat(H, 0)
        if sink is not None:
            mask[:, num_kv] = sink.astype(np.float64)
        rows_with_mass = np.isfinite(mask).any(axis=1)
        Q = torch.from_numpy(f32(q[t]))[:, None, :]  # [H, 1, D]
        logits = scale * (f32(q[t]) @ K.numpy().T) + mask  # [H, num_kv+1]
        out = torch.nn.functional.scaled_dot_product_attention(
            Q, K[None].expand(H, -1, -1), K[None].expand(H, -1, -1),
            attn_mask=torch.from_numpy(mask)[:, None, :], scale=scale).numpy()[:, 0, :]
        for h in range(H):
            if rows_with_mass[h]:
                o[t, h] = out[h]
                lse[t, h] = scipy.special.logsumexp(logits[h])
    return o, lse


@pytest.mark.parametrize("seed,sink", [(1, True), (2, False), (3, True)])
def test_matches_brute_force_random(seed, sink):
    q, kv, idx, s = random_case(seed, sink=sink)
    scale = synth.DEFAULT_SCALE
    r = oracle.forward(q, kv, idx, s, scale)
    o_ref, lse_ref = brute_force(q, kv, idx, s, scale)
    np.testing.assert_allclose(r["o"], o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)
    # the rounded output is the unrounded one rounded to bf16
    assert np.array_equal(r["o_bf16"], bf16(r["o"].astype(np.float32)))


def test_matches_brute_force_tiny_config():
    inp = synth.make_inputs("tiny")
    r = oracle.forward(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"])
    o_ref, lse_ref = brute_force(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"])
    np.testing.assert_allclose(r["o"], o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_ref, rtol=1e-12, atol=1e-12)
    assert int(r["n_valid"].sum()) == 1400


def test_closed_form_two_slots_and_sink():
    # q . k = 2 and 4 with scale 0.5 gives logits 1 and 2; the sink 0.5 is a
    # logit as given (it is not multiplied by scale); the natural log is used.
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    kv = np.zeros((3, D), np.float32)
    kv[0, 0], kv[0, 1] = 2.0, 1.0  # slot value a
    kv[2, 0], kv[2, 1] = 4.0, -3.0  # slot value b
    kv[1, :] = 7.0  # never referenced
    idx = np.array([[2, -1, 0]], np.int32)
    sink = np.array([0.5], np.float32)
    r = oracle.forward(bf16(q), bf16(kv), idx, sink, 0.5)
    wa, wb, ws = math.exp(1.0 - 2.0), 1.0, math.exp(0.5 - 2.0)
    Z = wa + wb + ws
    expect = (wa * kv[0].astype(np.float64) + wb * kv[2].astype(np.float64)) / Z
    np.testing.assert_allclose(r["o"][0, 0], expect, rtol=1e-14, atol=1e-15)
    assert abs(r["lse"][0, 0] - (2.0 + math.log(Z))) < 1e-14
    # without the sink
    r = oracle.forward(bf16(q), bf16(kv), idx, None, 0.5)
    Z = wa + wb
    assert abs(r["lse"][0, 0] - (2.0 + math.log(Z))) < 1e-14
    kv64 = kv.astype(np.float64)
    np.testing.assert_allclose(r["o"][0, 0], (wa * kv64[0] + wb * kv64[2]) / Z, rtol=1e-14, atol=1e-15)


def test_single_valid_slot_is_exact_gather():
    q, kv, idx, _ = random_case(11, T=8, H=3, num_kv=50, topk=16)
    rng = np.random.default_rng(5)
    idx[:] = -1
    rows = rng.choice(50, 8, replace=False)
    pos = rng.integers(0, 16, 8)
    for t in range(8):
        idx[t, pos[t]] = rows[t]
    scale = synth.DEFAULT_SCALE
    r = oracle.forward(q, kv, idx, None, scale)
    for t in range(8):
        for h in range(3):
            assert np.array_equal(r["o_bf16"][t, h], kv[rows[t]])
            x = scale * float(f32(q[t, h]) @ f32(kv[rows[t]]))
            assert abs(r["lse"][t, h] - x) < 1e-12


@pytest.mark.parametrize("with_sink", [False, True])
def test_zero_query_counts_valid_slots(with_sink):
    q, kv, idx, s = random_case(21, T=10, H=2, num_kv=64, topk=40, p_invalid=0.4, sink=with_sink)
    q[:] = 0
    r = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    for t in range(10):
        rr = idx[t].astype(np.int64)
        sel = rr[(rr >= 0) & (rr < 64)]
        n = sel.size
        assert r["n_valid"][t] == n
        mean = f32(kv[sel]).mean(axis=0)
        for h in range(2):
            if with_sink:
                es = math.exp(float(s[h]))
                assert abs(r["lse"][t, h] - math.log(n + es)) < 1e-12
                np.testing.assert_allclose(r["o"][t, h], mean * n / (n + es), rtol=1e-12, atol=1e-14)
            else:
                assert abs(r["lse"][t, h] - math.log(n)) < 1e-12
                np.testing.assert_allclose(r["o"][t, h], mean, rtol=1e-12, atol=1e-14)


def test_permutation_invariance():
    q, kv, idx, s = random_case(31, T=5, H=4, num_kv=80, topk=48)
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(48) for _ in range(5)])
    idx_p = np.take_along_axis(idx, perm, axis=1)
    a = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    b = oracle.forward(q, kv, idx_p, s, synth.DEFAULT_SCALE)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-13)
    assert np.array_equal(a["n_valid"], b["n_valid"])


def test_sink_minus_inf_equals_no_sink():
    q, kv, idx, s = random_case(41, T=6, H=4, num_kv=40, topk=24)
    idx[2, :] = -1  # an all-invalid row too
    s[:] = -np.inf
    a = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    b = oracle.forward(q, kv, idx, None, synth.DEFAULT_SCALE)
    assert np.array_equal(a["o_bf16"], b["o_bf16"])
    assert np.array_equal(a["o"], b["o"])
    assert np.array_equal(a["lse"], b["lse"])


def test_all_invalid_rows():
    q, kv, idx, s = random_case(51, T=4, H=3, num_kv=40, topk=24)
    idx[1] = -1
    idx[3] = np.array([40, INT32_MAX, INT32_MIN, -2] * 6, np.int32)
    a = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    b = oracle.forward(q, kv, idx, None, synth.DEFAULT_SCALE)
    for t in (1, 3):
        assert np.all(a["o_bf16"][t] == 0) and np.all(b["o_bf16"][t] == 0)
        assert np.all(a["o"][t] == 0.0) and not np.signbit(a["o"][t]).any()
        assert np.array_equal(a["lse"][t], s.astype(np.float64))
        assert np.all(np.isneginf(b["lse"][t]))
        assert a["n_valid"][t] == 0


def test_poisoned_unused_rows_do_not_leak():
    q, kv, idx, s = random_case(61, T=6, H=4, num_kv=60, topk=20)
    # keep row 0 unreferenced by any valid slot, as in the pages' poison test
    idx[(idx == 0)] = -1
    kv_big = np.vstack([kv, bf16(np.zeros((1, D)))])  # one extra row right past num_kv
    used = np.zeros(60, bool)
    r = idx.astype(np.int64)
    used[r[(r >= 0) & (r < 60)]] = True
    base = oracle.forward(q, kv_big[:60], idx, s, synth.DEFAULT_SCALE)
    poison = kv_big.copy()
    poison[np.flatnonzero(~used)[0::2]] = synth.BF16_NAN
    poison[np.flatnonzero(~used)[1::2]] = bf16(np.full(D, np.inf))
    poison[60] = synth.BF16_NAN
    got = oracle.forward(q, poison[:60], idx, s, synth.DEFAULT_SCALE)
    assert np.array_equal(base["o_bf16"], got["o_bf16"])
    assert np.array_equal(base["lse"], got["lse"])


def test_out_of_range_slots_behave_as_minus_one():
    q, kv, idx, s = random_case(71, T=6, H=3, num_kv=40, topk=30, p_invalid=0.0)
    rng = np.random.default_rng(3)
    bad = rng.random(idx.shape) < 0.35
    vals = np.array([-2, INT32_MIN, 40, 41, INT32_MAX], np.int64)
    idx_bad = np.where(bad, rng.choice(vals, idx.shape), idx).astype(np.int32)
    idx_m1 = np.where(bad, -1, idx).astype(np.int32)
    a = oracle.forward(q, kv, idx_bad, s, synth.DEFAULT_SCALE)
    b = oracle.forward(q, kv, idx_m1, s, synth.DEFAULT_SCALE)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    assert np.array_equal(a["n_valid"], b["n_valid"])


def test_duplicate_slot_counts_twice():
    q, kv, idx, _ = random_case(81, T=3, H=2, num_kv=30, topk=8)
    idx[:] = -1
    idx[:, 1] = 7
    one = oracle.forward(q, kv, idx, None, synth.DEFAULT_SCALE)
    idx[:, 5] = 7
    two = oracle.forward(q, kv, idx, None, synth.DEFAULT_SCALE)
    np.testing.assert_allclose(two["lse"], one["lse"] + math.log(2.0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(two["o"], one["o"], rtol=1e-15, atol=0)


def test_head_independence():
    q, kv, idx, s = random_case(91, T=4, H=7, num_kv=50, topk=20)
    full = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    for h in range(7):
        one = oracle.forward(np.ascontiguousarray(q[:, h:h + 1]), kv, idx, s[h:h + 1], synth.DEFAULT_SCALE)
        assert np.array_equal(one["o"][:, 0], full["o"][:, h])
        assert np.array_equal(one["lse"][:, 0], full["lse"][:, h])


def test_large_logits_stay_finite_and_convex():
    q, kv, idx, s = random_case(101, T=4, H=3, num_kv=50, topk=20)
    qb = bf16(f32(q) * 100.0)
    r = oracle.forward(qb, kv, idx, s, synth.DEFAULT_SCALE)
    assert np.all(np.isfinite(r["o"])) and np.all(np.isfinite(r["lse"]))
    for t in range(4):
        rr = idx[t].astype(np.int64)
        V = f32(kv[rr[(rr >= 0) & (rr < 50)]])
        lo = np.minimum(V.min(axis=0), 0.0)
        hi = np.maximum(V.max(axis=0), 0.0)
        assert np.all(r["o"][t] >= lo[None] - 1e-12) and np.all(r["o"][t] <= hi[None] + 1e-12)


def test_empty_shapes():
    q = np.zeros((0, 4, D), np.uint16)
    r = oracle.forward(q, np.zeros((3, D), np.uint16), np.zeros((0, 5), np.int32), None, 0.1)
    assert r["o"].shape == (0, 4, D) and r["lse"].shape == (0, 4)
    # empty pool: every slot invalid
    q = bf16(np.ones((2, 2, D)))
    r = oracle.forward(q, np.zeros((0, D), np.uint16), np.array([[0, -1], [1, 2]], np.int32),
                       np.array([0.25, -np.inf], np.float32), 0.1)
    assert np.all(r["o"] == 0) and np.all(r["lse"][:, 0] == np.float64(np.float32(0.25)))
    assert np.all(np.isneginf(r["lse"][:, 1]))


def test_nan_in_referenced_row_stays_local():
    q, kv, idx, s = random_case(111, T=5, H=2, num_kv=40, topk=16)
    rr = idx[2].astype(np.int64)
    victim = int(rr[(rr >= 0) & (rr < 40)][0])
    kv[victim, 3] = synth.BF16_NAN
    r = oracle.forward(q, kv, idx, s, synth.DEFAULT_SCALE)
    for t in range(5):
        refs = victim in set(idx[t].tolist())
        assert np.isnan(r["lse"][t]).all() == refs
        assert (~np.isfinite(r["o"][t])).any() == refs


def test_int64_indices_match_brute_force_and_never_wrap():
    """int64 top-k rows: values at or past 2^31 that an int32 cast would wrap onto valid rows
    (2^32 + r wraps to r) stay invalid; the result equals brute force on the same rows."""
    q, kv, idx32, s = random_case(41, T=5, H=3, num_kv=40, topk=20, p_invalid=0.0)
    idx = idx32.astype(np.int64)
    rng = np.random.default_rng(42)
    wrap = rng.random(idx.shape) < 0.3
    idx[wrap] = idx[wrap] + 2**32          # would alias the same row after a cast to int32
    idx[0, :3] = [2**31, -(2**40), 2**62]
    ref = oracle.forward(q, kv, idx, s, 0.07)
    bo, bl = brute_force(q, kv, idx, s, 0.07)
    np.testing.assert_allclose(ref["o"], bo, rtol=0, atol=1e-10)
    np.testing.assert_allclose(ref["lse"], bl, rtol=0, atol=1e-10)
    # the same as int32 rows with those slots marked -1, bit for bit
    idx_m = np.where((idx >= 0) & (idx < 40), idx, -1).astype(np.int32)
    ref32 = oracle.forward(q, kv, idx_m, s, 0.07)
    assert np.array_equal(ref["o"], ref32["o"]) and np.array_equal(ref["lse"], ref32["lse"])
    assert np.array_equal(ref["n_valid"], ((idx >= 0) & (idx < 40)).sum(axis=1))


# ---- fp8 (OCP E4M3) pools with one dequant scale ----

def fp8_decode_torch(codes):
    """Library decode of OCP FP8 E4M3 codes (torch's float8_e4m3fn), float64."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def brute_force_f64pool(q, pool, idx, sink, scale):
    """brute_force() on a float64 pool (dense masked attention by library routines)."""
    T, H, _ = q.shape
    num_kv = pool.shape[0]
    K = torch.from_numpy(np.vstack([pool, np.zeros((1, D))]))
    o = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        valid = np.zeros(num_kv + 1, bool)
        r = idx[t].astype(np.int64)
        valid[r[(r >= 0) & (r < num_kv)]] = True
        mask = np.where(valid, 0.0, -np.inf)[None, :].repeat(H, 0)
        if sink is not None:
            mask[:, num_kv] = sink.astype(np.float64)
        Q = torch.from_numpy(f32(q[t]))[:, None, :]
        logits = scale * (f32(q[t]) @ K.numpy().T) + mask
        out = torch.nn.functional.scaled_dot_product_attention(
            Q, K[None].expand(H, -1, -1), K[None].expand(H, -1, -1),
            attn_mask=torch.from_numpy(mask)[:, None, :], scale=scale).numpy()[:, 0, :]
        for h in range(H):
            if np.isfinite(mask[h]).any():
                o[t, h] = out[h]
                lse[t, h] = scipy.special.logsumexp(logits[h])
    return o, lse


def test_fp8_decode_matches_library_for_every_code():
    """A single valid slot and q = 0 return the row itself: every non-NaN code, times the scale,
    must equal torch's own decode of the format (subnormals, both zeros, the largest values)."""
    codes = np.arange(256, dtype=np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, 0, codes)  # NaN codes are covered by the NaN test
    pool = np.vstack([np.concatenate([codes, codes[::-1]])[None, :], np.full((1, D), 0x38, np.uint8)])
    q = np.zeros((1, 2, D), np.uint16)
    idx = np.array([[0, -1]], np.int32)
    for kv_scale in (1.0, 0.375, 2.0 ** -9):
        ref = oracle.forward(q, pool, idx, None, 0.1, kv_scale=kv_scale)
        want = fp8_decode_torch(pool[0]) * kv_scale
        assert np.array_equal(ref["o"][0, 0], want) and np.array_equal(ref["o"][0, 1], want)
        assert np.all(ref["lse"] == 0.0)


@pytest.mark.parametrize("seed,sink", [(51, True), (52, False)])
def test_fp8_pool_matches_brute_force(seed, sink):
    q, _, idx, s = random_case(seed, T=5, H=4, num_kv=40, topk=24, sink=sink)
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (40, D)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, 0x3A, codes)  # no NaN codes here
    kv_scale = 0.0625
    ref = oracle.forward(q, codes, idx, s, 0.05, kv_scale=kv_scale)
    bo, bl = brute_force_f64pool(q, fp8_decode_torch(codes) * kv_scale, idx, s, 0.05)
    np.testing.assert_allclose(ref["o"], bo, rtol=0, atol=1e-10)
    np.testing.assert_allclose(ref["lse"], bl, rtol=0, atol=1e-10)


def test_fp8_nan_codes_stay_local():
    """A NaN code (0x7F or 0xFF) in a referenced row makes that token NaN; in an unreferenced row it
    changes nothing."""
    q, _, idx, s = random_case(53, T=4, H=3, num_kv=30, topk=10, p_invalid=0.0)
    rng = np.random.default_rng(53)
    codes = rng.integers(0, 0x70, (30, D)).astype(np.uint8)
    base = oracle.forward(q, codes, idx, s, 0.05, kv_scale=0.5)
    unused = np.setdiff1d(np.arange(30), idx.ravel())
    poisoned = codes.copy()
    poisoned[unused, 5] = 0x7F
    r_used = idx[2, 3]
    poisoned[r_used, 7] = 0xFF
    ref = oracle.forward(q, poisoned, idx, s, 0.05, kv_scale=0.5)
    hit = np.array([(idx[t] == r_used).any() for t in range(4)])
    assert np.all(np.isnan(ref["o"][hit])) and np.all(np.isnan(ref["lse"][hit]))
    assert np.array_equal(ref["o"][~hit], base["o"][~hit]) and np.array_equal(ref["lse"][~hit], base["lse"][~hit])
