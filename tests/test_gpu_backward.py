"""Backward parity: the HIP path (through the C ABI) against the backward oracle.

Both sides get the same inputs: q, kv, top-k rows, sink, a seeded dO, and the
forward's o (bf16) and lse (fp32) as the GPU forward produced them.

Tolerance, from the arithmetic: every term of a gradient element passes
through bf16 at most three times on the GPU (P and scale dS enter their MFMAs
in bf16; a slot's dkv contribution is stored in bf16; dq and dkv are stored in
bf16), each a relative error of at most 2^-9, while the fp32 parts are ~2^-24.
So |d| <= 6 * 2^-9 * mag + 1e-6 * max(mag) elementwise, mag being the sum of
the absolute values of the element's terms (the oracle reports it), and the
cosine similarity of each tensor with the oracle's must be >= 0.9999 (the
pages' backward checks cos > 0.999). NaN patterns must match.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_top_amd import sparse_mla_backward, synth

from gpu_util import DEV, bf16_bits, run_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

G_MAG = 6 * 2.0**-9
G_COS = 0.9999


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def check_grad(got, ref, mag, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs" % what
    g, r, m = got[~nan_ref], ref[~nan_ref], mag[~nan_ref]
    if r.size == 0:
        return
    err = np.abs(g - r)
    bound = G_MAG * m + 1e-6 * float(m.max())
    bad = err > bound
    worst = int(np.argmax(err / np.maximum(bound, 1e-300)))
    assert not bad.any(), "%s: %d of %d out of tolerance (worst: err %.3g, mag %.3g, ref %.3g)" % (
        what, int(bad.sum()), r.size, float(err[worst]), float(m[worst]), float(r[worst]))
    nr, ng = np.linalg.norm(r), np.linalg.norm(g)
    if nr > 0:
        cos = float(np.dot(g, r) / (nr * ng))
        assert cos >= G_COS, "%s: cosine %.6f" % (what, cos)
    else:
        assert np.all(g == 0), "%s: reference is zero, got nonzero" % what


def run_backward(q, kv, dout, o_bits, lse, topk, sink, scale, chunk_tokens=None, idx_dtype=np.int32, kv_scale=None):
    qd, dd, od = to_dev_bf16(q), to_dev_bf16(dout), to_dev_bf16(o_bits)
    if kv_scale is not None:  # OCP FP8 E4M3 codes
        kvd = torch.from_numpy(np.ascontiguousarray(kv, dtype=np.uint8)).to(DEV).view(torch.float8_e4m3fn)
    else:
        kvd = to_dev_bf16(kv) if kv.shape[0] else torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    ld = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(DEV)
    td = torch.from_numpy(np.ascontiguousarray(topk, dtype=idx_dtype)).to(DEV)
    sd = None if sink is None else torch.from_numpy(np.ascontiguousarray(sink, dtype=np.float32)).to(DEV)
    dq, dkv, ds = sparse_mla_backward(qd, kvd, dd, od, ld, td, sd, scale, chunk_tokens=chunk_tokens, kv_scale=kv_scale)
    torch.cuda.synchronize()
    return (f64(bf16_bits(dq)), f64(bf16_bits(dkv)) if kv.shape[0] else np.zeros((0, 512)),
            None if ds is None else ds.cpu().numpy().astype(np.float64))


def full_case(q, kv, topk, sink, scale, seed, what, tokens=None, rows=None, chunk_tokens=None, kv_scale=None):
    """GPU forward, then GPU backward and oracle backward on the same inputs; compare."""
    print("backward case %s: T=%d H=%d topk=%d num_kv=%d sink=%s" % (
        what, q.shape[0], q.shape[1], topk.shape[1], kv.shape[0], sink is not None), flush=True)
    rng = np.random.default_rng(seed)
    dout = bf16(rng.standard_normal(q.shape))
    o_bits, lse = run_gpu(q, kv, topk, sink, scale, kv_scale=kv_scale)
    dq, dkv, ds = run_backward(q, kv, dout, o_bits, lse, topk, sink, scale, chunk_tokens, kv_scale=kv_scale)
    ref = oracle.backward(q, kv, dout, o_bits, lse, topk, sink, scale, tokens=tokens, rows=rows, want_mag=True,
                          kv_scale=kv_scale)
    check_grad(dq if tokens is None else dq[tokens], ref["dq"], ref["dq_mag"], what + " dq")
    check_grad(dkv if rows is None else dkv[rows], ref["dkv"], ref["dkv_mag"], what + " dkv")
    if sink is not None:
        check_grad(ds, ref["d_sink"], ref["d_sink_mag"], what + " d_sink")
    else:
        assert ds is None
    return dq, dkv, ds


def random_case(seed, T, H, topk, num_kv, p_invalid=0.2, sink=True, dup=False):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((T, H, 512)))
    kv = bf16(rng.standard_normal((num_kv, 512)))
    idx = np.empty((T, topk), np.int32)
    for t in range(T):
        rows = rng.choice(num_kv, topk, replace=dup or topk > num_kv).astype(np.int64)
        bad = rng.random(topk) < p_invalid
        rows[bad] = rng.choice(np.array([-1, num_kv, num_kv + 5, -(2**31), 2**31 - 1], np.int64), bad.sum())
        idx[t] = rows.astype(np.int32)
    s = rng.standard_normal(H).astype(np.float32) if sink else None
    return q, kv, idx, s


def test_backward_tiny_config():
    inp = synth.make_inputs("tiny")
    full_case(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], 1, "tiny")


@pytest.mark.parametrize("H,topk,sink,dup", [(128, 96, True, False), (64, 40, False, True), (100, 70, True, False),
                                             (8, 40, True, False), (24, 33, False, False), (16, 5, True, True)])
def test_backward_random(H, topk, sink, dup):
    q, kv, idx, s = random_case(H * 7 + topk, T=40, H=H, topk=topk, num_kv=300, sink=sink, dup=dup)
    full_case(q, kv, idx, s, synth.DEFAULT_SCALE, H + topk, "random H=%d topk=%d" % (H, topk))


@pytest.mark.parametrize("H,topk", [(17, 50), (32, 64), (33, 48), (65, 40), (127, 36)])
def test_backward_head_count_edges(H, topk):
    """The dq phase runs 1, 2 or 4 waves of 16 heads (H <= 16, <= 32, above) and more than 64 heads as two
    groups; the interm contraction pads H to a multiple of 16. One head past each step (17, 33, 65: a wave or a
    group holding a single real head), 32 exactly, and 127 (the last group one head short)."""
    q, kv, idx, s = random_case(H * 11 + topk, T=40, H=H, topk=topk, num_kv=300, sink=True, dup=False)
    full_case(q, kv, idx, s, synth.DEFAULT_SCALE, 3 * H + topk, "edge H=%d topk=%d" % (H, topk))


@pytest.mark.parametrize("H,chunk", [(16, None), (128, None), (64, 24)])
def test_backward_fp8_pool(H, chunk):
    """A pool of fp8 codes (every code value but NaN: both signs, subnormals, the largest) with a dequant scale:
    the GPU decodes it to bf16 code values and folds the scale into the logits, dP and dq; checked against the
    oracle on the decoded values, in one pass and in several."""
    q, _, idx, s = random_case(31 + H, T=48, H=H, topk=96, num_kv=300)
    rng = np.random.default_rng(32 + H)
    codes = rng.integers(0, 256, (300, 512)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, 0x30, codes)
    full_case(q, codes, idx, s, synth.DEFAULT_SCALE, 33 + H, "fp8 H=%d" % H, chunk_tokens=chunk, kv_scale=0.03)


def test_backward_multi_segment_row():
    """Rows longer than one 2048-entry compaction segment."""
    q, kv, idx, s = random_case(5, T=6, H=16, topk=2500, num_kv=3000, p_invalid=0.3)
    full_case(q, kv, idx, s, synth.DEFAULT_SCALE, 6, "topk 2500")


def test_backward_all_invalid_and_heavy_rows():
    """Tokens with no valid slot, and a row every token references many times."""
    q, kv, idx, s = random_case(9, T=32, H=16, topk=64, num_kv=200, p_invalid=0.1)
    idx[3] = -1
    idx[17] = 200
    idx[:, 5:12] = 7  # row 7: seven slots per token
    full_case(q, kv, idx, s, 0.07, 10, "invalid + heavy rows")


def test_backward_empty_topk_and_zero_tokens():
    q, kv, idx, s = random_case(11, T=8, H=16, topk=4, num_kv=50)
    idx0 = np.zeros((8, 0), np.int32)
    dq, dkv, ds = full_case(q, kv, idx0, s, synth.DEFAULT_SCALE, 12, "topk 0")
    assert np.all(dq == 0) and np.all(dkv == 0) and np.all(ds == 0)
    q0 = np.zeros((0, 16, 512), np.uint16)
    dq, dkv, ds = run_backward(q0, kv, q0, q0, np.zeros((0, 16), np.float32), np.zeros((0, 4), np.int32), s,
                               synth.DEFAULT_SCALE)
    assert dq.shape == (0, 16, 512) and np.all(dkv == 0) and np.all(ds == 0)


@pytest.mark.parametrize("T,H,topk,chunk,dup", [(40, 128, 96, 7, False), (33, 16, 70, 1, True),
                                                (64, 64, 128, 64, True), (50, 100, 40, 16, True)])
def test_backward_token_passes(T, H, topk, chunk, dup):
    """The backward in passes of `chunk` tokens (dkv summed across passes in
    fp32) against the oracle, and against the single-pass call: dq and d_sink
    are per token and come out bit-identical, dkv within the tolerance."""
    q, kv, idx, s = random_case(T * 3 + chunk, T=T, H=H, topk=topk, num_kv=250, sink=True, dup=dup)
    idx[:, :4] = 11  # a row shared by every pass
    what = "passes of %d: T=%d H=%d topk=%d" % (chunk, T, H, topk)
    dq, dkv, ds = full_case(q, kv, idx, s, synth.DEFAULT_SCALE, T + H, what, chunk_tokens=chunk)
    rng = np.random.default_rng(T + H)
    dout = bf16(rng.standard_normal(q.shape))
    o_bits, lse = run_gpu(q, kv, idx, s, synth.DEFAULT_SCALE)
    dq1, dkv1, ds1 = run_backward(q, kv, dout, o_bits, lse, idx, s, synth.DEFAULT_SCALE)
    assert np.array_equal(dq, dq1), what + ": dq differs from the single pass"
    assert np.array_equal(ds, ds1), what + ": d_sink differs from the single pass"


@pytest.mark.parametrize("H,chunk", [(16, None), (128, None), (16, 24)])
def test_backward_int64_rows_bitwise(H, chunk):
    """int64 rows, some of them 2^32 + r (which an int32 cast would turn into row r), 2^31 or large negatives: the
    gradients equal the int32 backward's on the equivalent rows (invalid -> -1) bit for bit, in one pass or several."""
    q, kv, idx, s = random_case(21 + H, T=64, H=H, topk=96, num_kv=300)
    rng = np.random.default_rng(22 + H)
    i64 = np.asarray(idx).astype(np.int64)
    wrap = (rng.random(i64.shape) < 0.2) & (i64 >= 0)
    i64[wrap] += 2**32
    i64[:, 0] = 2**31
    i64[:, 1] = -(2**40)
    i32 = np.where((i64 >= 0) & (i64 < 300), i64, -1).astype(np.int32)
    dout = bf16(rng.standard_normal(q.shape))
    o_bits, lse = run_gpu(q, kv, i32, s, synth.DEFAULT_SCALE)
    a = run_backward(q, kv, dout, o_bits, lse, i32, s, synth.DEFAULT_SCALE, chunk)
    b = run_backward(q, kv, dout, o_bits, lse, i64, s, synth.DEFAULT_SCALE, chunk, idx_dtype=np.int64)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_is_deterministic():
    q, kv, idx, s = random_case(13, T=64, H=128, topk=128, num_kv=400, dup=True)
    rng = np.random.default_rng(14)
    dout = bf16(rng.standard_normal(q.shape))
    o_bits, lse = run_gpu(q, kv, idx, s, synth.DEFAULT_SCALE)
    a = run_backward(q, kv, dout, o_bits, lse, idx, s, synth.DEFAULT_SCALE)
    b = run_backward(q, kv, dout, o_bits, lse, idx, s, synth.DEFAULT_SCALE)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("chunk", [None, 1000])
def test_backward_wide_full_size_sampled(chunk):
    """The wide workload (T=4096, H=128, topk=512) at full size, in one pass and
    in five token passes: dq of sampled tokens, dkv of sampled rows (window rows
    and heavily shared pool rows), and d_sink over all tokens, against the
    oracle."""
    inp = synth.make_inputs("wide")
    T = inp["T"]
    tokens = np.linspace(0, T - 1, 24).astype(np.int64)
    num_kv = inp["kv"].shape[0]
    rows = np.array([0, 1, T // 2, T - 1, T, T + 1, T + 300, num_kv - 1], np.int64)
    full_case(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], 15, "wide sampled (passes of %s)" % chunk,
              tokens=tokens, rows=rows, chunk_tokens=chunk)


@pytest.mark.parametrize("name", ["long", "tp4"])
def test_backward_full_size_sampled(name):
    """The backward page's T=8192 shape (H=128, topk=512, 9216 pool rows) and the
    16-head tp4 shape at full size: sampled tokens' dq, window and pool rows' dkv,
    d_sink over all tokens."""
    inp = synth.make_inputs(name)
    T = inp["T"]
    num_kv = inp["kv"].shape[0]
    tokens = np.linspace(0, T - 1, 16).astype(np.int64)
    rows = np.array([0, T // 3, T - 1, T, T + 7, (T + num_kv) // 2, num_kv - 1], np.int64)
    full_case(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], 17, name + " sampled", tokens=tokens,
              rows=rows)


def test_backward_one_head_and_minus_inf_sinks():
    q, kv, idx, _ = random_case(21, T=24, H=1, topk=48, num_kv=120)
    full_case(q, kv, idx, np.array([0.3], np.float32), 0.1, 22, "H=1")
    q, kv, idx, s = random_case(23, T=24, H=40, topk=48, num_kv=120)
    s[::3] = -np.inf  # those heads behave as if they had no sink: d_sink 0
    _, _, ds = full_case(q, kv, idx, s, synth.DEFAULT_SCALE, 24, "-inf sinks")
    assert np.all(ds[::3] == 0.0)


def test_backward_nan_rows():
    """NaN in a referenced row reaches exactly what the oracle says (the NaN
    pattern must match); NaN in rows no slot holds changes nothing at all."""
    q, kv, idx, s = random_case(25, T=32, H=16, topk=40, num_kv=200)
    referenced = np.unique(idx[(idx >= 0) & (idx < 200)])
    unref = np.setdiff1d(np.arange(200), referenced)
    assert unref.size > 0
    rng = np.random.default_rng(26)
    dout = bf16(rng.standard_normal(q.shape))
    o_bits, lse = run_gpu(q, kv, idx, s, synth.DEFAULT_SCALE)
    clean = run_backward(q, kv, dout, o_bits, lse, idx, s, synth.DEFAULT_SCALE)
    poisoned = kv.copy()
    poisoned[unref] = synth.BF16_NAN
    dirty = run_backward(q, poisoned, dout, o_bits, lse, idx, s, synth.DEFAULT_SCALE)
    for a, b in zip(clean, dirty):
        assert np.array_equal(a, b)
    assert np.all(clean[1][unref] == 0.0)
    kv_nan = kv.copy()
    kv_nan[referenced[0], 7] = synth.BF16_NAN
    full_case(q, kv_nan, idx, s, synth.DEFAULT_SCALE, 27, "NaN in a referenced row")
