"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes the oracle finishes in seconds are compared element by element for every
token; the full-size workloads (the launch the benchmark times) are compared
on sampled tokens, which always include the first and last token and the
tokens with the fewest and most valid slots.
"""

import math

import numpy as np
import pytest
import torch

from sparse_attention_top_amd import fp8_pool_decoded, set_fp8_pool_decode, synth

from gpu_util import DEV, compare, oracle_ref, run_case, run_gpu

pytestmark = pytest.mark.gpu

_FULL = {}


def full_case(name):
    """Generate a full-size workload once per session and run the GPU on it once."""
    if name not in _FULL:
        inp = synth.make_inputs(name)
        o, lse = run_case(inp)
        _FULL[name] = (inp, o, lse)
    return _FULL[name]


def sample_tokens(topk, num_kv, k, seed):
    T = topk.shape[0]
    nv = ((topk >= 0) & (topk < num_kv)).sum(axis=1)
    rng = np.random.default_rng(seed)
    pick = {0, T - 1, int(np.argmin(nv)), int(np.argmax(nv))}
    pick.update(rng.choice(T, size=min(T, k), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def test_tiny_all_tokens():
    inp = synth.make_inputs("tiny")
    o, lse = run_case(inp)
    stats = compare(o, lse, oracle_ref(inp), what="tiny")
    print("tiny", stats)


@pytest.mark.parametrize("name,T", [("small", None), ("tp4", 768), ("wide", 384), ("large", 320), ("glm", 512)])
def test_truncated_all_tokens(name, T):
    """Same draw recipe at a size the oracle covers fully (several tiles and a ragged tail per token)."""
    inp = synth.make_inputs(name, T=T)
    o, lse = run_case(inp)
    stats = compare(o, lse, oracle_ref(inp), what="%s T=%s" % (name, inp["T"]))
    print(name, inp["T"], stats)


@pytest.mark.parametrize("name,k", [("small", None), ("tp4", None), ("wide", None), ("large", 256), ("glm", 256)])
def test_full_size(name, k):
    """The benchmarked launches at full size: every token of small, tp4 and wide
    against the oracle, 256 sampled tokens of large and glm."""
    inp, o, lse = full_case(name)
    tok = None if k is None else sample_tokens(inp["topk"], inp["num_kv"], k, seed=7)
    ref = oracle_ref(inp, tokens=tok)
    stats = compare(o, lse, ref, tokens=tok, what="%s full" % name)
    print(name, "full", inp["T"] if tok is None else len(tok), "tokens", stats)


def test_full_size_properties():
    """Properties over every token of the full-size workloads: finite outputs and an lse
    no smaller than the sink (the denominator holds exp(sink))."""
    for name in ("small", "tp4", "wide", "large", "glm"):
        inp, o, lse = full_case(name)
        of = synth.bf16_bits_to_f32(o)
        assert np.all(np.isfinite(of)), name
        assert np.all(np.isfinite(lse)), name
        if inp["sink"] is not None:
            assert np.all(lse >= inp["sink"][None, :] - 1e-3), name


def test_rerun_is_bitwise_deterministic_and_out_reuse():
    inp = synth.make_inputs("wide", T=200)
    o1, l1 = run_case(inp)
    o2, l2 = run_case(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    # writing into caller buffers (pre-filled with garbage) gives the same bits
    out = torch.full((inp["T"], inp["H"], 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((inp["T"], inp["H"]), 12345.0, dtype=torch.float32, device=DEV)
    o3, l3 = run_gpu(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], out=out, lse=lse)
    assert np.array_equal(o1, o3) and np.array_equal(l1.view(np.uint32), l3.view(np.uint32))


def random_rows(rng, T, topk, num_kv, p_invalid):
    idx = np.empty((T, topk), np.int32)
    for t in range(T):
        idx[t] = rng.choice(num_kv, topk, replace=False)
    idx[rng.random((T, topk)) < p_invalid] = -1
    return idx


def make_random(seed, T, H, num_kv, topk, p_invalid=0.2, sink=True):
    rng = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits(rng.standard_normal((T, H, 512), dtype=np.float32))
    kv = synth.f32_to_bf16_bits(rng.standard_normal((num_kv, 512), dtype=np.float32))
    idx = random_rows(rng, T, topk, num_kv, p_invalid)
    s = rng.standard_normal(H).astype(np.float32) if sink else None
    return {"q": q, "kv": kv, "topk": idx, "sink": s, "scale": synth.DEFAULT_SCALE}


@pytest.mark.parametrize("H", [1, 3, 8, 16, 17, 24, 40, 64, 100, 128, 130, 200])
def test_head_counts(H):
    inp = make_random(1000 + H, T=24, H=H, num_kv=300, topk=96)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="H=%d" % H)


@pytest.mark.parametrize("T,H", [(100, 128), (1000, 128), (260, 200)])
def test_h128_persistent_schedule(T, H):
    """The persistent 128-head kernel deals units (token, group of 128 heads) to its workgroups by XCD when the grid
    is a multiple of the eight XCDs, and one unit per run of the grid otherwise. Top-k rows of 96 entries keep every
    shape on that kernel (the split path needs 128): a grid of 100 (not a multiple of 8), 1000 units on 256
    workgroups (a partial fourth run of 232), and 260 tokens of two head groups (520 units: a last run of 8). Every
    unit must be computed exactly once: all tokens are compared."""
    inp = make_random(2700 + T + H, T=T, H=H, num_kv=1500, topk=96, p_invalid=0.2)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="H=%d T=%d" % (H, T))


H16_EDGES = [(15, 40, 0.0), (16, 40, 0.0), (17, 40, 0.0), (512, 900, 0.0), (513, 900, 0.0), (640, 900, 0.0),
             (641, 900, 0.0), (1039, 2000, 0.0), (1100, 2000, 0.5), (1281, 2000, 0.0)]


@pytest.mark.parametrize("topk,num_kv,p_invalid", H16_EDGES)
def test_h16_tile_and_segment_edges(topk, num_kv, p_invalid):
    """H <= 16 runs 16-row tiles from 640-entry compaction segments: counts one short of, at and one past a tile and
    a segment, rows of two and three segments with a partial tile, and one where half the slots are invalid
    (segments whose valid counts are not multiples of 16); 512 and 513 are the edges of an earlier segment size.
    300 tokens: more (token, head group) units than the MI355X's 256 CUs, so every row takes the single-pass 16-row
    kernel, not the split path."""
    inp = make_random(2500 + topk, T=300, H=16, num_kv=num_kv, topk=topk, p_invalid=p_invalid)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="H=16 topk=%d" % topk)


def test_h128_rows_over_several_segments():
    """The H = 128 D-split workgroup compacts rows in 1024-entry segments: rows of 1500 entries (two segments, the
    second partial) on the single pass (300 tokens x 2 head groups), compared on sampled tokens."""
    inp = make_random(2600, T=300, H=128, num_kv=2000, topk=1500, p_invalid=0.3)
    o, lse = run_case(inp)
    tok = np.arange(0, 300, 15)
    compare(o, lse, oracle_ref(inp, tokens=tok), tokens=tok, what="H=128 topk=1500")


@pytest.mark.parametrize("topk,p_invalid", [(1023, 0.0), (1024, 0.0), (1025, 0.0), (1025, 0.3)])
def test_h128_kernel_switch_at_list_capacity(topk, p_invalid):
    """The persistent 128-head kernel compacts a whole top-k row into one 1024-entry list; a longer row goes to the
    D-split kernel (two 64-head groups, 1024-entry segments). Rows one short of, at and one past that capacity with
    every slot valid, and one past it with 30% of the slots invalid (fewer valid slots than the capacity: the kernel
    is chosen by the row length, so still the D-split one). 300 tokens keep the single pass; sampled tokens."""
    from sparse_attention_top_amd import kernel_name

    assert kernel_name(128, topk) == ("smla_fwd128_kernel" if topk <= 1024 else "smla_fwd_kernel<4, 2>")
    inp = make_random(2800 + topk + int(10 * p_invalid), T=300, H=128, num_kv=3000, topk=topk, p_invalid=p_invalid)
    o, lse = run_case(inp)
    tok = np.arange(0, 300, 13)
    compare(o, lse, oracle_ref(inp, tokens=tok), tokens=tok, what="H=128 topk=%d p_invalid=%.1f" % (topk, p_invalid))


@pytest.mark.parametrize("topk,num_kv", [(1, 50), (31, 40), (33, 100), (2048, 3000), (2500, 4000), (4500, 6000)])
def test_topk_extremes(topk, num_kv):
    """Single slots, tile-boundary counts and rows longer than one compaction segment."""
    inp = make_random(2000 + topk, T=6, H=16, num_kv=num_kv, topk=topk, p_invalid=0.1)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="topk=%d" % topk)


@pytest.mark.parametrize("name,T", [("wide", 160), ("tp4", 300)])
def test_permutation_invariance(name, T):
    inp = synth.make_inputs(name, T=T)
    rng = np.random.default_rng(3)
    perm = np.stack([rng.permutation(inp["topk_n"]) for _ in range(inp["T"])])
    inp_p = dict(inp, topk=np.take_along_axis(inp["topk"], perm, axis=1))
    o1, l1 = run_case(inp)
    o2, l2 = run_case(inp_p)
    compare(o2, l2, oracle_ref(inp), what="permuted")
    assert np.max(np.abs(l1 - l2)) <= 1e-3


def test_sink_minus_inf_equals_no_sink():
    inp = make_random(5, T=20, H=16, num_kv=200, topk=64)
    inp["topk"][3] = -1  # an all-invalid row
    o1, l1 = run_gpu(inp["q"], inp["kv"], inp["topk"], np.full(16, -np.inf, np.float32), inp["scale"])
    o2, l2 = run_gpu(inp["q"], inp["kv"], inp["topk"], None, inp["scale"])
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("H", [16, 128])
def test_all_invalid_rows(H):
    inp = make_random(6, T=8, H=H, num_kv=100, topk=40)
    inp["topk"][2] = -1
    inp["topk"][5] = np.array([100, 2**31 - 1, -(2**31), -2] * 10, np.int32)
    o, l = run_case(inp)
    o_ns, l_ns = run_gpu(inp["q"], inp["kv"], inp["topk"], None, inp["scale"])
    for t in (2, 5):
        assert np.all(o[t] == 0) and np.all(o_ns[t] == 0)  # exactly +0.0
        assert np.array_equal(l[t], inp["sink"])
        assert np.all(np.isneginf(l_ns[t]))


def test_empty_pool_and_empty_topk():
    inp = make_random(7, T=4, H=16, num_kv=10, topk=8)
    o, l = run_gpu(inp["q"], np.zeros((0, 512), np.uint16), inp["topk"], inp["sink"], inp["scale"])
    assert np.all(o == 0) and np.array_equal(l, np.broadcast_to(inp["sink"], l.shape))
    o, l = run_gpu(inp["q"], inp["kv"], np.zeros((4, 0), np.int32), None, inp["scale"])
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_zero_sequence():
    q = torch.empty((0, 16, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((5, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    from sparse_attention_top_amd import sparse_mla_prefill

    o, l = sparse_mla_prefill(q, kv, idx)
    assert o.shape == (0, 16, 512) and l.shape == (0, 16)


@pytest.mark.parametrize("H", [16, 128])
def test_single_valid_slot_is_exact_gather(H):
    """One valid slot: P = 1 exactly, so o is the gathered row bit for bit (16-row and D-split kernels)."""
    inp = make_random(8, T=40, H=H, num_kv=500, topk=64, sink=False)
    rng = np.random.default_rng(9)
    rows = rng.choice(500, 40, replace=False)
    inp["topk"][:] = -1
    inp["topk"][np.arange(40), rng.integers(0, 64, 40)] = rows
    o, l = run_case(inp)
    for t in range(40):
        assert np.array_equal(o[t], np.broadcast_to(inp["kv"][rows[t]], (H, 512)))


@pytest.mark.parametrize("name,T", [("large", 600), ("tp4", 300)])
@pytest.mark.parametrize("sink", [False, True])
def test_zero_query_counts_exact_valid_slots(sink, name, T):
    """q = 0 makes every logit 0, so lse = ln(n) (or ln(n + e^sink)): the count n of
    gathered slots is pinned exactly (neighbouring counts differ by > 9e-4), on the
    H = 128 D-split kernel and the H = 16 16-row kernel."""
    inp = synth.make_inputs(name, T=T)
    inp["q"][:] = 0
    if not sink:
        inp["sink"] = None
    o, l = run_case(inp)
    n = ((inp["topk"] >= 0) & (inp["topk"] < inp["num_kv"])).sum(axis=1).astype(np.float64)
    if sink:
        expect = np.log(n[:, None] + np.exp(inp["sink"].astype(np.float64))[None, :])
    else:
        expect = np.log(n)[:, None]
    assert np.max(np.abs(l - expect)) < 2e-4


@pytest.mark.parametrize("H", [16, 128])
def test_poisoned_unused_rows_and_out_of_range_slots(H):
    """Rows no valid slot references (row 0 included, and the row just past
    num_kv inside the same allocation) are filled with NaN/Inf, and invalid
    slots take -2, INT32_MIN, num_kv, num_kv+1, INT32_MAX: bitwise the same
    output as the clean run with -1 (16-row and D-split kernels)."""
    inp = make_random(10, T=32, H=H, num_kv=400, topk=96, p_invalid=0.0)
    rng = np.random.default_rng(11)
    inp["topk"][inp["topk"] == 0] = 1  # row 0 unreferenced
    inp["topk"] = np.where(inp["topk"] == 1, -1, inp["topk"]).astype(np.int32)
    bad = rng.random(inp["topk"].shape) < 0.3
    clean_idx = np.where(bad, -1, inp["topk"]).astype(np.int32)
    vals = np.array([-2, -(2**31), 400, 401, 2**31 - 1], np.int64)
    dirty_idx = np.where(bad, rng.choice(vals, bad.shape), inp["topk"]).astype(np.int32)
    o1, l1 = run_gpu(inp["q"], inp["kv"], clean_idx, inp["sink"], inp["scale"])
    used = np.zeros(401, bool)
    used[clean_idx[clean_idx >= 0]] = True
    kv_p = np.vstack([inp["kv"], np.zeros((1, 512), np.uint16)])
    unused = np.flatnonzero(~used)
    kv_p[unused[0::2]] = synth.BF16_NAN
    kv_p[unused[1::2]] = np.uint16(0x7F80)  # +inf
    kvd = torch.from_numpy(kv_p.view(np.int16)).view(torch.bfloat16).to(DEV)[:400]  # row 400 poisoned, past the pool
    from gpu_util import bf16_bits, to_dev_bf16
    from sparse_attention_top_amd import sparse_mla_prefill

    o2, l2 = sparse_mla_prefill(to_dev_bf16(inp["q"]), kvd, torch.from_numpy(dirty_idx).to(DEV),
                                torch.from_numpy(inp["sink"]).to(DEV), inp["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(o1, bf16_bits(o2))
    assert np.array_equal(l1.view(np.uint32), l2.cpu().numpy().view(np.uint32))


def test_duplicate_slots_count_each_occurrence():
    inp = make_random(12, T=16, H=16, num_kv=100, topk=48)
    inp["topk"][:, 40:48] = inp["topk"][:, 0:8]  # repeats (valid or not)
    o, l = run_case(inp)
    compare(o, l, oracle_ref(inp), what="duplicates")


def test_head_independence():
    inp = make_random(13, T=12, H=40, num_kv=200, topk=80)
    o, l = run_case(inp)
    for h in (0, 17, 39):
        o1, l1 = run_gpu(np.ascontiguousarray(inp["q"][:, h:h + 1]), inp["kv"], inp["topk"], inp["sink"][h:h + 1],
                         inp["scale"])
        a = synth.bf16_bits_to_f32(o1[:, 0]).astype(np.float64)
        b = synth.bf16_bits_to_f32(o[:, h]).astype(np.float64)
        assert np.all(np.abs(a - b) <= 2e-2 + 2e-2 * np.abs(b))
        assert np.max(np.abs(l1[:, 0] - l[:, h])) <= 1e-3


@pytest.mark.parametrize("H,T,topk,mult", [(16, 16, 64, 100.0), (128, 260, 200, 100.0), (128, 260, 200, 10.0)])
def test_large_logits_stay_finite(H, T, topk, mult):
    """Logits of spread 10 to 100 move the lazy reference max across tiles, so earlier tiles' sums are rescaled: in
    the 16-row kernel in place, in the H = 128 D-split kernel by factors the owner waves publish to every wave
    (260 tokens: single pass, 7 tiles per row)."""
    inp = make_random(14, T=T, H=H, num_kv=400, topk=topk)
    inp["q"] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp["q"]) * mult)
    o, l = run_case(inp)
    assert np.all(np.isfinite(synth.bf16_bits_to_f32(o))) and np.all(np.isfinite(l))
    compare(o, l, oracle_ref(inp), what="large logits")


@pytest.mark.parametrize("scale", [0.0, -0.05, 1.0])
def test_any_finite_scale(scale):
    inp = make_random(15, T=12, H=16, num_kv=150, topk=64)
    inp["scale"] = scale
    o, l = run_case(inp)
    compare(o, l, oracle_ref(inp), what="scale=%g" % scale)


@pytest.mark.parametrize("name", ["tp4", "wide"])
def test_nan_in_referenced_row_stays_local(name):
    """A NaN in one referenced row reaches exactly the tokens that reference it (all their heads), on the 16-row
    kernel (tp4) and the D-split kernel (wide: the NaN enters S and P.V in every wave of both head groups)."""
    inp = synth.make_inputs(name, T=300)
    victim = 250  # a token row inside the windows of tokens 250..299 only (windows of at least 50 tokens)
    inp["kv"][victim, 7] = synth.BF16_NAN
    o, l = run_case(inp)
    refs = np.array([victim in set(r.tolist()) for r in inp["topk"]])
    of = synth.bf16_bits_to_f32(o)
    assert np.array_equal(np.isnan(l).all(axis=1), refs) and np.array_equal(np.isnan(l).any(axis=1), refs)
    assert np.array_equal(np.isnan(of).any(axis=(1, 2)), refs)
    ok = ~refs
    tok = np.flatnonzero(ok)[::7]
    compare(o, l, oracle_ref(inp, tokens=tok), tokens=tok, what="nan locality")


def test_kv_inside_large_allocation():
    """kv placed more than 4 GiB into one allocation: 64-bit row addressing."""
    inp = synth.make_inputs("tp4", T=256)
    nbytes = inp["kv"].nbytes
    offset = (4 << 30) + 4096
    try:
        big = torch.empty(offset + nbytes, dtype=torch.uint8, device=DEV)
    except RuntimeError:
        pytest.skip("not enough device memory for the >4 GiB placement")
    kv_view = big[offset:offset + nbytes].view(torch.bfloat16).view(-1, 512)
    kv_view.copy_(torch.from_numpy(inp["kv"].view(np.int16)).view(torch.bfloat16))
    from gpu_util import bf16_bits, to_dev_bf16
    from sparse_attention_top_amd import sparse_mla_prefill

    o, l = sparse_mla_prefill(to_dev_bf16(inp["q"]), kv_view, torch.from_numpy(inp["topk"]).to(DEV),
                              torch.from_numpy(inp["sink"]).to(DEV), inp["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = run_case(inp)
    assert np.array_equal(bf16_bits(o), o_ref)
    assert np.array_equal(l.cpu().numpy().view(np.uint32), l_ref.view(np.uint32))
    del big


def test_binding_rejects_bad_inputs():
    from sparse_attention_top_amd import sparse_mla_prefill

    q = torch.zeros((4, 16, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((10, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((4, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(RuntimeError, match="kv dtype mismatch"):
        sparse_mla_prefill(q, kv.float(), idx)
    with pytest.raises(RuntimeError, match="bfloat16"):
        sparse_mla_prefill(q.half(), kv, idx)
    with pytest.raises(RuntimeError, match="int32 or int64"):
        sparse_mla_prefill(q, kv, idx.short())
    with pytest.raises(RuntimeError, match="GPU"):
        sparse_mla_prefill(q.cpu(), kv, idx)
    with pytest.raises(RuntimeError, match="contiguous"):
        sparse_mla_prefill(q, kv, idx, out=torch.empty((16, 4, 512), dtype=torch.bfloat16, device=DEV).transpose(0, 1))
    with pytest.raises(RuntimeError, match="attn_sink"):
        sparse_mla_prefill(q, kv, idx, attn_sink=torch.zeros(16, device=DEV, dtype=torch.float64))
    with pytest.raises(RuntimeError, match="scale"):
        sparse_mla_prefill(q, kv, idx, scale=math.inf)


# ---- few tokens: each top-k row is split over several workgroups, then merged ----

@pytest.mark.parametrize("T,H,topk,num_kv", [(1, 16, 640, 20480), (2, 16, 2048, 4096), (4, 128, 1024, 9216),
                                             (8, 64, 4500, 6000), (16, 16, 640, 2000), (3, 200, 1500, 3000),
                                             (5, 8, 600, 900), (12, 32, 777, 1000)])
def test_split_rows_few_tokens(T, H, topk, num_kv):
    inp = make_random(3000 + T * 7 + H, T=T, H=H, num_kv=num_kv, topk=topk, p_invalid=0.15)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="split T=%d H=%d topk=%d" % (T, H, topk))


@pytest.mark.parametrize("sink", [False, True])
def test_split_rows_with_empty_splits(sink):
    """Rows whose valid slots sit in one split, or nowhere: empty splits carry no mass and an
    all-invalid row gives o = 0 and lse = sink (or -inf) exactly."""
    rng = np.random.default_rng(77)
    T, H, topk, num_kv = 4, 16, 1024, 2000
    inp = make_random(78, T=T, H=H, num_kv=num_kv, topk=topk, p_invalid=0.0, sink=sink)
    idx = inp["topk"]
    idx[0, :] = -1                       # no valid slot at all
    idx[1, :-1] = -1                     # one valid slot, in the last split
    idx[2, 300:] = num_kv + 5            # valid slots only at the front (out-of-range values elsewhere)
    idx[3, rng.random(topk) < 0.5] = -1  # random half
    o, lse = run_case(inp)
    ref = oracle_ref(inp)
    compare(o, lse, ref, what="split empty sink=%s" % sink)
    assert np.all(synth.bf16_bits_to_f32(o[0]) == 0.0)
    if sink:
        assert np.array_equal(lse[0], inp["sink"])
    else:
        assert np.all(lse[0] == -np.inf)


def test_decode_workload_full():
    """The decode-sized call (last 16 tokens of the tp4 sequence) against the oracle, every token."""
    inp = synth.make_inputs("decode")
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="decode")


# ---- int64 top-k rows ----

@pytest.mark.parametrize("T,H,topk,num_kv", [(40, 16, 300, 1000), (24, 128, 512, 2000), (3, 16, 1024, 4000),
                                             (300, 16, 640, 2000), (300, 8, 1281, 3000), (40, 16, 100, 500)])
def test_int64_indices_never_wrap(T, H, topk, num_kv):
    """int64 rows: values 2^32 + r (which an int32 cast would turn into row r), 2^31 and large
    negatives are invalid; the result equals the oracle and, bitwise, the int32 path on the
    equivalent rows (invalid -> -1). At H <= 16 in a single pass (300 tokens, or rows under 128
    entries) the 16-row kernel reads the int64 rows itself, over one, two or three list segments;
    the other shapes convert the rows first."""
    inp = make_random(5000 + T + H, T=T, H=H, num_kv=num_kv, topk=topk, p_invalid=0.1)
    rng = np.random.default_rng(T * H)
    idx = inp["topk"].astype(np.int64)
    wrap = (rng.random(idx.shape) < 0.25) & (idx >= 0)
    idx[wrap] += 2**32
    idx[:, 0] = 2**31
    idx[:, 1] = -(2**40)
    o64, l64 = run_gpu(inp["q"], inp["kv"], idx, inp["sink"], inp["scale"])
    ref = oracle_ref(dict(inp, topk=idx))
    compare(o64, l64, ref, what="int64 T=%d H=%d" % (T, H))
    idx32 = np.where((idx >= 0) & (idx < num_kv), idx, -1).astype(np.int32)
    o32, l32 = run_gpu(inp["q"], inp["kv"], idx32, inp["sink"], inp["scale"])
    assert np.array_equal(o64, o32) and np.array_equal(l64.view(np.uint32), l32.view(np.uint32))


def test_int64_rows_full_size_tp4_bitwise():
    """tp4 at full size with its rows as int64 and every invalid entry written as 2^32 + 5 (row 5 after an int32
    cast): the 16-row kernel reads them itself, and the result equals the int32 call bit for bit."""
    inp, o32, l32 = full_case("tp4")
    idx = inp["topk"].astype(np.int64)
    idx[idx < 0] = 2**32 + 5
    o64, l64 = run_gpu(inp["q"], inp["kv"], idx, inp["sink"], inp["scale"])
    assert np.array_equal(o64, o32) and np.array_equal(l64.view(np.uint32), l32.view(np.uint32))


# ---- fp8 (OCP E4M3) pools ----
# Each case runs both ways an fp8 pool is read: by the fp8 kernels ("direct")
# and decoded once per call into a bf16 copy for the bf16 kernels ("decoded").

@pytest.fixture(params=["direct", "decoded"])
def fp8_path(request):
    prev = set_fp8_pool_decode("never" if request.param == "direct" else "always")
    yield request.param
    set_fp8_pool_decode(prev)


@pytest.mark.parametrize("name,T", [("tiny_fp8", None), ("tp4_fp8", 768), ("wide_fp8", 384), ("glm_fp8", 512)])
def test_fp8_pool_truncated_all_tokens(name, T, fp8_path):
    inp = synth.make_inputs(name, T=T)
    o, lse = run_case(inp)
    stats = compare(o, lse, oracle_ref(inp), what="%s T=%s" % (name, inp["T"]))
    print(name, inp["T"], stats)


@pytest.mark.parametrize("name,k,decoded", [("tp4_fp8", 32, True), ("glm_fp8", 16, False)])
def test_fp8_pool_full_size_sampled(name, k, decoded):
    """At full size under the default mode: tp4's 20 MiB pool is decoded, glm's 2.1 GiB paged pool is not."""
    inp, o, lse = full_case(name)
    assert fp8_pool_decoded(inp["T"], inp["topk_n"], inp["num_kv"]) == decoded
    tok = sample_tokens(inp["topk"], inp["num_kv"], k, seed=9)
    compare(o, lse, oracle_ref(inp, tokens=tok), tokens=tok, what="%s full" % name)


def make_random_fp8(seed, T, H, num_kv, topk, p_invalid=0.15, sink=True, kv_scale=0.03):
    rng = np.random.default_rng(seed)
    inp = make_random(seed, T=T, H=H, num_kv=num_kv, topk=topk, p_invalid=p_invalid, sink=sink)
    codes = rng.integers(0, 256, (num_kv, 512)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, 0x30, codes)  # NaN codes only where a test puts them
    return dict(inp, kv=codes, kv_scale=kv_scale)


@pytest.mark.parametrize("T,H,topk,num_kv", [(20, 16, 300, 900), (16, 128, 200, 600), (3, 16, 1024, 3000),
                                             (2, 128, 777, 2000), (9, 40, 96, 300), (12, 24, 150, 500),
                                             (7, 65, 96, 400)])
def test_fp8_pool_random(T, H, topk, num_kv, fp8_path):
    """Random rows and every code value (subnormals, both signs, the largest); few-token shapes
    take the split path."""
    inp = make_random_fp8(6000 + T + H, T, H, num_kv, topk)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="fp8 T=%d H=%d topk=%d" % (T, H, topk))


@pytest.mark.parametrize("topk,num_kv,p_invalid", H16_EDGES)
def test_fp8_h16_tile_and_segment_edges(topk, num_kv, p_invalid, fp8_path):
    """The fp8 16-row kernel (8 KiB slab tiles, 512-entry segments) at the same tile and segment edges, single pass
    (300 tokens)."""
    inp = make_random_fp8(7500 + topk, 300, 16, num_kv, topk, p_invalid=p_invalid)
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="fp8 H=16 topk=%d" % topk)


def test_fp8_nan_code_stays_local_and_invalid_rows(fp8_path):
    inp = make_random_fp8(6100, T=12, H=16, num_kv=400, topk=64, p_invalid=0.1)
    idx = inp["topk"]
    idx[0, :] = -1                                   # no valid slot
    unused = np.setdiff1d(np.arange(400), idx.ravel())
    inp["kv"][unused[:5], 3] = 0x7F                   # NaN codes in unreferenced rows: no effect
    r = idx[5][idx[5] >= 0][0]
    inp["kv"][r, 100] = 0xFF                          # NaN code in a referenced row
    o, lse = run_case(inp)
    compare(o, lse, oracle_ref(inp), what="fp8 NaN")
    hit = np.array([(idx[t] == r).any() for t in range(12)])
    of = synth.bf16_bits_to_f32(o)
    assert np.all(np.isnan(of[hit])) and np.all(np.isfinite(of[~hit]))
    assert np.all(of[0] == 0.0) and np.array_equal(lse[0], inp["sink"])
