"""The seeded input generator: structure, counts and determinism (CPU only)."""

import numpy as np
import pytest

from sparse_attention_top_amd import synth

# Valid-slot totals: for window W, pool P and compression c the count is
# sum_t min(t+1, W) + min((t+1)//c, P), independent of which pool rows the rng
# picks. Written out here as numbers so that a change of recipe is caught.
EXPECTED_VALID = {"tiny": 1400, "tp4": 9952832, "wide": 1793728, "large": 5994368}
SMALL_VALID_BEFORE_DROPS = 251872


def closed_form_valid(cfg):
    t = np.arange(cfg.T)
    return int(np.minimum(t + 1, cfg.window).sum() + np.minimum((t + 1) // cfg.compression, cfg.pool_slots).sum())


@pytest.mark.parametrize("name", ["tiny", "small", "tp4", "wide", "large"])
def test_valid_counts_closed_form(name):
    cfg = synth.CONFIGS[name]
    n = closed_form_valid(cfg)
    if name == "small":
        assert n == SMALL_VALID_BEFORE_DROPS
    else:
        assert n == EXPECTED_VALID[name]


@pytest.mark.parametrize("name", ["tiny", "small", "wide"])
def test_topk_structure(name):
    cfg = synth.CONFIGS[name]
    rng = np.random.default_rng(7)
    idx = synth.build_topk(rng, cfg.T, cfg.topk, cfg.window, cfg.pool_slots, cfg.compression)
    assert idx.shape == (cfg.T, cfg.topk) and idx.dtype == np.int32
    assert synth.valid_slot_count(idx, cfg.num_kv) == closed_form_valid(cfg)
    W, P, c, T = cfg.window, cfg.pool_slots, cfg.compression, cfg.T
    for t in range(0, T, max(1, T // 97)):
        row = idx[t]
        win = row[:W]
        exp_win = np.arange(t - W + 1, t + 1)
        assert np.array_equal(win, np.where(exp_win >= 0, exp_win, -1))
        assert row[W - 1] == t  # the token's own row is always in its window
        pool = row[W:W + P]
        pool = pool[pool >= 0]
        assert np.all(np.diff(pool) > 0)  # sorted, no duplicates
        j = pool - T
        assert np.all(j >= 0) and np.all(c * (j + 1) <= t + 1)  # causally visible
        assert pool.size == min((t + 1) // c, P)
        assert np.all(row[W + P:] == -1)


def closed_form_valid_paged(cfg):
    t = np.arange(cfg.T)
    return int(np.minimum(t + 1, cfg.window).sum() + np.minimum(np.maximum(t + 1 - cfg.window, 0), cfg.pool_slots).sum())


def test_paged_layout_counts_and_structure():
    cfg = synth.CONFIGS["glm"]
    assert closed_form_valid_paged(cfg) == 31458304  # written out: catches a change of recipe
    inp = synth.make_inputs("glm", T=700)
    idx, kv, W, P = inp["topk"], inp["kv"], cfg.window, cfg.pool_slots
    assert inp["num_kv"] == cfg.pool_rows and inp["num_kv"] * 1024 > 2 * 2**30  # the pool is over 2 GiB
    small = synth.dataclasses.replace(cfg, T=700)
    assert synth.valid_slot_count(idx, inp["num_kv"]) == closed_form_valid_paged(small)
    assert np.all((idx == -1) | ((idx >= 0) & (idx < inp["num_kv"])))
    # the token's own row: its row is the last window slot, and it is the only slot holding it
    own = idx[:, W - 1]
    assert np.all(own >= 0) and len(set(own.tolist())) == 700
    for t in range(0, 700, 37):
        row = idx[t]
        valid = row[row >= 0]
        assert len(set(valid.tolist())) == valid.size  # distinct rows
        assert valid.size == min(t + 1, W) + min(max(t + 1 - W, 0), P)
        assert np.all(row[W + P:] == -1)
    # referenced rows carry the sequence's values, the rest of the pool is zero
    ref = np.unique(idx[idx >= 0])
    assert ref.size == 700
    assert not np.all(kv[ref] == 0)
    untouched = np.setdiff1d(np.arange(0, inp["num_kv"], 997), ref)
    assert np.all(kv[untouched] == 0)


def test_fp8_pool_draw():
    """The fp8 configs keep the bf16 configs' draws: same q and rows; the pool is the same kv draw
    as OCP FP8 E4M3 codes of x / s (s = max|x| / 448), within fp8 rounding of the bf16 values."""
    import torch

    a, b = synth.make_inputs("tiny"), synth.make_inputs("tiny_fp8")
    assert b["kv"].dtype == np.uint8 and b["kv_scale"] > 0
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["topk"], b["topk"])
    dec = torch.from_numpy(b["kv"]).view(torch.float8_e4m3fn).double().numpy() * b["kv_scale"]
    x = synth.bf16_bits_to_f32(a["kv"]).astype(np.float64)
    assert np.all(np.abs(dec - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * b["kv_scale"] + 2.0 ** -8 * np.abs(x))
    g = synth.make_inputs("glm_fp8", T=300)
    assert g["kv"].dtype == np.uint8 and g["kv"].shape == (2_200_000, 512)


def test_deterministic_and_seeded():
    a = synth.make_inputs("tiny")
    b = synth.make_inputs("tiny")
    assert synth.fingerprint(a) == synth.fingerprint(b)
    other = synth.make_inputs(synth.Config("x", T=64, H=16, topk=32, window=16, pool_slots=16,
                                           compression=4, seed=999))
    assert synth.fingerprint(other) != synth.fingerprint(a)


def test_small_config_drops_and_nan_rows():
    inp = synth.make_inputs("small")
    idx, kv, T = inp["topk"], inp["kv"], inp["T"]
    n = synth.valid_slot_count(idx, inp["num_kv"])
    frac = 1.0 - n / idx.size
    assert 0.08 < frac < 0.12  # "about 10%" invalid
    assert np.all(idx[:, inp["config"].window - 1] == np.arange(T))  # own slot never dropped
    used = np.zeros(inp["num_kv"], bool)
    used[idx[idx >= 0]] = True
    nan_rows = np.all(kv == synth.BF16_NAN, axis=1)
    assert np.array_equal(nan_rows, ~used)
    assert inp["sink"] is None


def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 0.0, np.float32(3.0e38)], np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even (1 + 2^-6) wins.
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2.0**-6
    assert back[3] == -2.5 and back[4] == 0.0
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
