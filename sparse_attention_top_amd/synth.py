"""Seeded synthetic inputs for sparse MLA prefill (forward).

This module only *draws inputs*: it holds none of the attention arithmetic.
Both the HIP path and the CPU oracle consume what it returns, so it must stay
free of anything either side computes.

Structure of the top-k rows (after the DeepSeek-V4 sparse MLA backward page,
"Performance" section: a sliding window plus a causally visible compressed
pool, not uniform random; and its note that a V4 top-k always keeps the token
itself):

* KV pool layout ``[num_kv, 512]``: rows ``0..T-1`` belong to the tokens, rows
  ``T + j`` (``j < T // c``) are compressed-pool rows, each covering ``c``
  tokens. Pool row ``T + j`` is causally visible to token ``t`` iff
  ``c * (j + 1) <= t + 1``.
* Row ``t`` of ``topk``: slots ``0..W-1`` hold the window tokens
  ``t-W+1 .. t`` ascending (``-1`` where negative, so the window includes
  ``t``); slots ``W..W+P-1`` hold the visible pool rows -- all of them when at
  most ``P`` are visible, else a seeded ``rng.choice`` of ``P`` -- sorted and
  offset by ``T``; the remaining slots are ``-1``.
* Optional random drops (probability ``drop_p``) of valid slots other than the
  token's own slot, and optional NaN filling of every KV row that no valid slot
  references.

A second layout, ``paged``, stands in for a serving engine's KV pool (the
GLM-shaped test on the forward review page: 16 heads, top-k 2048, a pool over
2 GiB): the sequence's ``T`` rows live in pages of ``page`` rows placed at
random page slots of a pool of ``pool_rows`` rows; the other rows are zero.
Row ``t`` of ``topk`` holds the window ``t-W+1 .. t`` then up to ``P``
distinct earlier positions ``< t-W+1`` (all when at most ``P``, else a seeded
``rng.choice``), sorted, each mapped through the page table; the rest ``-1``.

``q``, ``kv`` are N(0,1) fp32 rounded to bf16 (round to nearest, ties to even)
and returned as their raw ``uint16`` bit patterns; ``attn_sink`` is N(0,1)
fp32. With ``kv_fp8`` the same kv draw is stored as OCP FP8 E4M3 codes
(``uint8``) of ``x / kv_scale``, ``kv_scale = max|x| / 448`` (round to nearest
even, by torch's float8_e4m3fn conversion), and ``kv_scale`` is returned.
The draw order is fixed: q, kv (the sequence's rows, for ``paged``),
sink, then (``paged``) the page placement, then per-token choices in token
order, then the drop mask.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np

D = 512
DEFAULT_SCALE = 1.0 / math.sqrt(D)
BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    topk: int
    window: int
    pool_slots: int
    compression: int
    seed: int
    sink: bool = True
    drop_p: float = 0.0
    nan_unused: bool = False
    layout: str = "pool"  # "pool" (window + compressed pool) or "paged"
    tail: int = 0         # keep only the last `tail` tokens' q and top-k rows (decode-sized calls)
    kv_fp8: bool = False  # pool as OCP FP8 E4M3 codes with one dequant scale
    pool_rows: int = 0    # paged: rows in the whole pool
    page: int = 64        # paged: rows per page

    @property
    def num_kv(self) -> int:
        if self.layout == "paged":
            return self.pool_rows
        return self.T + self.T // self.compression


# The five workloads: shapes from the forward pages (TP4 shard, H=16, 640
# slots), the backward page's benchmark shapes (H=128), a tiny case and a
# small-head case with drops and NaN-filled unused rows.
CONFIGS = {
    "tiny": Config("tiny", T=64, H=16, topk=32, window=16, pool_slots=16, compression=4, seed=101),
    "small": Config("small", T=2048, H=8, topk=128, window=64, pool_slots=64, compression=4, seed=102,
                    sink=False, drop_p=1.0 / 16.0, nan_unused=True),
    "tp4": Config("tp4", T=16384, H=16, topk=640, window=128, pool_slots=512, compression=4, seed=103),
    "wide": Config("wide", T=4096, H=128, topk=512, window=128, pool_slots=384, compression=4, seed=104),
    "large": Config("large", T=8192, H=128, topk=1024, window=256, pool_slots=768, compression=8, seed=105),
    # the backward page's other two benchmark shapes (T=4096 / topk=1024 / Kv=5120 and T=8192 / topk=512 / Kv=9216)
    "wide_k1024": Config("wide_k1024", T=4096, H=128, topk=1024, window=128, pool_slots=896, compression=4, seed=107),
    "long": Config("long", T=8192, H=128, topk=512, window=128, pool_slots=384, compression=8, seed=108),
    # GLM-shaped prefill on a server-sized paged pool (2.2 M rows = 2.1 GiB)
    "glm": Config("glm", T=16384, H=16, topk=2048, window=128, pool_slots=1920, compression=1, seed=106,
                  sink=False, layout="paged", pool_rows=2_200_000, page=64),
    # a decode-sized call: the last 16 tokens of the tp4 sequence (same pool and rows)
    "decode": Config("decode", T=16384, H=16, topk=640, window=128, pool_slots=512, compression=4, seed=103,
                     tail=16),
}
# the same draws with the pool stored as fp8 codes
for _name in ("tiny", "tp4", "wide", "glm"):
    CONFIGS[_name + "_fp8"] = dataclasses.replace(CONFIGS[_name], name=_name + "_fp8", kv_fp8=True)


def to_fp8_codes(x: np.ndarray):
    """fp32 values -> (OCP FP8 E4M3 codes of x / s, s) with s = max|x| / 448."""
    import torch

    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    codes = torch.from_numpy(np.ascontiguousarray(x / s, dtype=np.float32)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy(), float(s)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def build_topk(rng: np.random.Generator, T: int, topk: int, window: int, pool_slots: int,
               compression: int) -> np.ndarray:
    """Sliding-window + causally-visible-pool top-k rows, ``int32 [T, topk]``."""
    if window + pool_slots > topk:
        raise ValueError("window + pool_slots must fit in topk")
    idx = np.full((T, topk), -1, dtype=np.int32)
    t = np.arange(T, dtype=np.int64)[:, None]
    w = t - (window - 1) + np.arange(window, dtype=np.int64)[None, :]
    idx[:, :window] = np.where(w >= 0, w, -1).astype(np.int32)
    for tok in range(T):
        vis = (tok + 1) // compression
        if vis <= pool_slots:
            rows = np.arange(vis, dtype=np.int64)
        else:
            rows = np.sort(rng.choice(vis, pool_slots, replace=False))
        idx[tok, window:window + rows.size] = (rows + T).astype(np.int32)
    return idx


def build_topk_paged(rng: np.random.Generator, T: int, topk: int, window: int, pool_slots: int,
                     row_of: np.ndarray) -> np.ndarray:
    """Window + earlier-position top-k rows over sequence positions, mapped to pool rows."""
    if window + pool_slots > topk:
        raise ValueError("window + pool_slots must fit in topk")
    pos = np.full((T, topk), -1, dtype=np.int64)
    t = np.arange(T, dtype=np.int64)[:, None]
    w = t - (window - 1) + np.arange(window, dtype=np.int64)[None, :]
    pos[:, :window] = np.where(w >= 0, w, -1)
    for tok in range(T):
        vis = tok + 1 - window  # earlier positions 0 .. vis-1
        if vis <= 0:
            continue
        if vis <= pool_slots:
            rows = np.arange(vis, dtype=np.int64)
        else:
            rows = np.sort(rng.choice(vis, pool_slots, replace=False))
        pos[tok, window:window + rows.size] = rows
    return np.where(pos >= 0, row_of[np.maximum(pos, 0)], -1).astype(np.int32)


def make_inputs(cfg: Config | str, *, T: int | None = None) -> dict:
    """Draw one seeded workload.

    ``T`` optionally truncates the sequence (same draw recipe at a smaller
    size, used for parity cases the oracle finishes in seconds).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if T is not None and T != cfg.T:
        cfg = dataclasses.replace(cfg, T=T)
    rng = np.random.default_rng(cfg.seed)
    T_, H = cfg.T, cfg.H
    num_kv = cfg.num_kv
    q = f32_to_bf16_bits(rng.standard_normal((T_, H, D), dtype=np.float32))
    kv_scale = None
    if cfg.layout == "paged":
        seqf = rng.standard_normal((T_, D), dtype=np.float32)
        if cfg.kv_fp8:
            seq, kv_scale = to_fp8_codes(seqf)
        else:
            seq = f32_to_bf16_bits(seqf)
        sink = rng.standard_normal(H, dtype=np.float32) if cfg.sink else None
        n_pages = -(-T_ // cfg.page)
        if n_pages * cfg.page > num_kv:
            raise ValueError("pool too small for the sequence")
        slots = rng.permutation(num_kv // cfg.page)[:n_pages].astype(np.int64)
        p_ = np.arange(T_, dtype=np.int64)
        row_of = slots[p_ // cfg.page] * cfg.page + p_ % cfg.page
        kv = np.zeros((num_kv, D), dtype=np.uint8 if cfg.kv_fp8 else np.uint16)  # untouched pages stay unallocated
        kv[row_of] = seq
        topk = build_topk_paged(rng, T_, cfg.topk, cfg.window, cfg.pool_slots, row_of)
    else:
        kvf = rng.standard_normal((num_kv, D), dtype=np.float32)
        if cfg.kv_fp8:
            kv, kv_scale = to_fp8_codes(kvf)
        else:
            kv = f32_to_bf16_bits(kvf)
        sink = rng.standard_normal(H, dtype=np.float32) if cfg.sink else None
        topk = build_topk(rng, T_, cfg.topk, cfg.window, cfg.pool_slots, cfg.compression)
    if cfg.drop_p > 0.0:
        drop = rng.random((T_, cfg.topk)) < cfg.drop_p
        drop[:, cfg.window - 1] = False  # the token's own slot is always kept
        topk[drop & (topk >= 0)] = -1
    if cfg.tail:
        q = np.ascontiguousarray(q[-cfg.tail:])
        topk = np.ascontiguousarray(topk[-cfg.tail:])
        T_ = cfg.tail
    n_unused = 0
    if cfg.nan_unused:
        used = np.zeros(num_kv, dtype=bool)
        valid = topk[(topk >= 0) & (topk < num_kv)]
        used[valid] = True
        n_unused = int((~used).sum())
        kv[~used] = 0x7F if cfg.kv_fp8 else BF16_NAN
    return {
        "config": cfg,
        "q": q,
        "kv": kv,
        "topk": topk,
        "sink": sink,
        "scale": DEFAULT_SCALE,
        "T": T_,
        "H": H,
        "num_kv": num_kv,
        "topk_n": cfg.topk,
        "n_unused_nan_rows": n_unused,
        "kv_scale": kv_scale,
    }


def valid_slot_count(topk: np.ndarray, num_kv: int) -> int:
    """Number of slots whose index lies in ``[0, num_kv)`` (the work units)."""
    return int(((topk >= 0) & (topk < num_kv)).sum())


def fingerprint(inp: dict) -> str:
    """SHA-256 over the generated tensors (recorded with every result)."""
    h = hashlib.sha256()
    for key in ("q", "kv", "topk"):
        h.update(np.ascontiguousarray(inp[key]).tobytes())
    if inp["sink"] is not None:
        h.update(np.ascontiguousarray(inp["sink"]).tobytes())
    return h.hexdigest()
