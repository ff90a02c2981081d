"""Helpers shared by the GPU tests: moving generator output to the device,
calling the HIP path, and comparing against the oracle at the stated
tolerances (o: |d| <= 2e-2 + 2e-2 |ref|; lse: |d| <= 1e-3, -inf exactly)."""

import numpy as np
import torch

import oracle
from sparse_attention_top_amd import sparse_mla_prefill, synth

O_ATOL = 2e-2
O_RTOL = 2e-2
LSE_ATOL = 1e-3
DEV = torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(q, kv, topk, sink, scale, out=None, lse=None, kv_scale=None):
    """numpy inputs (bf16 bits, int32 or int64 rows, fp32) -> (o bits uint16, lse float32), via the C ABI."""
    qd = to_dev_bf16(q)
    if kv_scale is not None:  # OCP FP8 E4M3 codes
        kvd = torch.from_numpy(np.ascontiguousarray(kv, dtype=np.uint8)).to(DEV).view(torch.float8_e4m3fn)
    else:
        kvd = to_dev_bf16(kv) if kv.shape[0] else torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    topk = np.asarray(topk)
    td = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int64 if topk.dtype == np.int64 else np.int32)).to(DEV)
    sd = None if sink is None else torch.from_numpy(np.ascontiguousarray(sink, dtype=np.float32)).to(DEV)
    o, l = sparse_mla_prefill(qd, kvd, td, sd, scale, out=out, lse=lse, kv_scale=kv_scale)
    torch.cuda.synchronize()
    return bf16_bits(o), l.cpu().numpy()


def run_case(inp):
    return run_gpu(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], kv_scale=inp.get("kv_scale"))


def compare(o_bits, lse, ref, tokens=None, what=""):
    """Elementwise check against the oracle; returns error statistics."""
    if tokens is not None:
        o_bits = o_bits[tokens]
        lse = lse[tokens]
    o = synth.bf16_bits_to_f32(o_bits).astype(np.float64)
    ro, rl = ref["o"], ref["lse"]
    assert o.shape == ro.shape, (o.shape, ro.shape)
    nan_ref = np.isnan(ro)
    assert np.array_equal(np.isnan(o), nan_ref), "%s: NaN pattern differs" % what
    fin = ~nan_ref
    err = np.abs(o[fin] - ro[fin])
    bound = O_ATOL + O_RTOL * np.abs(ro[fin])
    bad = err > bound
    assert not bad.any(), "%s: %d of %d o elements out of tolerance (max err %.3g)" % (
        what, int(bad.sum()), err.size, float(err.max()))
    ninf = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), ninf), "%s: -inf pattern of lse differs" % what
    lnan = np.isnan(rl)
    assert np.array_equal(np.isnan(lse), lnan), "%s: NaN pattern of lse differs" % what
    ok = ~ninf & ~lnan
    lerr = np.abs(lse[ok].astype(np.float64) - rl[ok])
    assert lerr.size == 0 or lerr.max() <= LSE_ATOL, "%s: lse max err %.3g" % (what, float(lerr.max()))
    rel_l2 = float(np.linalg.norm(o[fin] - ro[fin]) / max(np.linalg.norm(ro[fin]), 1e-30))
    return {"o_max_abs": float(err.max()) if err.size else 0.0, "lse_max_abs": float(lerr.max()) if lerr.size else 0.0,
            "o_rel_l2": rel_l2}


def oracle_ref(inp, tokens=None):
    return oracle.forward(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], tokens=tokens,
                          kv_scale=inp.get("kv_scale"))
