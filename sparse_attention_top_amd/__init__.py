"""Sparse MLA prefill forward and backward (DeepSeek-V4) for MI355X / gfx950.

``sparse_mla_prefill`` and ``sparse_mla_backward`` marshal torch tensors to the C ABI of
``libsparse_mla.so`` (declared in ``include/sparse_mla.h``); every step of the
computation runs in the HIP kernels. torch provides device memory and the
current stream only.
"""

from __future__ import annotations

import math

from . import _lib

HEAD_DIM = 512
DEFAULT_SCALE = 1.0 / math.sqrt(HEAD_DIM)

__all__ = ["sparse_mla_prefill", "sparse_mla_backward", "kernel_name", "set_fp8_pool_decode", "fp8_pool_decoded",
           "HEAD_DIM", "DEFAULT_SCALE"]


def _check(cond: bool, msg: str):
    if not cond:
        raise RuntimeError(msg)


def sparse_mla_prefill(q, kv, topk_indices, attn_sink=None, scale=None, out=None, lse=None, kv_scale=None):
    """Sparse MLA prefill forward; returns ``(out, lse)``.

    q: bf16 [T, H, 512]; kv: bf16 [num_kv, 512] (K == V); topk_indices: int32
    or int64 [T, topk] (any value outside [0, num_kv) is an invalid slot; int64
    values are compared without narrowing); attn_sink:
    fp32 [H] or None; scale: float (default 1/sqrt(512)); kv may instead be a
    float8_e4m3fn [num_kv, 512] pool with its dequant scale ``kv_scale`` (K == V ==
    code * kv_scale; int32 rows only); out: optional bf16
    [T, H, 512] buffer; lse: optional fp32 [T, H] buffer. All tensors on the
    same GPU and contiguous. The work is enqueued on the current stream.
    """
    import torch

    _check(q.is_cuda, "q must be a GPU tensor (got %s)" % q.device)
    dev = q.device
    _check(q.dtype == torch.bfloat16, "q must be bfloat16, got %s" % q.dtype)
    _check(q.dim() == 3 and q.shape[2] == HEAD_DIM, "q must be [T, H, 512], got %s" % (tuple(q.shape),))
    _check(q.is_contiguous(), "q must be contiguous")
    T, H, _ = q.shape
    _check(kv.device == dev, "kv must be on %s, got %s" % (dev, kv.device))
    fp8 = kv.dtype == torch.float8_e4m3fn
    _check(kv.dtype == q.dtype or fp8,
           "kv dtype mismatch: kv is %s, q is %s (or float8_e4m3fn with kv_scale)" % (kv.dtype, q.dtype))
    _check(fp8 == (kv_scale is not None), "kv_scale goes with a float8_e4m3fn pool, and only with one")
    _check(kv.dim() == 2 and kv.shape[1] == HEAD_DIM, "kv must be [num_kv, 512], got %s" % (tuple(kv.shape),))
    _check(kv.is_contiguous(), "kv must be contiguous")
    _check(topk_indices.device == dev, "topk_indices must be on %s" % dev)
    _check(topk_indices.dtype in (torch.int32, torch.int64),
           "topk_indices must be int32 or int64, got %s" % topk_indices.dtype)
    _check(topk_indices.dim() == 2 and topk_indices.shape[0] == T, "topk_indices must be [T, topk]")
    _check(topk_indices.is_contiguous(), "topk_indices must be contiguous")
    if attn_sink is not None:
        _check(attn_sink.device == dev, "attn_sink must be on %s, got %s" % (dev, attn_sink.device))
        _check(attn_sink.dtype == torch.float32, "attn_sink must be float32, got %s" % attn_sink.dtype)
        _check(tuple(attn_sink.shape) == (H,), "attn_sink must be [H]")
        _check(attn_sink.is_contiguous(), "attn_sink must be contiguous")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out.device == dev and out.dtype == q.dtype and out.shape == q.shape,
               "out must match q's shape, dtype and device")
        _check(out.is_contiguous(), "out must be contiguous")
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    else:
        _check(lse.device == dev and lse.dtype == torch.float32 and tuple(lse.shape) == (T, H),
               "lse must be float32 [T, H] on q's device")
        _check(lse.is_contiguous(), "lse must be contiguous")
    if scale is None:
        scale = DEFAULT_SCALE
    lib = _lib.load()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        kvp = kv.data_ptr() if kv.numel() else None
        tkp = topk_indices.data_ptr() if topk_indices.numel() else None
        skp = attn_sink.data_ptr() if attn_sink is not None else None
        if fp8:
            _check(topk_indices.dtype == torch.int32, "a float8_e4m3fn pool takes int32 topk_indices")
            rc = lib.sparse_mla_prefill_fp8(q.data_ptr(), kvp, float(kv_scale), tkp, skp, float(scale),
                                            out.data_ptr(), lse.data_ptr(), T, H, kv.shape[0], topk_indices.shape[1],
                                            stream)
        else:
            entry = lib.sparse_mla_prefill if topk_indices.dtype == torch.int32 else lib.sparse_mla_prefill_i64
            rc = entry(q.data_ptr(), kvp, tkp, skp, float(scale), out.data_ptr(), lse.data_ptr(), T, H, kv.shape[0],
                       topk_indices.shape[1], stream)
    if rc != 0:
        raise RuntimeError("sparse_mla_prefill failed: %s (status %d)" % (_lib.status_string(rc), rc))
    return out, lse


def sparse_mla_backward(q, kv, dout, o, lse, topk_indices, attn_sink=None, scale=None, chunk_tokens=None,
                        kv_scale=None):
    """Gradients of ``sparse_mla_prefill``; returns ``(dq, dkv, d_sink)``.

    q, dout, o: bf16 [T, H, 512] (o and lse are the forward's outputs, lse
    sink-inclusive fp32 [T, H]); kv: bf16 [num_kv, 512], or float8_e4m3fn codes
    with ``kv_scale`` (K == V == code * kv_scale; int32 rows); topk_indices: int32
    or int64 [T, topk]; attn_sink: fp32 [H] or None (then d_sink is None); scale: float
    (default 1/sqrt(512)). H <= 128. dq and dkv come back bf16, d_sink fp32.
    chunk_tokens: tokens per pass (None: passes chosen so that one pass's
    scratch stays under 4 GiB). All tensors on the same GPU and contiguous;
    enqueued on the current stream.
    """
    import torch

    _check(q.is_cuda, "q must be a GPU tensor (got %s)" % q.device)
    dev = q.device
    _check(q.dtype == torch.bfloat16, "q must be bfloat16, got %s" % q.dtype)
    _check(q.dim() == 3 and q.shape[2] == HEAD_DIM, "q must be [T, H, 512], got %s" % (tuple(q.shape),))
    T, H, _ = q.shape
    for name, x in (("dout", dout), ("o", o)):
        _check(x.device == dev and x.dtype == torch.bfloat16 and x.shape == q.shape,
               "%s must be bfloat16 %s on %s" % (name, tuple(q.shape), dev))
    fp8 = kv.dtype == torch.float8_e4m3fn
    _check(kv.device == dev and (kv.dtype == torch.bfloat16 or fp8), "kv must be bfloat16 or float8_e4m3fn on %s" % dev)
    _check(fp8 == (kv_scale is not None), "kv_scale goes with a float8_e4m3fn pool (and only with one)")
    _check(kv.dim() == 2 and kv.shape[1] == HEAD_DIM, "kv must be [num_kv, 512], got %s" % (tuple(kv.shape),))
    _check(lse.device == dev and lse.dtype == torch.float32 and tuple(lse.shape) == (T, H),
           "lse must be float32 [T, H] on q's device")
    _check(topk_indices.device == dev and topk_indices.dtype in (torch.int32, torch.int64),
           "topk_indices must be int32 or int64 on %s" % dev)
    _check(topk_indices.dim() == 2 and topk_indices.shape[0] == T, "topk_indices must be [T, topk]")
    if attn_sink is not None:
        _check(attn_sink.device == dev and attn_sink.dtype == torch.float32 and tuple(attn_sink.shape) == (H,),
               "attn_sink must be float32 [H] on q's device")
    for name, x in (("q", q), ("kv", kv), ("dout", dout), ("o", o), ("lse", lse), ("topk_indices", topk_indices)):
        _check(x.is_contiguous(), "%s must be contiguous" % name)
    if attn_sink is not None:
        _check(attn_sink.is_contiguous(), "attn_sink must be contiguous")
    if scale is None:
        scale = DEFAULT_SCALE
    _check(chunk_tokens is None or int(chunk_tokens) >= 1, "chunk_tokens must be >= 1 (or None)")
    dq = torch.empty_like(q)
    dkv = torch.empty(kv.shape, dtype=torch.bfloat16, device=dev)
    d_sink = torch.empty((H,), dtype=torch.float32, device=dev) if attn_sink is not None else None
    lib = _lib.load()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        kvp = kv.data_ptr() if kv.numel() else None
        rest = (dout.data_ptr(), o.data_ptr(), lse.data_ptr(), topk_indices.data_ptr() if topk_indices.numel() else None,
                attn_sink.data_ptr() if attn_sink is not None else None, float(scale),
                dq.data_ptr(), dkv.data_ptr() if dkv.numel() else None,
                d_sink.data_ptr() if d_sink is not None else None, T, H, kv.shape[0], topk_indices.shape[1],
                int(chunk_tokens or 0), stream)
        if fp8:
            _check(topk_indices.dtype == torch.int32, "an fp8 pool takes int32 top-k rows in the backward")
            rc = lib.sparse_mla_backward_fp8(q.data_ptr(), kvp, float(kv_scale), *rest)
        elif topk_indices.dtype == torch.int64:
            rc = lib.sparse_mla_backward_i64(q.data_ptr(), kvp, *rest)
        else:
            rc = lib.sparse_mla_backward_chunked(q.data_ptr(), kvp, *rest)
    if rc != 0:
        raise RuntimeError("sparse_mla_backward failed: %s (status %d)" % (_lib.status_string(rc), rc))
    return dq, dkv, d_sink


def kernel_name(H: int, topk: int, kv_fp8: bool = False) -> str:
    """Name of the kernel launched for H heads and top-k rows of `topk` entries
    over a bf16 pool, or an fp8 one with kv_fp8 (as profilers show it)."""
    name = _lib.load().sparse_mla_kernel_name(int(H), int(topk), int(bool(kv_fp8)))
    if name is None:
        raise ValueError("need H >= 1 and topk >= 0")
    return name.decode()


_FP8_MODES = {"never": _lib.FP8_POOL_DECODE_NEVER, "auto": _lib.FP8_POOL_DECODE_AUTO,
              "always": _lib.FP8_POOL_DECODE_ALWAYS}


def set_fp8_pool_decode(mode: str) -> str:
    """How an fp8 pool is read, process-wide: "never" (the fp8 kernels gather
    codes), "auto" (the default: decode the pool once per call into a bf16
    copy and run the bf16 kernels when the call gathers many times the pool's
    rows) or "always". Returns the previous mode."""
    _check(mode in _FP8_MODES, "mode must be one of %s" % sorted(_FP8_MODES))
    prev = _lib.load().sparse_mla_set_fp8_pool_decode(_FP8_MODES[mode])
    return {v: k for k, v in _FP8_MODES.items()}[prev]


def fp8_pool_decoded(T: int, topk: int, num_kv: int) -> bool:
    """Whether an fp8 call of these sizes decodes its pool under the current mode."""
    return bool(_lib.load().sparse_mla_fp8_pool_decoded(int(T), int(topk), int(num_kv)))
