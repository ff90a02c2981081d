"""CPU oracle for the sparse MLA prefill forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
(``sparse_attention_top_amd``) and neither imports the other; the seeded input
generator is the only module both sides use.

The arithmetic lives in ``smla_oracle.c`` (forward) and ``smla_oracle_bwd.c``
(backward): plain C, double precision, sequential loops per token and head.
This module only compiles them with gcc and marshals numpy arrays through
ctypes. The definitions they follow, with every reading of the pages they take,
are in the files' header comments.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "smla_oracle.c"), os.path.join(_HERE, "smla_oracle_bwd.c")]
_LIB = os.path.join(_HERE, "libsmla_oracle.so")
D = 512

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O3 (portable x86-64 code: no -march, since the
    library may run on another host; ISO C, so no floating-point contraction), OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-o", tmp, *_SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.smla_oracle_forward.restype = ctypes.c_int
        lib.smla_oracle_forward.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.smla_oracle_forward_ix.restype = ctypes.c_int
        lib.smla_oracle_forward_ix.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.smla_oracle_forward_kv.restype = ctypes.c_int
        lib.smla_oracle_forward_kv.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.smla_oracle_backward.restype = ctypes.c_int
        lib.smla_oracle_backward.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.smla_oracle_threads.restype = ctypes.c_int
        lib.smla_oracle_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward(q, kv, topk, sink, scale, tokens=None, *, want_exact=True, want_bf16=True, threads=0, kv_scale=None):
    """Evaluate the definition for the given tokens (all tokens when None).

    q: uint16 bf16 bits [T, H, 512]; kv: uint16 bf16 bits [num_kv, 512], or
    uint8 OCP FP8 E4M3 codes [num_kv, 512] with ``kv_scale`` (K == V == code * kv_scale);
    topk: int32 or int64 [T, topk]; sink: float32 [H] or None; scale: float.
    Returns a dict with ``o`` (float64 [n, H, 512], unrounded), ``o_bf16``
    (uint16 bits [n, H, 512]), ``lse`` (float64 [n, H], natural log) and
    ``n_valid`` (int64 [n]).
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv_fp8 = kv_scale is not None
    kv = np.ascontiguousarray(kv, dtype=np.uint8 if kv_fp8 else np.uint16)
    topk = np.asarray(topk)
    topk = np.ascontiguousarray(topk, dtype=np.int64 if topk.dtype == np.int64 else np.int32)
    T, H, d = q.shape
    if d != D or kv.ndim != 2 or (kv.shape[0] > 0 and kv.shape[1] != D):
        raise ValueError("head dim must be 512")
    if topk.ndim != 2 or topk.shape[0] != T:
        raise ValueError("topk must be [T, topk]")
    num_kv = kv.shape[0]
    if sink is not None:
        sink = np.ascontiguousarray(sink, dtype=np.float32)
        if sink.shape != (H,):
            raise ValueError("sink must be [H]")
    if tokens is None:
        tok = None
        n = T
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tok.size
    o = np.empty((n, H, D), np.float64) if want_exact else None
    ob = np.empty((n, H, D), np.uint16) if want_bf16 else None
    lse = np.empty((n, H), np.float64)
    nv = np.empty((n,), np.int64)
    rc = _load().smla_oracle_forward_kv(
        _ptr(q), _ptr(kv) if num_kv > 0 else None, int(kv_fp8), float(kv_scale) if kv_fp8 else 1.0,
        _ptr(topk), topk.itemsize, _ptr(sink), float(scale),
        T, H, num_kv, topk.shape[1], _ptr(tok), n, _ptr(o), _ptr(ob), _ptr(lse), _ptr(nv), int(threads))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments (rc=%d)" % rc)
    return {"o": o, "o_bf16": ob, "lse": lse, "n_valid": nv}


def _bf16_to_f64(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def backward(q, kv, dout, o, lse, topk, sink, scale, tokens=None, rows=None, *, want_dq=True, want_dkv=True,
             want_mag=False, threads=0, kv_scale=None):
    """Gradients of the forward, written out from its definition.

    q, dout: uint16 bf16 bits [T, H, 512]; kv: uint16 bf16 bits [num_kv, 512], or
    uint8 OCP FP8 E4M3 codes [num_kv, 512] with ``kv_scale`` (kv == code * kv_scale);
    o: the forward's output, uint16 bf16 bits or float64 [T, H, 512]; lse: float32
    or float64 [T, H] (sink-inclusive, natural log); topk: int32 [T, topk];
    sink: float32 [H] or None; scale: float. ``tokens`` selects the tokens whose
    dq is evaluated (all when None); ``rows`` the pool rows whose dkv is (all
    when None). Returns a dict with ``dq`` (float64 [n_tokens, H, 512]),
    ``dkv`` (float64 [n_rows, 512]) and ``d_sink`` (float64 [H], or None without
    a sink); with ``want_mag``, also ``dq_mag``, ``dkv_mag`` and ``d_sink_mag``:
    per element, the sum of the absolute values of the terms added into it.
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    dout = np.ascontiguousarray(dout, dtype=np.uint16)
    kv_fp8 = kv_scale is not None
    kv = np.ascontiguousarray(kv, dtype=np.uint8 if kv_fp8 else np.uint16)
    o = np.asarray(o)
    o = _bf16_to_f64(o) if o.dtype == np.uint16 else np.ascontiguousarray(o, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    T, H, d = q.shape
    num_kv = kv.shape[0]
    if d != D or dout.shape != q.shape or o.shape != q.shape or lse.shape != (T, H):
        raise ValueError("shapes")
    if topk.ndim != 2 or topk.shape[0] != T:
        raise ValueError("topk must be [T, topk]")
    if sink is not None:
        sink = np.ascontiguousarray(sink, dtype=np.float32)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n_tok = T if tok is None else tok.size
    rws = np.arange(num_kv, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    dq = np.empty((n_tok, H, D), np.float64) if want_dq else None
    dkv = np.empty((rws.size, D), np.float64) if want_dkv else None
    ds = np.empty((H,), np.float64)
    dqm = np.empty_like(dq) if (want_mag and dq is not None) else None
    dkvm = np.empty_like(dkv) if (want_mag and dkv is not None) else None
    dsm = np.empty((H,), np.float64) if want_mag else None
    rc = _load().smla_oracle_backward(
        _ptr(q), _ptr(kv) if num_kv > 0 else None, int(kv_fp8), float(kv_scale) if kv_fp8 else 1.0, _ptr(dout),
        _ptr(o), _ptr(lse), _ptr(topk), _ptr(sink),
        float(scale), T, H, num_kv, topk.shape[1], _ptr(tok), n_tok, _ptr(dq), _ptr(rws), rws.size, _ptr(dkv),
        _ptr(ds), _ptr(dqm), _ptr(dkvm), _ptr(dsm), int(threads))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments (rc=%d)" % rc)
    out = {"dq": dq, "dkv": dkv, "d_sink": ds if sink is not None else None}
    if want_mag:
        out.update(dq_mag=dqm, dkv_mag=dkvm, d_sink_mag=dsm if sink is not None else None)
    return out


def threads() -> int:
    return int(_load().smla_oracle_threads())
