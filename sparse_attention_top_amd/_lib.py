"""ctypes loader for libsparse_mla.so (the C ABI in include/sparse_mla.h).

There is no fallback: if the library is missing the import of the op fails
loudly with the build command to run.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_mla.so")

# Every function include/sparse_mla.h declares, with its ctypes signature.
SIGNATURES = {
    "sparse_mla_prefill": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, topk, sink
        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,  # scale, out, lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_prefill_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, topk, sink
        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,  # scale, out, lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_prefill_fp8": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, kv_scale, topk, sink
        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,  # scale, out, lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_prefill_i64": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, topk (int64), sink
        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,  # scale, out, lse
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_backward": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, dout, o, lse
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,  # topk, sink, scale
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # dq, dkv, d_sink
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_backward_chunked": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, dout, o, lse
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,  # topk, sink, scale
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # dq, dkv, d_sink
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_int64,  # chunk_tokens
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_backward_i64": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # q, kv, dout, o, lse
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,  # topk (int64), sink, scale
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # dq, dkv, d_sink
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_int64,  # chunk_tokens
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_backward_fp8": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,  # q, kv (fp8 codes), kv_scale
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # dout, o, lse
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,  # topk, sink, scale
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # dq, dkv, d_sink
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,  # T, H, num_kv, topk
        ctypes.c_int64,  # chunk_tokens
        ctypes.c_void_p,  # stream
    ]),
    "sparse_mla_set_fp8_pool_decode": (ctypes.c_int, [ctypes.c_int]),
    "sparse_mla_fp8_pool_decoded": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "sparse_mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sparse_mla_kernel_name": (ctypes.c_char_p, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "sparse_mla_version": (ctypes.c_int, []),
}

SMLA_OK = 0
SMLA_ERR_NULL_POINTER = -1
SMLA_ERR_BAD_SIZE = -2
SMLA_ERR_MISALIGNED = -3
SMLA_ERR_BAD_SCALE = -4
SMLA_ERR_NO_DEVICE = -5
SMLA_ERR_LAUNCH = -6
SMLA_ERR_NO_MEMORY = -7
SMLA_ERR_SCRATCH_LIMIT = -8

FP8_POOL_DECODE_NEVER = 0
FP8_POOL_DECODE_AUTO = 1
FP8_POOL_DECODE_ALWAYS = 2

_lib = None


def load():
    """Load (once) and return the ctypes handle; raises if the library is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libsparse_mla.so is not built (expected at %s); run "
                "`python -m sparse_attention_top_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(rc: int) -> str:
    return load().sparse_mla_status_string(int(rc)).decode()
