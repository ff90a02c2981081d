"""The C-ABI library: it loads, exports every function the header declares, and
rejects bad arguments before touching a device (CPU only: no compute call)."""

import ctypes
import os
import re

import pytest

from sparse_attention_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_mla_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert "sparse_mla_prefill" in names and "sparse_mla_status_string" in names
    assert set(names) == set(_lib.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    exported = os.popen("nm -D --defined-only %s" % _lib.LIB_PATH).read()
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, exported), name


def call(q=0x1000, kv=0x2000, topk=0x3000, sink=None, scale=0.0441, out=0x4000, lse=0x5000,
         T=4, H=8, num_kv=16, k=8):
    return _lib.load().sparse_mla_prefill(q, kv, topk, sink, scale, out, lse, T, H, num_kv, k, None)


def test_status_strings_and_version():
    lib = _lib.load()
    for rc in range(-8, 1):
        assert _lib.status_string(rc)
    assert _lib.status_string(17) == "unknown status"
    assert lib.sparse_mla_version() >= 100


def test_kernel_names():
    lib = _lib.load()
    assert lib.sparse_mla_kernel_name(0, 64, 0) is None
    assert lib.sparse_mla_kernel_name(8, -1, 1) is None
    assert lib.sparse_mla_kernel_name(8, 64, 0) == lib.sparse_mla_kernel_name(16, 64, 0)
    assert lib.sparse_mla_kernel_name(64, 512, 0).startswith(b"smla_fwd_kernel<")
    assert lib.sparse_mla_kernel_name(128, 2048, 0) == b"smla_fwd_kernel<4, 2>"  # two 64-head groups
    assert lib.sparse_mla_kernel_name(128, 1024, 0) == b"smla_fwd128_kernel"  # persistent, 128 heads per unit
    assert lib.sparse_mla_kernel_name(96, 512, 0) == b"smla_fwd128_kernel"
    assert lib.sparse_mla_kernel_name(64, 512, 0) == b"smla_fwd_kernel<4, 2>"
    assert lib.sparse_mla_kernel_name(16, 640, 0).startswith(b"smla_fwd16_kernel<")  # 16-row tiles at H <= 16
    assert lib.sparse_mla_kernel_name(16, 2048, 1).startswith(b"smla_fwd16_fp8_kernel<")
    assert lib.sparse_mla_kernel_name(128, 512, 1).startswith(b"smla_fwd_fp8_kernel<8,")


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), _lib.SMLA_ERR_BAD_SIZE),
    (dict(H=0), _lib.SMLA_ERR_BAD_SIZE),
    (dict(num_kv=-5), _lib.SMLA_ERR_BAD_SIZE),
    (dict(k=-1), _lib.SMLA_ERR_BAD_SIZE),
    (dict(T=2**31), _lib.SMLA_ERR_BAD_SIZE),
    (dict(T=2**30, H=2**12), _lib.SMLA_ERR_BAD_SIZE),
    (dict(scale=float("nan")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(scale=float("inf")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(scale=float("-inf")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(q=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(out=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(lse=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(topk=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(kv=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(q=0x1008), _lib.SMLA_ERR_MISALIGNED),
    (dict(kv=0x2004), _lib.SMLA_ERR_MISALIGNED),
    (dict(out=0x4002), _lib.SMLA_ERR_MISALIGNED),
    (dict(lse=0x5001), _lib.SMLA_ERR_MISALIGNED),
    (dict(topk=0x3002), _lib.SMLA_ERR_MISALIGNED),
    (dict(sink=0x6003), _lib.SMLA_ERR_MISALIGNED),
])
def test_argument_errors_return_before_any_launch(kw, rc):
    assert call(**kw) == rc


def call_noalloc(q=0x1000, kv=0x2000, topk=0x3000, sink=None, scale=0.0441, out=0x4000, lse=0x5000,
                 T=4, H=8, num_kv=16, k=8):
    return _lib.load().sparse_mla_prefill_noalloc(q, kv, topk, sink, scale, out, lse, T, H, num_kv, k, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), _lib.SMLA_ERR_BAD_SIZE),
    (dict(H=0), _lib.SMLA_ERR_BAD_SIZE),
    (dict(scale=float("nan")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(q=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(topk=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(out=0x4002), _lib.SMLA_ERR_MISALIGNED),
])
def test_noalloc_entry_argument_errors(kw, rc):
    assert call_noalloc(**kw) == rc
    assert call_noalloc(T=0, q=None, out=None, lse=None, topk=None, kv=None) == _lib.SMLA_OK


def call64(q=0x1000, kv=0x2000, topk=0x3000, sink=None, scale=0.0441, out=0x4000, lse=0x5000,
           T=4, H=8, num_kv=16, k=8):
    return _lib.load().sparse_mla_prefill_i64(q, kv, topk, sink, scale, out, lse, T, H, num_kv, k, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), _lib.SMLA_ERR_BAD_SIZE),
    (dict(scale=float("nan")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(topk=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(topk=0x3004), _lib.SMLA_ERR_MISALIGNED),  # int64 rows need 8-byte alignment
    (dict(q=0x1008), _lib.SMLA_ERR_MISALIGNED),
])
def test_int64_entry_argument_errors(kw, rc):
    assert call64(**kw) == rc


def call8(q=0x1000, kv=0x2000, kv_scale=0.5, topk=0x3000, sink=None, scale=0.0441, out=0x4000, lse=0x5000,
          T=4, H=8, num_kv=16, k=8):
    return _lib.load().sparse_mla_prefill_fp8(q, kv, kv_scale, topk, sink, scale, out, lse, T, H, num_kv, k, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(kv_scale=float("nan")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(kv_scale=float("inf")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(kv_scale=1e30, scale=1e30), _lib.SMLA_ERR_BAD_SCALE),  # the product overflows
    (dict(kv=0x2008), _lib.SMLA_ERR_MISALIGNED),
    (dict(topk=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(H=0), _lib.SMLA_ERR_BAD_SIZE),
])
def test_fp8_entry_argument_errors(kw, rc):
    assert call8(**kw) == rc


def callbwd(q=0x1000, kv=0x2000, dout=0x3000, o=0x4000, lse=0x5000, topk=0x6000, sink=None, scale=0.0441,
            dq=0x7000, dkv=0x8000, d_sink=None, T=4, H=8, num_kv=16, k=8):
    return _lib.load().sparse_mla_backward(q, kv, dout, o, lse, topk, sink, scale, dq, dkv, d_sink, T, H, num_kv, k,
                                           None)


@pytest.mark.parametrize("kw,rc", [
    (dict(T=-1), _lib.SMLA_ERR_BAD_SIZE),
    (dict(H=0), _lib.SMLA_ERR_BAD_SIZE),
    (dict(H=129), _lib.SMLA_ERR_BAD_SIZE),  # the backward handles up to 128 heads
    (dict(num_kv=2**31), _lib.SMLA_ERR_BAD_SIZE),
    (dict(T=2**26, k=64), _lib.SMLA_ERR_BAD_SIZE),  # T * round_up(topk, 32) >= 2^31
    (dict(scale=float("nan")), _lib.SMLA_ERR_BAD_SCALE),
    (dict(q=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(dout=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(o=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(lse=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(dq=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(dkv=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(topk=None), _lib.SMLA_ERR_NULL_POINTER),
    (dict(sink=0x9000), _lib.SMLA_ERR_NULL_POINTER),  # a sink needs d_sink
    (dict(dq=0x7008), _lib.SMLA_ERR_MISALIGNED),
    (dict(dkv=0x8004), _lib.SMLA_ERR_MISALIGNED),
    (dict(lse=0x5002), _lib.SMLA_ERR_MISALIGNED),
    (dict(sink=0x9000, d_sink=0xA001), _lib.SMLA_ERR_MISALIGNED),
])
def test_backward_argument_errors(kw, rc):
    assert callbwd(**kw) == rc


def test_backward_chunked_argument_errors():
    lib = _lib.load()
    args = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0.0441, 0x7000, 0x8000, None, 4, 8, 16, 8]
    assert lib.sparse_mla_backward_chunked(*args, -1, None) == _lib.SMLA_ERR_BAD_SIZE  # negative pass size
    bad = list(args)
    bad[12] = 129
    assert lib.sparse_mla_backward_chunked(*bad, 2, None) == _lib.SMLA_ERR_BAD_SIZE
    bad = list(args)
    bad[8] = 0x7008
    assert lib.sparse_mla_backward_chunked(*bad, 2, None) == _lib.SMLA_ERR_MISALIGNED


def test_backward_int64_argument_errors():
    """The int64-row backward checks its arguments (int64 rows 8-byte aligned) before any device work."""
    lib = _lib.load()
    args = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0.0441, 0x7000, 0x8000, None, 4, 8, 16, 8, 0, None]
    bad = list(args)
    bad[5] = 0x6004  # 4-byte aligned only
    assert lib.sparse_mla_backward_i64(*bad) == _lib.SMLA_ERR_MISALIGNED
    bad = list(args)
    bad[5] = None
    assert lib.sparse_mla_backward_i64(*bad) == _lib.SMLA_ERR_NULL_POINTER
    bad = list(args)
    bad[12] = 129
    assert lib.sparse_mla_backward_i64(*bad) == _lib.SMLA_ERR_BAD_SIZE
    bad = list(args)
    bad[15] = -1
    assert lib.sparse_mla_backward_i64(*bad) == _lib.SMLA_ERR_BAD_SIZE


def test_fp8_pool_decode_policy():
    """An fp8 call decodes its pool to a bf16 copy (by default) when it gathers at least 8x the pool's rows and
    the copy is at most 256 MiB; the mode switch returns the previous mode and refuses unknown values."""
    from sparse_attention_top_amd import fp8_pool_decoded, set_fp8_pool_decode

    lib = _lib.load()
    assert set_fp8_pool_decode("auto") == "auto"
    assert fp8_pool_decoded(16384, 640, 20480)          # tp4: 10.5 M slots over a 20 MiB pool
    assert fp8_pool_decoded(4096, 512, 5120)            # wide
    assert not fp8_pool_decoded(16, 640, 20480)         # decode-sized call: fewer slots than 8x the pool
    assert not fp8_pool_decoded(16384, 2048, 2200000)   # a 2.1 GiB paged pool: its copy is too large
    assert fp8_pool_decoded(1 << 20, 64, 262144) and not fp8_pool_decoded(1 << 20, 64, 262145)
    assert not fp8_pool_decoded(0, 640, 100) and not fp8_pool_decoded(10, 0, 100) and not fp8_pool_decoded(10, 10, 0)
    assert set_fp8_pool_decode("always") == "auto"
    assert fp8_pool_decoded(16, 640, 20480) and fp8_pool_decoded(16384, 2048, 2200000)
    assert set_fp8_pool_decode("never") == "always"
    assert not fp8_pool_decoded(16384, 640, 20480)
    assert lib.sparse_mla_set_fp8_pool_decode(7) == -1 and lib.sparse_mla_set_fp8_pool_decode(-1) == -1
    assert set_fp8_pool_decode("auto") == "never"
    with pytest.raises(RuntimeError):
        set_fp8_pool_decode("sometimes")


def test_empty_sequence_is_ok_without_a_device():
    assert call(T=0, q=None, out=None, lse=None, topk=None, kv=None) == _lib.SMLA_OK


def test_null_allowed_where_size_is_zero():
    # with topk == 0 neither the index array nor the pool is read; kv may be NULL when num_kv == 0
    rc_k0 = call(topk=None, k=0, kv=None)
    rc_nkv0 = call(kv=None, num_kv=0)
    # both pass validation; without a GPU the next step reports the missing device
    for rc in (rc_k0, rc_nkv0):
        assert rc in (_lib.SMLA_OK, _lib.SMLA_ERR_NO_DEVICE, _lib.SMLA_ERR_LAUNCH)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()
