"""The entry point that allocates nothing (sparse_mla_prefill_noalloc), through
the C ABI: on the same inputs it must give what sparse_mla_prefill gives (the
same split decision, so the same bits) and match the oracle at the forward's
tolerances, on two calls in a row with the second one smaller (the array keeps
the first call's partials), and it must refuse a call whose partials exceed
its array before enqueueing anything."""

import numpy as np
import pytest
import torch

from sparse_attention_top_amd import _lib, synth

from gpu_util import DEV, bf16_bits, compare, oracle_ref, to_dev_bf16

pytestmark = pytest.mark.gpu


def _call(entry, inp, fill=None):
    lib = _lib.load()
    q = to_dev_bf16(inp["q"])
    kv = to_dev_bf16(inp["kv"])
    tk = torch.from_numpy(np.ascontiguousarray(inp["topk"], dtype=np.int32)).to(DEV)
    sk = None if inp["sink"] is None else torch.from_numpy(np.ascontiguousarray(inp["sink"])).to(DEV)
    T, H = inp["q"].shape[:2]
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    if fill is not None:
        out.view(torch.int16).fill_(fill)
        lse.fill_(float(fill))
    stream = torch.cuda.current_stream(DEV).cuda_stream
    rc = getattr(lib, entry)(q.data_ptr(), kv.data_ptr(), tk.data_ptr(), None if sk is None else sk.data_ptr(),
                             float(inp["scale"]), out.data_ptr(), lse.data_ptr(), T, H, kv.shape[0],
                             tk.shape[1], stream)
    torch.cuda.synchronize()
    return rc, bf16_bits(out), lse.cpu().numpy()


def _sub(inp, tokens, cols):
    """A smaller call on the same pool: some of the tokens, the first `cols` top-k entries."""
    d = dict(inp)
    d["q"] = np.ascontiguousarray(inp["q"][tokens])
    d["topk"] = np.ascontiguousarray(inp["topk"][tokens, :cols])
    d["T"], d["topk_n"] = len(tokens), cols
    return d


def _same_and_close(inp, what):
    rc0, o0, l0 = _call("sparse_mla_prefill", inp)
    rc1, o1, l1 = _call("sparse_mla_prefill_noalloc", inp, fill=0x7FC0)  # outputs poisoned first (bf16 NaN)
    assert rc0 == _lib.SMLA_OK and rc1 == _lib.SMLA_OK, (rc0, rc1)
    assert np.array_equal(o0, o1), "%s: o differs from sparse_mla_prefill" % what
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), "%s: lse differs from sparse_mla_prefill" % what
    print(what, compare(o1, l1, oracle_ref(inp), what=what))


def _wide_tail():
    full = synth.make_inputs("wide", T=512)
    return _sub(full, np.arange(504, 512), 512)


@pytest.mark.parametrize("case", ["decode_h16", "tail_h128"])
def test_noalloc_split_path_two_calls(case):
    """Few-token calls split each top-k row; the partials live in the static array.
    First a call, then a smaller one (fewer tokens and shorter rows)."""
    if case == "decode_h16":
        inp = synth.make_inputs("decode")                     # T=16, H=16, topk=640
        small = _sub(inp, np.arange(3, 9), 400)
    else:
        inp = _wide_tail()                                    # T=8, H=128, topk=512
        small = _sub(inp, np.array([1, 4, 6]), 256)
    _same_and_close(inp, case + " first")
    _same_and_close(small, case + " second (smaller)")


def test_noalloc_single_pass_uses_no_scratch():
    """A call that does not split (short rows) runs the single-pass kernel."""
    inp = synth.make_inputs("tiny")
    _same_and_close(inp, "tiny")
    _same_and_close(_sub(inp, np.arange(10, 30), 24), "tiny second (smaller)")


def test_noalloc_rejects_partials_beyond_its_array():
    """100 tokens at H = 128 with 512-entry rows: 200 head-group units, 3 splits,
    64 heads of 2056 bytes each -> 79 MB > 64 MiB: refused, outputs untouched."""
    full = synth.make_inputs("wide", T=512)
    inp = _sub(full, np.arange(400, 500), 512)
    rc, o, l = _call("sparse_mla_prefill_noalloc", inp, fill=0x1234)
    assert rc == _lib.SMLA_ERR_SCRATCH_LIMIT, rc
    assert np.all(o == 0x1234) and np.all(l == float(0x1234))
    assert "no-allocation" in _lib.status_string(rc)
    # the allocating entry point takes the same call
    rc0, o0, l0 = _call("sparse_mla_prefill", inp)
    assert rc0 == _lib.SMLA_OK
    compare(o0, l0, oracle_ref(inp), what="wide 100-token split")
