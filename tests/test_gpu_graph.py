"""HIP-graph capture of the forward, through the C ABI.

A serving loop captures the forward once and replays it. Every path a
capture can take is a plain kernel launch on the given stream: the single
pass (16-row H <= 16 kernel, persistent 128-head kernel) and, for
decode-sized calls, the split path of the entry point that allocates nothing
(its partials in the library's static array, no memory set: every partial a
call reads is written by the same call). Each graph is replayed several times
with the program's own eager work and synchronisations in between (outputs
poisoned, eager calls of the same entry point on other buffers), and every
replay must give the eager result bit for bit."""

import numpy as np
import pytest
import torch

from sparse_attention_top_amd import _lib, synth

from gpu_util import DEV, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(case):
    if case == "tp4_single_pass":  # 512 units of H = 16: more than the CUs, single pass
        return "sparse_mla_prefill", synth.make_inputs("tp4", T=512)
    if case == "wide_persistent":  # H = 128, 384 units: the persistent kernel
        return "sparse_mla_prefill", synth.make_inputs("wide", T=384)
    if case == "decode_noalloc_split":  # 16 tokens, 640-entry rows: split, partials in the static array
        return "sparse_mla_prefill_noalloc", synth.make_inputs("decode")
    full = synth.make_inputs("wide", T=512)  # 8 tokens at H = 128, 512-entry rows: split
    d = dict(full)
    d["q"] = np.ascontiguousarray(full["q"][504:512])
    d["topk"] = np.ascontiguousarray(full["topk"][504:512])
    d["T"] = 8
    return "sparse_mla_prefill_noalloc", d


def _launcher(entry, q, kv, tk, sk, scale, out, lse):
    lib = _lib.load()
    fn = getattr(lib, entry)
    T, H = q.shape[:2]

    def call():
        stream = torch.cuda.current_stream(DEV).cuda_stream  # the capture stream while capturing
        rc = fn(q.data_ptr(), kv.data_ptr(), tk.data_ptr(), None if sk is None else sk.data_ptr(), float(scale),
                out.data_ptr(), lse.data_ptr(), T, H, kv.shape[0], tk.shape[1], stream)
        assert rc == _lib.SMLA_OK, _lib.status_string(rc)

    return call


@pytest.mark.parametrize("case", ["tp4_single_pass", "wide_persistent", "decode_noalloc_split",
                                  "wide_tail_noalloc_split"])
def test_graph_replays_match_eager(case):
    entry, inp = _inputs(case)
    q = to_dev_bf16(inp["q"])
    kv = to_dev_bf16(inp["kv"])
    tk = torch.from_numpy(np.ascontiguousarray(inp["topk"], dtype=np.int32)).to(DEV)
    sk = None if inp["sink"] is None else torch.from_numpy(np.ascontiguousarray(inp["sink"])).to(DEV)
    T, H = inp["q"].shape[:2]
    new_o = lambda: torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    new_l = lambda: torch.empty((T, H), dtype=torch.float32, device=DEV)

    # eager reference
    out_e, lse_e = new_o(), new_l()
    _launcher(entry, q, kv, tk, sk, inp["scale"], out_e, lse_e)()
    torch.cuda.synchronize()
    o_ref, l_ref = bf16_bits(out_e), lse_e.cpu().numpy()

    # capture (torch's recipe: one warm-up call on a side stream first)
    out, lse = new_o(), new_l()
    call = _launcher(entry, q, kv, tk, sk, inp["scale"], out, lse)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    out_x, lse_x = new_o(), new_l()
    eager_between = _launcher(entry, q, kv, tk, sk, inp["scale"], out_x, lse_x)
    for r in range(4):
        out.view(torch.int16).fill_(0x7FC0 + r)  # bf16 NaNs: a replay that writes nothing fails
        lse.fill_(float("nan"))
        eager_between()  # the program's own work between replays (same entry point, other buffers)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out), o_ref), "%s: replay %d o differs from the eager call" % (case, r)
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), l_ref.view(np.uint32)), \
            "%s: replay %d lse differs from the eager call" % (case, r)
        assert np.array_equal(bf16_bits(out_x), o_ref), "%s: eager call between replays differs" % case
