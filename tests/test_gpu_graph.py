"""HIP-graph capture of the forward and the backward.

A serving or training loop captures the call once and replays it. Every forward path a
capture can take is a plain kernel launch on the given stream: the single
pass (16-row H <= 16 kernel, persistent 128-head kernel) and, for
decode-sized calls, the split path of the entry point that allocates nothing
(its partials in the library's static array, no memory set: every partial a
call reads is written by the same call). The backward takes stream-ordered
scratch (allocation nodes in the graph) and sets no memory. Each graph is
replayed several times with the program's own eager work and synchronisations
in between (outputs poisoned, eager calls of the same entry point), and every
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


@pytest.mark.parametrize("case,chunk", [("wide", None), ("tp4", 100)])
def test_backward_graph_replays_match_eager(case, chunk):
    """The backward captured into a HIP graph: its scratch is stream-ordered (allocation nodes in the graph) and
    its sort sets no memory, so each replay, with poisoned outputs and an eager backward in between, gives the
    eager gradients bit for bit; tp4 in passes of 100 tokens (the fp32 dkv accumulator path)."""
    from sparse_attention_top_amd import sparse_mla_backward, sparse_mla_prefill

    inp = synth.make_inputs(case, T=256 if case == "wide" else 300)
    q = to_dev_bf16(inp["q"])
    kv = to_dev_bf16(inp["kv"])
    tk = torch.from_numpy(np.ascontiguousarray(inp["topk"], dtype=np.int32)).to(DEV)
    sk = torch.from_numpy(np.ascontiguousarray(inp["sink"])).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    dout = torch.randn(q.shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    o, lse = sparse_mla_prefill(q, kv, tk, sk, inp["scale"])
    ref = [x.clone() for x in sparse_mla_backward(q, kv, dout, o, lse, tk, sk, inp["scale"], chunk_tokens=chunk)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sparse_mla_backward(q, kv, dout, o, lse, tk, sk, inp["scale"], chunk_tokens=chunk)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = sparse_mla_backward(q, kv, dout, o, lse, tk, sk, inp["scale"], chunk_tokens=chunk)
    torch.cuda.synchronize()
    for r in range(3):
        for x in outs:
            x.fill_(float("nan"))
        eager = sparse_mla_backward(q, kv, dout, o, lse, tk, sk, inp["scale"], chunk_tokens=chunk)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b, e in zip(("dq", "dkv", "d_sink"), outs, ref, eager):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                "%s replay %d: %s differs from the eager call" % (case, r, name)
            assert torch.equal(e, b), "%s: eager call between replays differs (%s)" % (case, name)
