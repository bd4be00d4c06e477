"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) replay to the eager result.

A decode loop that captures its step replays the library's launches with the
kernel arguments (slot table included) frozen at capture.  The library
enqueues kernels only (no memset, no allocation once the stream's workspace is
large enough), so a warm-up call before the capture is all a caller needs.
Every replay is checked bitwise against the eager output, with unrelated eager
work and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_codebook_inputs, make_inputs


pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", [((256,), 1, 1, 64, False, 0), ((4096, 1000), 16, 8, 256, True, 0),
                                  ((20000,), 16, 8, 256, False, 1024)], ids=["tiny", "split", "window"])
def test_graph_replay_matches_eager(case):
    seq, nq, nkv, d, i8, W = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=8800)
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    vs = None if inp.v_scales is None else inp.v_scales.to(dev)
    side = torch.cuda.Stream()
    out = torch.full((inp.n_slots, nq, d), float("nan"), dtype=torch.float32, device=dev)
    seq_a = np.asarray(seq, dtype=np.int32)

    def call():
        binding.attn_decode_ex(q, k, v, vs, seq_a, W, out, inp.n_slots, nq, nkv, d, inp.scale, stream=side)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                      # eager, also sizes the stream's workspace
    torch.cuda.synchronize()
    eager = out.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=dev)
    for i in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001)        # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"


def test_graph_of_codebook_attend_and_undo():
    ci = make_codebook_inputs((3000, 64), 16, 8, 256, 8, 8900)
    dev = torch.device("cuda:0")
    q, k, vc, vn, cb, sg = (t.to(dev) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook, ci.signs))
    side = torch.cuda.Stream()
    out = torch.empty((ci.n_slots, 16, 256), dtype=torch.float32, device=dev)
    seq_a = np.asarray(ci.seq_lens, dtype=np.int32)

    def call():
        binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq_a, 0, out, ci.n_slots, 16, 8, 256, ci.scale, stream=side)
        binding.attn_fwht_undo(out, sg, out, stream=side)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
