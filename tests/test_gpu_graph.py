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


# 300 short int8 slots at head_dim 256: a launch group of 256 rows (the large query table, 18.5 KB
# of arguments frozen in the graph node) and one of 44 (the small table), both on the single-buffer
# lane kernel
_MANY = tuple(int(x) for x in np.random.default_rng(8850).integers(129, 2049, size=300))


@pytest.mark.parametrize("merge_mode", [1, 2])
@pytest.mark.parametrize("case", [((256,), 1, 1, 64, False, 0), ((4096, 1000), 16, 8, 256, True, 0),
                                  ((20000,), 16, 8, 256, False, 1024), (_MANY, 16, 8, 256, True, 0)],
                         ids=["tiny", "split", "window", "many_slots"])
def test_graph_replay_matches_eager(case, merge_mode):
    """Both merge modes; the single-launch merge's flagged pairs must be back at zero after
    every replay, or the next replay would merge before its chunks are written."""
    seq, nq, nkv, d, i8, W = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=8800)
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    vs = None if inp.v_scales is None else inp.v_scales.to(dev)
    side = torch.cuda.Stream()
    out = torch.full((inp.n_slots, nq, d), float("nan"), dtype=torch.float32, device=dev)
    seq_a = np.asarray(seq, dtype=np.int32)

    def call():
        binding.attn_decode_ex(q, k, v, vs, seq_a, W, out, inp.n_slots, nq, nkv, d, inp.scale, stream=side,
                               merge_mode=merge_mode)

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


def test_graph_of_codebook_serving_step():
    """The hybrid decode step on a ring cache -- append (K fp16, V codebook-encoded), attend,
    undo -- captured once and replayed; each replay rewrites the same cache rows and must give
    the eager output and cache bit for bit."""
    from decode_attention_kv_02_amd.workloads import make_cache_codebook_inputs
    sid, pos = (0, 1, 2), (3000, 1023, 77)
    ci = make_cache_codebook_inputs(3, 1024, 1, sid, pos, 16, 2, 256, 8, 9000)
    dev = torch.device("cuda:0")
    q, k, vc, vn, cb, sg = (t.to(dev) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook, ci.signs))
    g = torch.Generator("cpu").manual_seed(9001)
    kn = torch.randn((3, 2, 256), generator=g).to(dev)
    vnew = torch.randn((3, 2, 256), generator=g).to(dev)
    out = torch.empty((3, 16, 256), dtype=torch.float32, device=dev)
    k0, vc0, vn0 = k.clone(), vc.clone(), vn.clone()
    side = torch.cuda.Stream()

    def call():
        binding.attn_kv_append_cb(kn, vnew, k, vc, vn, sg, cb, 8, sid, pos, 3, 3, 1024, 1, 2, 256, stream=side)
        binding.attn_decode_cache_cb(q, k, vc, vn, cb, 8, sid, pos, 3, 3, 1024, 1, 0, out, 16, 2, 256, ci.scale,
                                     stream=side)
        binding.attn_fwht_undo(out, sg, out, stream=side)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.synchronize()
    eager = (out.clone(), k.clone(), vc.clone(), vn.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        k.copy_(k0)
        vc.copy_(vc0)
        vn.copy_(vn0)             # the appended rows must be written again by the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((out, k, vc, vn), eager, ("out", "k", "codes", "norms")):
            assert torch.equal(got, want), f"replay {i}: {name}"


def test_graph_replays_after_the_workspace_grows():
    """A graph captured while the stream's workspace was small keeps working after a larger eager
    call on the same stream has grown the workspace: the outgrown buffer, whose address the graph
    holds, stays allocated (it is freed only by attn_decode_release)."""
    dev = torch.device("cuda:0")
    small = make_inputs((3000, 700), 16, 8, 256, True, seed_base=8900)
    big = make_inputs((30000, 20000, 9000), 16, 8, 256, False, seed_base=8901)
    side = torch.cuda.Stream()

    def tensors(inp):
        return (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                None if inp.v_scales is None else inp.v_scales.to(dev))

    ts, tb = tensors(small), tensors(big)
    out_s = torch.full((small.n_slots, 16, 256), float("nan"), dtype=torch.float32, device=dev)
    out_b = torch.full((big.n_slots, 16, 256), float("nan"), dtype=torch.float32, device=dev)
    seq_s = np.asarray(small.seq_lens, dtype=np.int32)
    seq_b = np.asarray(big.seq_lens, dtype=np.int32)

    def call_small():
        binding.attn_decode_ex(*ts, seq_s, 0, out_s, small.n_slots, 16, 8, 256, small.scale, stream=side)

    def call_big():
        binding.attn_decode_ex(*tb, seq_b, 0, out_b, big.n_slots, 16, 8, 256, big.scale, stream=side)

    ws_s = binding.attn_decode_plan(small.seq_lens, 0, 16, 8, 256, v_int8=True)["workspace_bytes"]
    ws_b = binding.attn_decode_plan(big.seq_lens, 0, 16, 8, 256, v_int8=False)["workspace_bytes"]
    assert ws_b > 2 * ws_s, (ws_s, ws_b)   # the big call must outgrow what the small one allocated

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call_small()                # eager: sizes the stream's workspace for the small call only
    torch.cuda.synchronize()
    eager_s = out_s.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call_small()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        call_big()                  # grows the workspace: a new buffer, the old one retired
    torch.cuda.synchronize()
    eager_b = out_b.clone()
    for i in range(4):
        out_s.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_s, eager_s), f"replay {i}"
        with torch.cuda.stream(side):
            call_big()              # eager work on the grown workspace between replays
        torch.cuda.synchronize()
        assert torch.equal(out_b, eager_b), f"eager call after replay {i}"
