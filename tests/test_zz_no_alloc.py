"""attn_decode_noalloc: attn_decode_ex with its partials in the library's fixed device scratch.

It must give attn_decode_ex's results bit for bit (same plan, same kernels, same merge), on
calls in a row that reuse the scratch (the second smaller than the first), also when captured
into a HIP graph, and reject a call whose partials do not fit before any GPU work.
"""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_inputs

from gpu_util import assert_parity, run_oracle, to_device

SCRATCH = 16 * 1024 * 1024


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()


def _pair(inp, tens, W, chunk=0):
    """(attn_decode_ex output, attn_decode_noalloc output), each into a NaN-poisoned buffer."""
    shape = (inp.n_slots, inp.n_q_heads, inp.head_dim)
    outs = []
    for fn in (binding.attn_decode_ex, binding.attn_decode_noalloc):
        out = torch.full(shape, float("nan"), dtype=torch.float32, device=tens[0].device)
        fn(*tens, inp.seq_lens, W, out, inp.n_slots, inp.n_q_heads, inp.n_kv_heads, inp.head_dim, inp.scale,
           chunk=chunk)
        torch.cuda.synchronize()
        outs.append(out)
    return outs


@pytest.mark.gpu
def test_noalloc_equals_attn_decode_ex_on_calls_in_a_row():
    _gpu()
    cases = [
        # the ragged four-slot workload: 1792 partial rows, 1.8 MB of scratch
        ((1024, 8192, 32768, 2000), 16, 8, 256, False, 0, 7910),
        # smaller: one 4096-position slot, int8 V, then a window (fewer partials again)
        ((4096,), 16, 8, 256, True, 0, 7911),
        ((5000, 300), 16, 8, 256, False, 1000, 7912),
    ]
    for seq, nq, nkv, d, i8, W, seed in cases:
        inp = make_inputs(seq, nq, nkv, d, i8, seed_base=seed)
        plan = binding.attn_decode_plan(seq, W, nq, nkv, d, v_int8=i8)
        assert 0 < plan["workspace_bytes"] <= SCRATCH
        ref_ex, got = _pair(inp, to_device(inp), W)
        assert torch.equal(got, ref_ex), f"{seq} W={W}"
        err = assert_parity(got.cpu().numpy(), run_oracle(inp, W), f"{seq} W={W}")
        print(f"[noalloc] {seq} W={W}: bitwise equal to attn_decode_ex; max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}",
              flush=True)


@pytest.mark.gpu
def test_noalloc_replays_from_a_captured_graph():
    _gpu()
    inp = make_inputs((3000, 700, 9000), 16, 8, 256, True, seed_base=7920)
    dev = to_device(inp)
    side = torch.cuda.Stream()
    out = torch.full((inp.n_slots, 16, 256), float("nan"), dtype=torch.float32, device=dev[0].device)
    seq = np.asarray(inp.seq_lens, dtype=np.int32)

    def call():
        binding.attn_decode_noalloc(*dev, seq, 0, out, inp.n_slots, 16, 8, 256, inp.scale, stream=side)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    other = make_inputs((20000,), 16, 8, 256, False, seed_base=7921)
    for i in range(3):
        _pair(other, to_device(other), 0)      # another no-allocation call in between overwrites the scratch
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"


def test_noalloc_rejects_what_does_not_fit_before_any_gpu_work():
    lib = binding.load_library()
    # 32 slots of 32768 positions, 16 q / 8 kv heads, head_dim 256: 16.9 MB of partials
    seq = [32768] * 32
    plan = binding.attn_decode_plan(seq, 0, 16, 8, 256)
    assert plan["workspace_bytes"] > SCRATCH
    arr = (ctypes.c_int32 * len(seq))(*seq)
    far = [ctypes.c_void_p(k << 40) for k in (1, 2, 3, 4)]   # aligned, disjoint, never touched
    rc = lib.attn_decode_noalloc(far[0], far[1], far[2], None, arr, 0, far[3], len(seq), 16, 8, 256,
                                 ctypes.c_float(0.0625), None, None)
    assert rc == binding.ATTN_DECODE_EINVAL
    assert "scratch" in binding.last_error()
    # one slot fewer fits
    plan = binding.attn_decode_plan(seq[:30], 0, 16, 8, 256)
    assert plan["workspace_bytes"] <= SCRATCH


def test_noalloc_rejects_the_single_launch_merge():
    lib = binding.load_library()
    seq = (ctypes.c_int32 * 1)(4096)
    opts = binding._Options(0, 2, None, None, 0)
    far = [ctypes.c_void_p(k << 40) for k in (1, 2, 3, 4)]
    rc = lib.attn_decode_noalloc(far[0], far[1], far[2], None, seq, 0, far[3], 1, 16, 8, 256,
                                 ctypes.c_float(0.0625), None, ctypes.byref(opts))
    assert rc == binding.ATTN_DECODE_EINVAL
    assert "merge_mode" in binding.last_error()
