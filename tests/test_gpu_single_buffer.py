"""The single-buffer lane kernel (attn_partial_single_kernel) against the oracle and the buffered form.

The planner sends a lane-kernel launch with one-byte V at head_dim 256 to the single-buffer form
when every chunk is at most one iteration of the four waves (64 positions) and the launch has at
least 1024 workgroups; a lone short slot stays on the buffered form.  So a large batch of short
slots runs the single-buffer form while each of its slots alone runs the buffered one, and the
batched rows must equal the per-slot rows bit for bit (the two forms do the same arithmetic),
besides matching the fp64 oracle over the whole output.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_codebook_inputs, make_inputs

from gpu_util import assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

ONE_PASS = 64       # positions of one iteration: one-byte V, head_dim 256
MIN_ITEMS = 1024    # workgroups from which the planner takes the single-buffer form


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _report(name, err):
    print(f"[single] {name}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)


def _takes_single(seq, window, nq, nkv, d):
    p = binding.attn_decode_plan(seq, window, nq, nkv, d, v_int8=True)
    return p["partial_workgroups"] >= MIN_ITEMS and max(p["chunk"]) <= ONE_PASS


def _slot(inp, s):
    d, nkv = inp.head_dim, inp.n_kv_heads
    off = sum(inp.seq_lens[:s]) * nkv * d
    n = inp.seq_lens[s] * nkv * d
    vs = inp.v_scales[off // 32:(off + n) // 32].clone()
    return type(inp)(inp.q[s:s + 1].clone(), inp.k[off:off + n].clone(), inp.v[off:off + n].clone(),
                     vs, (inp.seq_lens[s],), inp.n_q_heads, nkv, d, inp.scale)


SHAPES = [
    # seq_lens, n_q, n_kv, window
    ((2048,) * 16, 16, 8, 0),
    ((2048, 1000, 64, 1, 0, 1500, 2048, 700) * 2, 16, 8, 0),
    ((2048, 1000, 64, 1, 0, 1500, 2048, 700) * 4, 16, 8, 500),
    ((1024,) * 24, 8, 8, 0),      # one head per kv head
]


@pytest.mark.parametrize("merge_mode", [0, 2])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{i}" for i in range(len(SHAPES))])
def test_int8_batch_of_short_slots(shape, merge_mode):
    seq, nq, nkv, W = shape
    print(f"[single] int8 {len(seq)} slots, {nq}/{nkv} heads, window {W}, merge_mode {merge_mode}", flush=True)
    assert _takes_single(seq, W, nq, nkv, 256), "the shape must take the single-buffer form"
    inp = make_inputs(seq, nq, nkv, 256, True, seed_base=9700 + SHAPES.index(shape))
    batched = run_gpu(inp, W, merge_mode=merge_mode)
    _report(f"{len(seq)} slots W={W} mm={merge_mode}",
            assert_parity(batched.cpu().numpy(), run_oracle(inp, W), str(shape)))
    for s in range(len(seq)):
        alone = _slot(inp, s)
        assert not _takes_single(alone.seq_lens, W, nq, nkv, 256)
        solo = run_gpu(alone, W, merge_mode=merge_mode)
        assert torch.equal(batched[s:s + 1], solo), (shape, s)


def test_codebook_batch_of_short_slots():
    seq = (1024,) * 8
    assert _takes_single(seq, 0, 16, 8, 256)
    ci = make_codebook_inputs(seq, 16, 8, 256, 8, 9750)
    d = torch.device("cuda:0")
    q, k, vc, vn, cb = ci.q.to(d), ci.k.to(d), ci.v_codes.to(d), ci.v_norms.to(d), ci.codebook.to(d)
    full = torch.full((8, 16, 256), float("nan"), dtype=torch.float32, device=d)
    binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq, 0, full, 8, 16, 8, 256, ci.scale)
    torch.cuda.synchronize()
    from oracle import oracle_attn_decode_cb
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), 8, seq, 0, 16, 8, 256, ci.scale)
    _report("codebook 8 x 1024", assert_parity(full.cpu().numpy(), ref, "codebook 8 x 1024"))
    n = 1024 * 8 * 256
    for s in range(8):
        one = torch.full((1, 16, 256), float("nan"), dtype=torch.float32, device=d)
        binding.attn_decode_cb(q[s:s + 1].contiguous(), k[s * n:(s + 1) * n], vc[s * n:(s + 1) * n],
                               vn[s * n // 256:(s + 1) * n // 256], cb, 8, [1024], 0, one, 1, 16, 8, 256, ci.scale)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[s]), s


def test_noalloc_takes_the_same_form():
    """attn_decode_noalloc on a batch that takes the single-buffer form equals attn_decode_ex."""
    seq = (2048,) * 16
    inp = make_inputs(seq, 16, 8, 256, True, seed_base=9760)
    dev = to_device(inp)
    a = run_gpu(inp, 0, dev_tensors=dev)
    q, k, v, vs = dev
    b = torch.full_like(a, float("nan"))
    binding.attn_decode_noalloc(q, k, v, vs, np.asarray(seq, dtype=np.int32), 0, b, len(seq), 16, 8, 256, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_ring_cache_queries_take_the_same_form():
    """80 queries over 40 ring slots of 2048 rows, positions past the wrap: one large-table launch
    on the single-buffer form, against the oracle and against each slot's queries alone."""
    from decode_attention_kv_02_amd.workloads import make_cache_inputs
    from gpu_util import run_gpu_cache, run_oracle_cache
    rng = np.random.default_rng(9770)
    sid = tuple(s for s in range(40) for _ in range(2))
    pos = tuple(int(x) for x in rng.integers(2048, 9000, size=80))
    p = binding.attn_decode_cache_plan(sid, pos, 40, 2048, 1, 0, 16, 8, 256, "int8")
    assert p["partial_workgroups"] >= MIN_ITEMS and max(p["chunk"]) <= ONE_PASS
    ci = make_cache_inputs(40, 2048, 1, sid, pos, 16, 8, 256, True, seed_base=9770)
    dev = to_device(ci)
    got = run_gpu_cache(ci, 0, dev_tensors=dev)
    _report("ring 80 queries", assert_parity(got.cpu().numpy(), run_oracle_cache(ci, 0), "ring 80 queries"))
    q, k, v, vs = dev
    for s in (0, 17, 39):
        rows = [2 * s, 2 * s + 1]
        out = torch.full((2, 16, 256), float("nan"), dtype=torch.float32, device=q.device)
        binding.attn_decode_cache(q[rows].contiguous(), k, v, vs, (s, s), (pos[2 * s], pos[2 * s + 1]), 2, 40,
                                  2048, 1, 0, out, 16, 8, 256, ci.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, got[rows]), s
