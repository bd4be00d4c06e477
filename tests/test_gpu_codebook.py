"""Parity of the codebook-V path (attn_decode_cb) and of the Walsh-Hadamard
undo (attn_fwht_undo) with the CPU fp64 oracle, through the C ABI.

Bar: max-abs <= 2e-3 and relative-L2 <= 1e-3 over each output (fp32 GPU output
vs the fp64 oracle), as for the other V formats, plus batched == per-slot
bitwise and the rejections of bad arguments.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_codebook_inputs
from oracle import oracle_attn_decode_cb, oracle_fwht_undo

from gpu_util import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _report(name, err):
    print(f"[codebook] {name}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)


def _dev(ci):
    d = torch.device("cuda:0")
    return (ci.q.to(d), ci.k.to(d), ci.v_codes.to(d), ci.v_norms.to(d), ci.codebook.to(d))


def _run_gpu(ci, window, chunk=0, merge_mode=0, dev=None):
    q, k, vc, vn, cb = dev if dev is not None else _dev(ci)
    out = torch.full((ci.n_slots, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32, device=q.device)
    binding.attn_decode_cb(q, k, vc, vn, cb, ci.codebook_bits, ci.seq_lens, window, out, ci.n_slots,
                           ci.n_q_heads, ci.n_kv_heads, ci.head_dim, ci.scale, chunk=chunk,
                           merge_mode=merge_mode)
    torch.cuda.synchronize()
    return out


def _run_oracle(ci, window, rows=None):
    return oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                 ci.codebook.numpy(), ci.codebook_bits, ci.seq_lens, window, ci.n_q_heads,
                                 ci.n_kv_heads, ci.head_dim, ci.scale, rows=rows)


CASES = [
    # seq_lens, n_q, n_kv, D, bits, window
    ((256,), 1, 1, 64, 8, 0),
    ((4096,), 16, 8, 256, 8, 0),
    ((1024, 0, 3000, 77), 16, 8, 256, 5, 0),
    ((1000, 2500), 8, 2, 128, 6, 0),
    ((700, 1, 2049), 8, 2, 512, 8, 0),
    ((3000, 129), 16, 4, 512, 6, 300),
    ((5000,), 16, 8, 256, 8, 1024),
    ((63, 65, 1), 4, 1, 64, 5, 0),
    ((6000, 2049), 16, 2, 512, 8, 0),      # G = 8: the global-layer shape
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_codebook_matches_oracle(case):
    seq, n_q, n_kv, D, bits, W = case
    ci = make_codebook_inputs(seq, n_q, n_kv, D, bits, 500 + D + bits)
    got = _run_gpu(ci, W).cpu().numpy()
    ref = _run_oracle(ci, W)
    _report(f"{seq} D={D} bits={bits} W={W}", assert_parity(got, ref, str(case)))


@pytest.mark.parametrize("merge_mode", [0, 2])
@pytest.mark.parametrize("chunk", [1, 16, 200])
def test_codebook_chunking_changes_only_rounding(chunk, merge_mode):
    ci = make_codebook_inputs((900, 2, 333), 8, 2, 256, 8, 77)
    got = _run_gpu(ci, 0, chunk=chunk, merge_mode=merge_mode).cpu().numpy()
    assert_parity(got, _run_oracle(ci, 0), f"chunk={chunk}")


def test_codebook_batched_equals_per_slot_bitwise():
    seq = (2000, 5, 0, 700)
    ci = make_codebook_inputs(seq, 16, 8, 256, 8, 91)
    q, k, vc, vn, cb = _dev(ci)
    full = _run_gpu(ci, 0, dev=(q, k, vc, vn, cb))
    off = 0
    for s, L in enumerate(seq):
        n = L * ci.n_kv_heads * ci.head_dim
        one = torch.full((1, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32, device=q.device)
        binding.attn_decode_cb(q[s:s + 1].contiguous(), k[off:off + n], vc[off:off + n],
                               vn[off // 256:(off + n) // 256], cb, 8, [L], 0, one, 1, ci.n_q_heads,
                               ci.n_kv_heads, ci.head_dim, ci.scale)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[s]), f"slot {s}"
        off += n


def test_codebook_full_size_full_output():
    """8 slots x 32768 positions, 16 / 8 heads, D 256, the pages' 8-bit codebook: the hybrid
    workload shape with the pages' own V format, every output row against the oracle."""
    seq = (32768,) * 8
    ci = make_codebook_inputs(seq, 16, 8, 256, 8, 3000, direct=True)
    got = _run_gpu(ci, 0).cpu().numpy()
    ref = _run_oracle(ci, 0)
    assert ref.shape == got.shape
    _report("8x32768 D=256 bits=8 (all 128 rows)", assert_parity(got, ref, "full size"))


# ------------------------------------------------------------------ undo

@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("in_place", [False, True])
def test_undo_matches_oracle(D, in_place):
    r = np.random.default_rng(D)
    x = r.standard_normal((37, D)).astype(np.float32)
    s = np.where(r.random(D) < 0.5, -1.0, 1.0).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    sd = torch.from_numpy(s).cuda()
    y = xd if in_place else torch.full_like(xd, float("nan"))
    binding.attn_fwht_undo(xd, sd, y)
    torch.cuda.synchronize()
    ref = oracle_fwht_undo(x.astype(np.float64), s)
    got = y.cpu().numpy()
    # fp32 butterflies: log2(D) roundings of values of the row's norm (~sqrt(D))
    assert np.abs(got - ref).max() <= 1e-5 * math.sqrt(D)


def test_encode_attend_undo_chain_matches_oracle_chain():
    seq = (1500, 40)
    ci = make_codebook_inputs(seq, 16, 8, 256, 8, 4321)
    out = _run_gpu(ci, 0)
    binding.attn_fwht_undo(out, ci.signs.cuda(), out)
    torch.cuda.synchronize()
    ref = oracle_fwht_undo(_run_oracle(ci, 0), ci.signs.numpy())
    _report("attend + undo", assert_parity(out.cpu().numpy(), ref, "chain"))


def test_undo_of_nothing_is_a_no_op():
    x = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    binding.attn_fwht_undo(x, torch.ones(256, device="cuda"), x)


# ------------------------------------------------------------------ rejections

def test_codebook_rejects_bad_arguments():
    ci = make_codebook_inputs((10,), 2, 1, 64, 5, 1)
    q, k, vc, vn, cb = _dev(ci)
    out = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    lib = binding.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    seq_arr = np.array([10], dtype=np.int32)
    seq = seq_arr.ctypes.data

    def call(bits=5, codebook=cb.data_ptr(), norms=vn.data_ptr()):
        return lib.attn_decode_cb(q.data_ptr(), k.data_ptr(), vc.data_ptr(), norms, codebook, bits, seq, 0,
                                  out.data_ptr(), 1, 2, 1, 64, 0.125, stream, None)

    assert call() == 0
    torch.cuda.synchronize()
    assert call(bits=0) == binding.ATTN_DECODE_EINVAL
    assert call(bits=9) == binding.ATTN_DECODE_EINVAL
    assert call(codebook=None) == binding.ATTN_DECODE_EINVAL
    assert call(norms=None) == binding.ATTN_DECODE_EINVAL
    assert call(norms=vn.data_ptr() + 2) == binding.ATTN_DECODE_EINVAL
    assert call(codebook=out.data_ptr()) == binding.ATTN_DECODE_EINVAL   # out overlaps the codebook
    signs = torch.ones(64, dtype=torch.float32, device="cuda")
    assert lib.attn_fwht_undo(out.data_ptr(), signs.data_ptr(), out.data_ptr(), 1, 96, stream) == \
        binding.ATTN_DECODE_EINVAL
    assert lib.attn_fwht_undo(out.data_ptr(), signs.data_ptr(), out.data_ptr() + 16, 1, 64, stream) == \
        binding.ATTN_DECODE_EINVAL
    assert lib.attn_fwht_undo(out.data_ptr(), out.data_ptr(), out.data_ptr(), 1, 64, stream) == \
        binding.ATTN_DECODE_EINVAL   # y overlaps signs
    del seq_arr
