"""Parity of the matrix-core partial kernel (groups of 8 or more query heads per
kv head, head_dim >= 128) with the CPU fp64 oracle, through the C ABI.

Same bar as the lane kernel: max-abs <= 2e-3 and relative-L2 <= 1e-3 over each
output tensor, batched == per-slot bitwise, and the lane kernel (forced with
path=1) within the same bar on the same inputs.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_cache_inputs, make_codebook_inputs, make_inputs
from oracle import oracle_attn_decode_cb

from gpu_util import assert_parity, run_gpu_cache, run_oracle, run_oracle_cache, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _report(name, err):
    print(f"[mfma] {name}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)


def _run(inp, W, path=0, chunk=0, merge_mode=0, dev=None):
    q, k, v, vs = dev if dev is not None else to_device(inp)
    out = torch.full((inp.n_slots, inp.n_q_heads, inp.head_dim), float("nan"), dtype=torch.float32,
                     device=q.device)
    binding.attn_decode_ex(q, k, v, vs, inp.seq_lens, W, out, inp.n_slots, inp.n_q_heads, inp.n_kv_heads,
                           inp.head_dim, inp.scale, chunk=chunk, merge_mode=merge_mode, path=path)
    torch.cuda.synchronize()
    return out


CASES = [
    # seq_lens, n_q, n_kv, D, int8 V, window
    ((4096,), 16, 2, 512, False, 0),          # gemma4 global layer: 8 heads per kv head, D 512
    ((3000, 0, 17, 1025), 16, 2, 512, True, 0),
    ((2000, 700), 64, 8, 128, False, 0),      # 8 heads per kv head at D 128
    ((1500,), 32, 2, 128, True, 100),         # 16 heads per kv head, windowed
    ((999, 5000), 32, 1, 256, False, 0),      # 32 heads: two blocks of 16
    ((777, 64, 1), 48, 2, 256, True, 0),      # 24 heads: three blocks of 8
    ((16, 15, 1, 33), 16, 1, 256, False, 0),  # tails shorter than a 16-key tile
    ((20000,), 16, 2, 256, True, 1024),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_matrix_core_path_matches_oracle(case):
    seq, nq, nkv, d, i8, W = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=7100 + 13 * CASES.index(case))
    dev = to_device(inp)
    ref = run_oracle(inp, W)
    got = _run(inp, W, path=2, dev=dev).cpu().numpy()
    _report(f"{case} matrix", assert_parity(got, ref, f"{case} matrix"))
    lanes = _run(inp, W, path=1, dev=dev).cpu().numpy()
    _report(f"{case} lanes", assert_parity(lanes, ref, f"{case} lanes"))
    # the automatic choice: the matrix cores wherever they apply (8k heads per kv head, head_dim >= 128)
    auto = _run(inp, W, path=0, dev=dev).cpu().numpy()
    assert np.array_equal(auto, got), "automatic choice"
    for s, L in enumerate(seq):
        if L == 0:
            assert np.all(got[s] == 0.0)


@pytest.mark.parametrize("chunk", [1, 16, 17, 200, 5000])
@pytest.mark.parametrize("merge_mode", [0, 2])
def test_matrix_core_chunking_changes_only_rounding(chunk, merge_mode):
    inp = make_inputs((900, 2, 333), 16, 2, 256, False, seed_base=7300)
    got = _run(inp, 0, path=2, chunk=chunk, merge_mode=merge_mode).cpu().numpy()
    assert_parity(got, run_oracle(inp, 0), f"chunk={chunk}")


def test_matrix_core_batched_equals_per_slot_bitwise():
    seq = (2000, 5, 0, 700, 4097)
    inp = make_inputs(seq, 32, 2, 256, True, seed_base=7400)
    full = _run(inp, 0)
    for s, L in enumerate(seq):
        off = sum(seq[:s]) * 2 * 256
        n = L * 2 * 256
        q = inp.q[s:s + 1].contiguous().cuda()
        k = inp.k[off:off + n].cuda()
        v = inp.v[off:off + n].cuda()
        vs = inp.v_scales[off // 32:(off + n) // 32].cuda()
        out = torch.full((1, 32, 256), float("nan"), dtype=torch.float32, device="cuda")
        binding.attn_decode(q, k, v, vs, [L], 0, out, 1, 32, 2, 256, inp.scale)
        torch.cuda.synchronize()
        assert torch.equal(out[0], full[s]), f"slot {s}"


def test_matrix_core_codebook_v():
    seq = (3000, 2049, 0)
    ci = make_codebook_inputs(seq, 16, 2, 512, 8, 7500)
    d = torch.device("cuda:0")
    q, k, vc, vn, cb = (t.to(d) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook))
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), 8, seq, 0, 16, 2, 512, ci.scale)
    for path in (2, 1):
        out = torch.full((3, 16, 512), float("nan"), dtype=torch.float32, device=d)
        binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq, 0, out, 3, 16, 2, 512, ci.scale, path=path)
        torch.cuda.synchronize()
        _report(f"codebook D=512 G=8 path {path}", assert_parity(out.cpu().numpy(), ref, f"path {path}"))


@pytest.mark.parametrize("ring", [0, 1])
def test_matrix_core_cache_layouts(ring):
    # 4 cache slots of 1536 rows; queries at positions past the capacity wrap on the ring
    pos = (1535, 200, 3000, 0) if ring else (1535, 200, 1000, 0)
    ci = make_cache_inputs(4, 1536, ring, (0, 1, 2, 3), pos, 16, 2, 256, ring == 1, seed_base=7600 + ring)
    got = run_gpu_cache(ci, 0).cpu().numpy()
    _report(f"cache ring={ring}", assert_parity(got, run_oracle_cache(ci, 0), f"ring={ring}"))


def test_matrix_core_path_is_rejected_where_it_does_not_apply():
    inp = make_inputs((100,), 8, 2, 256, False, seed_base=7700)     # 4 heads per kv head
    with pytest.raises(binding.AttnDecodeError) as ei:
        _run(inp, 0, path=2)
    assert ei.value.code == binding.ATTN_DECODE_EINVAL
    inp = make_inputs((100,), 16, 2, 64, False, seed_base=7701)     # head_dim 64
    with pytest.raises(binding.AttnDecodeError):
        _run(inp, 0, path=2)
    ok = _run(inp, 0, path=0).cpu().numpy()                          # the lane kernel there
    assert_parity(ok, run_oracle(inp, 0), "auto at head_dim 64")


@pytest.mark.parametrize("d,nq,nkv,i8", [(128, 16, 2, False), (256, 32, 2, True), (512, 16, 2, False),
                                         (512, 16, 2, True)])
def test_large_and_rising_logits(d, nq, nkv, i8):
    """Logits of several hundred, and for head 0 a ramp rising by about 64 (natural log) over
    each slot, so the running maximum moves at almost every tile: the softmax reference of the
    matrix-core kernel (which moves only past a headroom) and the lanes' exact one must both
    match the oracle."""
    seq = (3000, 1500)
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=7800 + d)
    inp.q.mul_(3.0)
    k = inp.k.numpy()                       # fp16 view, packed [slot][kv][pos][D]
    off = 0
    for s, L in enumerate(seq):
        v = np.sign(inp.q[s, 0].numpy().astype(np.float32))   # q . v = sum |q|
        ramp = (5.0 * np.arange(L) / L).astype(np.float32)[:, None] * v[None, :]
        rows = k[off:off + L * d].reshape(L, d)                  # kv head 0 of slot s
        rows[:] = (rows.astype(np.float32) * 0.5 + ramp).astype(np.float16)
        off += nkv * L * d
    ref = run_oracle(inp, 0)
    dev = to_device(inp)
    for path in (2, 1):
        got = _run(inp, 0, path=path, dev=dev).cpu().numpy()
        _report(f"rising logits D={d} path {path}", assert_parity(got, ref, f"path {path}"))


@pytest.mark.parametrize("d,nq,nkv,bits,W", [(256, 16, 2, 5, 0), (128, 64, 4, 6, 0), (512, 32, 2, 6, 0),
                                              (256, 16, 2, 8, 700), (512, 16, 2, 5, 1500)])
def test_matrix_core_codebook_bits(d, nq, nkv, bits, W):
    seq = (2100, 700, 0)
    ci = make_codebook_inputs(seq, nq, nkv, d, bits, 7900 + d + bits)
    dv = torch.device("cuda:0")
    q, k, vc, vn, cb = (t.to(dv) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook))
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), bits, seq, W, nq, nkv, d, ci.scale)
    out = torch.full((len(seq), nq, d), float("nan"), dtype=torch.float32, device=dv)
    binding.attn_decode_cb(q, k, vc, vn, cb, bits, seq, W, out, len(seq), nq, nkv, d, ci.scale, path=2)
    torch.cuda.synchronize()
    _report(f"codebook {bits}-bit D={d} G={nq // nkv} W={W}", assert_parity(out.cpu().numpy(), ref, "codebook"))


SMALL_G_CASES = [
    # seq_lens, n_q, n_kv, D, V: one query with 4 to 7 heads per kv head goes to the matrix cores
    # by itself (4 columns are enough where that kernel takes fp16 products)
    ((3000, 1, 700), 32, 8, 128, "fp16"),
    ((2500, 40), 24, 4, 256, "int8"),       # 6 heads
    ((1800, 33), 20, 4, 512, "fp16"),       # 5 heads
    ((999,), 28, 4, 256, "fp16"),           # 7 heads
    ((2100, 700), 32, 8, 256, "codebook"),  # 4 heads
]


@pytest.mark.parametrize("case", SMALL_G_CASES, ids=[f"g{i}" for i in range(len(SMALL_G_CASES))])
def test_one_query_with_four_to_seven_heads_on_the_matrix_cores(case):
    seq, nq, nkv, d, fmt = case
    # the matrix-core chunk rule (at least 512 positions) tells the planner's choice from the lanes' (64)
    assert binding.attn_decode_plan(list(seq), 0, nq, nkv, d, v_int8=fmt != "fp16")["chunk"][0] == 512
    dv = torch.device("cuda:0")
    if fmt == "codebook":
        ci = make_codebook_inputs(seq, nq, nkv, d, 8, 8100 + d)
        ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                    ci.codebook.numpy(), 8, seq, 0, nq, nkv, d, ci.scale)
        q, k, vc, vn, cb = (t.to(dv) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook))
        for path in (0, 1):
            out = torch.full((len(seq), nq, d), float("nan"), dtype=torch.float32, device=dv)
            binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq, 0, out, len(seq), nq, nkv, d, ci.scale, path=path)
            torch.cuda.synchronize()
            _report(f"{case} path {path}", assert_parity(out.cpu().numpy(), ref, f"path {path}"))
        return
    inp = make_inputs(seq, nq, nkv, d, fmt == "int8", seed_base=8200 + d + nq)
    ref = run_oracle(inp, 0)
    dev = to_device(inp)
    for path in (0, 1):
        _report(f"{case} path {path}", assert_parity(_run(inp, 0, path=path, dev=dev).cpu().numpy(), ref,
                                                     f"path {path}"))
