"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle.

Bar: max-abs <= 2e-3 and relative-L2 <= 1e-3 over each output tensor (fp32
GPU output vs the fp64 oracle), plus exact structural contracts: batched ==
per-slot bitwise, run-to-run bitwise determinism, immunity to a recycled
(unzeroed, NaN-poisoned) workspace (the contract behind tessl nn.rs's
unzeroed decode scratch), and exact single-key results.

Inputs are the seeded workloads of ``decode_attention_kv_02_amd.workloads``.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import WORKLOADS, make_inputs, workload_inputs

from gpu_util import assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _report(name, err):
    print(f"[parity] {name}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_workload_full_output(idx):
    cfg = WORKLOADS[idx]
    inp = workload_inputs(cfg)
    for W in cfg.windows:
        got = run_gpu(inp, W).cpu().numpy()
        ref = run_oracle(inp, W)
        _report(f"{cfg.name} W={W}", assert_parity(got, ref, cfg.name))


def test_workload_hybrid_int8_full_output():
    """Config 3 at full size (8 x 32768, int8 V): every one of the 128 output rows against the
    oracle, the acceptance bar over the whole tensor."""
    cfg = WORKLOADS[3]
    inp = workload_inputs(cfg)
    got = run_gpu(inp, 0).cpu().numpy()
    ref = run_oracle(inp, 0)
    assert ref.shape == got.shape == (cfg.n_slots, cfg.n_q_heads, cfg.head_dim)
    _report(cfg.name + " (all 128 rows)", assert_parity(got, ref, cfg.name))


def test_workload_long_context_full_and_window():
    cfg = WORKLOADS[4]
    inp = workload_inputs(cfg)
    dev = to_device(inp)
    for W in cfg.windows:
        got = run_gpu(inp, W, dev_tensors=dev).cpu().numpy()
        ref = run_oracle(inp, W)
        _report(f"{cfg.name} W={W}", assert_parity(got, ref, cfg.name))


# ------------------------------------------------------------------ edge cases

EDGE = [
    # seq_lens, n_q, n_kv, D, v_int8, window
    ((1,), 1, 1, 64, False, 0),
    ((0, 5, 0, 64, 65, 127, 128, 129, 1000), 4, 2, 128, False, 0),
    ((300, 1), 8, 8, 256, True, 0),
    ((777,), 16, 2, 256, False, 0),
    ((513, 2), 6, 2, 512, False, 0),
    ((4000, 10, 2500), 16, 8, 256, True, 100),
    ((2049,), 4, 1, 64, True, 2048),
    ((3000,), 2, 1, 512, True, 1),
    ((1500, 1500), 32, 8, 128, False, 999),
    ((0, 0), 2, 2, 256, False, 0),
    ((63, 64, 65, 4095, 4096, 4097), 16, 8, 256, False, 0),
    ((5000, 3000, 1), 32, 2, 256, True, 0),     # G = 16: four head blocks per chunk
    ((9000, 700), 16, 2, 512, False, 0),        # G = 8 at D = 512
    ((4096, 1000, 513, 512), 8, 8, 64, True, 0),   # 256-position chunks at D = 64, ragged tails
    ((4096, 3001, 257), 16, 8, 128, False, 0),     # 128-position chunks at D = 128
]


@pytest.mark.parametrize("case", EDGE, ids=[f"e{i}" for i in range(len(EDGE))])
def test_edge_cases(case):
    seq, nq, nkv, d, i8, W = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=5000 + 17 * EDGE.index(case))
    got = run_gpu(inp, W).cpu().numpy()
    ref = run_oracle(inp, W)
    _report(f"edge {case}", assert_parity(got, ref, str(case)))
    for s, L in enumerate(seq):
        if L == 0:
            assert np.all(got[s] == 0.0)


@pytest.mark.parametrize("merge_mode", [0, 2])
@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 200, 5000])
@pytest.mark.parametrize("i8", [False, True])
def test_chunking_changes_only_rounding(chunk, i8, merge_mode):
    # chunk 3 splits the slots into 1001 / 234 / 1 chunks: in the in-kernel merge
    # mode the first still goes through the combine kernel, the second does not
    seq = (3001, 700, 1)
    inp = make_inputs(seq, 8, 4, 256, i8, seed_base=7100)
    ref = run_oracle(inp, 0)
    got = run_gpu(inp, 0, chunk=chunk, merge_mode=merge_mode).cpu().numpy()
    _report(f"chunk {chunk} int8={i8} merge={merge_mode}", assert_parity(got, ref, f"chunk={chunk}"))


@pytest.mark.parametrize("D,nq,nkv", [(64, 4, 1), (128, 8, 2), (256, 16, 2), (512, 4, 4), (512, 16, 4)])
def test_in_kernel_merge_every_geometry(D, nq, nkv):
    # every (head_dim, heads per workgroup) layout of the in-kernel merge, at its bound of 64 chunks
    inp = make_inputs((64 * 5, 70), nq, nkv, D, D % 32 == 0 and nq == 16, seed_base=7150 + D + nq)
    ref = run_oracle(inp, 0)
    got = run_gpu(inp, 0, chunk=5, merge_mode=2).cpu().numpy()
    _report(f"merge geometry D={D} G={nq // nkv}", assert_parity(got, ref, f"D={D}"))


SINGLE_LAUNCH = [
    # seq_lens, n_q, n_kv, D, int8 V, window, chunk
    ((4096,), 16, 8, 256, False, 0, 0),                  # config 1's shape
    ((1024, 8192, 32768, 2000), 16, 8, 256, False, 0, 0),  # config 2's shape
    ((131072,), 16, 8, 256, False, 1024, 0),             # config 4's window
    ((9000, 0, 1, 3000), 16, 8, 256, True, 0, 0),
    ((5000, 700), 32, 4, 128, True, 0, 0),              # 8 heads per kv head: two head blocks
    ((3000, 2500), 4, 4, 64, False, 0, 0),
    ((2600, 1300), 8, 2, 512, True, 999, 0),
    ((64 * 5, 70), 16, 8, 256, False, 0, 5),             # 64 chunks: at the single-launch bound
    ((64 * 5 + 3, 70), 16, 8, 256, False, 0, 5),         # 65 chunks: over it (combine kernel)
    ((40 * 5, 1000, 17), 8, 8, 512, True, 0, 5),         # D = 512: two merge workgroups per head
    ((33 * 7, 31 * 7), 4, 2, 64, False, 0, 7),           # D = 64: one slice, 33 and 31 chunks
]


@pytest.mark.parametrize("case", SINGLE_LAUNCH, ids=[f"{c[0]}-D{c[3]}-G{c[1] // c[2]}" for c in SINGLE_LAUNCH])
def test_single_launch_merge_equals_combine_kernel_bitwise(case):
    """The merge workgroups at the end of the partial kernel's grid run the combine kernel's
    arithmetic on the same partials, so both merge modes give the same bits; twice in a row on
    one stream (each call leaves the flagged pairs all zero for the next)."""
    seq, nq, nkv, d, i8, W, chunk = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=7170 + d + nq)
    dev = to_device(inp)
    two = run_gpu(inp, W, chunk=chunk, dev_tensors=dev, merge_mode=1)
    for rep in range(2):
        one = run_gpu(inp, W, chunk=chunk, dev_tensors=dev, merge_mode=2)
        assert torch.equal(one, two), f"repeat {rep}"
    ref = run_oracle(inp, W)
    _report(f"single launch {seq} D={d}", assert_parity(one.cpu().numpy(), ref, "single launch"))


def test_single_key_is_exact():
    for i8 in (False, True):
        inp = make_inputs((1, 1), 4, 2, 256, i8, seed_base=7200)
        got = run_gpu(inp, 0).cpu().numpy()
        ref = run_oracle(inp, 0)
        assert np.array_equal(got.astype(np.float64), ref), f"int8={i8}"


def test_large_logits_stay_stable():
    inp = make_inputs((2500, 333), 16, 8, 256, False, seed_base=7300)
    inp.q.mul_(12.0)   # logits of several hundred: exp must not overflow
    got = run_gpu(inp, 0).cpu().numpy()
    ref = run_oracle(inp, 0)
    _report("large logits", assert_parity(got, ref, "large logits"))


@pytest.mark.parametrize("n_slots", [49, 150, 300])
def test_many_slots(n_slots):
    """Query tables of both capacities: up to 48 rows per launch take the small table, more the
    large one (up to 256); 300 slots are one launch of 256 and one of 44."""
    rng = np.random.default_rng(7400 + n_slots)
    seq = tuple(int(x) for x in rng.integers(0, 400, size=n_slots))
    inp = make_inputs(seq, 4, 2, 128, True, seed_base=7400 + n_slots)
    got = run_gpu(inp, 0).cpu().numpy()
    ref = run_oracle(inp, 0)
    _report(f"{n_slots} slots", assert_parity(got, ref, f"{n_slots} slots"))


@pytest.mark.parametrize("case", [
    ((2048,) * 48, 16, 8, 256, True),          # floor 768: three chunks per slot
    ((1024, 8192, 32768, 2000), 16, 8, 256, False),
    ((300,) * 60, 16, 8, 256, False),
    ((512,) * 64, 32, 4, 128, False),          # matrix cores, eight heads per kv head
    ((16384,) * 8, 16, 2, 512, True),          # matrix cores at head_dim 512: 1024 instead of 512
], ids=["int8_48x2048", "ragged", "60x300", "mfma_64x512", "mfma_d512_8x16384"])
def test_per_call_chunk_floor(case):
    """chunk = CHUNK_PER_CALL: every output against the oracle, and the same call twice bitwise."""
    seq, nq, nkv, d, i8 = case
    inp = make_inputs(seq, nq, nkv, d, i8, seed_base=7470 + len(seq))
    dev = to_device(inp)
    got = run_gpu(inp, 0, chunk=binding.CHUNK_PER_CALL, dev_tensors=dev)
    _report(f"per-call floor {len(seq)} slots", assert_parity(got.cpu().numpy(), run_oracle(inp, 0), str(case)))
    assert torch.equal(got, run_gpu(inp, 0, chunk=binding.CHUNK_PER_CALL, dev_tensors=dev))


def test_many_slots_equal_per_slot_bitwise():
    """A slot's result does not depend on which table or launch carried it: rows of a 300-slot call
    (large table, then small) equal the same slots called alone."""
    rng = np.random.default_rng(7450)
    seq = tuple(int(x) for x in rng.integers(1, 600, size=300))
    inp = make_inputs(seq, 16, 8, 256, False, seed_base=7450)
    batched = run_gpu(inp, 0)
    for s in (0, 1, 47, 48, 200, 255, 256, 299):
        assert torch.equal(batched[s:s + 1], run_gpu(_slot_inputs(inp, s), 0)), s


# ------------------------------------------------------------------ structural contracts

def _slot_inputs(inp, s):
    d, nkv = inp.head_dim, inp.n_kv_heads
    off = sum(inp.seq_lens[:s]) * nkv * d
    n = inp.seq_lens[s] * nkv * d
    vs = None if inp.v_scales is None else inp.v_scales[off // 32:(off + n) // 32].clone()
    return type(inp)(inp.q[s:s + 1].clone(), inp.k[off:off + n].clone(), inp.v[off:off + n].clone(),
                     vs, (inp.seq_lens[s],), inp.n_q_heads, nkv, d, inp.scale)


@pytest.mark.parametrize("i8", [False, True])
@pytest.mark.parametrize("merge_mode", [0, 2])
def test_batched_equals_per_slot_bitwise(i8, merge_mode):
    seq = (1024, 8192, 0, 2000, 1, 333, 40000)
    inp = make_inputs(seq, 16, 8, 256, i8, seed_base=7500)
    for W in (0, 700):
        batched = run_gpu(inp, W, merge_mode=merge_mode)
        for s in range(len(seq)):
            solo = run_gpu(_slot_inputs(inp, s), W, merge_mode=merge_mode)
            assert torch.equal(batched[s:s + 1], solo), (W, s)


@pytest.mark.parametrize("merge_mode", [0, 2])
def test_run_to_run_bitwise_determinism(merge_mode):
    inp = make_inputs((5000, 1234, 77), 16, 8, 256, True, seed_base=7600)
    dev = to_device(inp)
    a = run_gpu(inp, 0, dev_tensors=dev, merge_mode=merge_mode)
    b = run_gpu(inp, 0, dev_tensors=dev, merge_mode=merge_mode)
    assert torch.equal(a, b)


@pytest.mark.parametrize("merge_mode", [0, 2])
def test_recycled_workspace_is_never_read_stale(merge_mode):
    # A long call with a NaN query leaves NaN partials all over the workspace;
    # shorter and longer calls afterwards must not read any of them.
    long_nan = make_inputs((20000, 9000), 16, 8, 256, False, seed_base=7700)
    long_nan.q[:] = float("nan")
    run_gpu(long_nan, 0, merge_mode=merge_mode)
    for seq, seed in (((3000,), 7701), ((600, 20000), 7702), ((9000, 100, 5), 7703)):
        inp = make_inputs(seq, 16, 8, 256, False, seed_base=seed)
        got = run_gpu(inp, 0, merge_mode=merge_mode).cpu().numpy()
        ref = run_oracle(inp, 0)
        assert_parity(got, ref, f"after NaN workspace {seq}")
        run_gpu(long_nan, 0, merge_mode=merge_mode)


def test_side_stream():
    inp = make_inputs((4096, 100), 16, 8, 256, False, seed_base=7800)
    dev = to_device(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        got = run_gpu(inp, 0, dev_tensors=dev, stream=s)
    ref = run_oracle(inp, 0)
    assert_parity(got.cpu().numpy(), ref, "side stream")


def test_binding_rejects_wrong_dtype_on_gpu():
    inp = make_inputs((10,), 2, 1, 64, False, seed_base=7900)
    q, k, v, _ = to_device(inp)
    out = torch.empty((1, 2, 64), dtype=torch.float16, device=q.device)
    with pytest.raises(TypeError):
        binding.attn_decode(q, k, v, None, (10,), 0, out, 1, 2, 1, 64, inp.scale)


def test_default_stream_is_torchs_current_stream():
    """The binding's default stream handle is torch's current stream, also inside a stream context."""
    assert binding._stream_handle(None, 0) == torch.cuda.current_stream(0).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert binding._stream_handle(None, 0) == s.cuda_stream == torch.cuda.current_stream(0).cuda_stream
    assert binding._stream_handle(None, 0) == torch.cuda.current_stream(0).cuda_stream
