"""Parity of attn_decode_cache (fixed-capacity linear / ring caches) with the oracle.

Query rows name a cache slot and the absolute position of their token; ring
storage keeps position p in row p mod capacity (mlx-native
flash_attn_vec_hybrid.metal, batched kernels: kv_seq_len = min(pos + 1,
capacity) on the ring and the logical-to-physical row remap).  Bar as for the
packed path: max-abs <= 2e-3 and relative L2 <= 1e-3 against the fp64 oracle,
bitwise per-query independence, bitwise agreement with the packed entry point
when both hold the same rows.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import CacheInputs, make_cache_inputs, make_inputs

from gpu_util import assert_parity, run_gpu, run_gpu_cache, run_oracle_cache, to_device

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


CASES = [
    # n_cache_slots, capacity, ring, slot_ids, positions, n_q, n_kv, D, v_int8, window
    (3, 300, 0, (2, 0, 1, 1), (299, 0, 150, 151), 4, 2, 128, False, 0),
    (2, 256, 1, (0, 1, 1), (255, 256, 1000), 8, 4, 256, True, 0),          # exactly full, one wrap, many laps
    (2, 1024, 1, (1, 0), (5000, 1023), 16, 8, 256, False, 700),            # window inside the ring
    (1, 64, 1, (0, 0, 0, 0), (63, 64, 65, 127), 2, 1, 64, True, 0),       # every wrap offset
    (4, 512, 0, (3, 3, 3, 3), (400, 401, 402, 403), 16, 2, 512, False, 0),  # verify shape, G = 8
    (2, 777, 1, (1, 0), (777 * 3 + 5, 776), 6, 2, 256, True, 100),         # odd capacity, G = 3
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_cache_parity(case):
    nc, cap, ring, sid, pos, nq, nkv, d, i8, W = case
    ci = make_cache_inputs(nc, cap, ring, sid, pos, nq, nkv, d, i8, seed_base=9000 + 31 * CASES.index(case))
    got = run_gpu_cache(ci, W).cpu().numpy()
    ref = run_oracle_cache(ci, W)
    _report(f"cache {case}", assert_parity(got, ref, str(case)))


@pytest.mark.parametrize("chunk", [1, 7, 64, 300])
def test_ring_chunks_across_the_wrap(chunk):
    ci = make_cache_inputs(2, 500, 1, (0, 1), (1234, 499), 8, 4, 256, True, seed_base=9100)
    got = run_gpu_cache(ci, 0, chunk=chunk).cpu().numpy()
    ref = run_oracle_cache(ci, 0)
    _report(f"ring chunk {chunk}", assert_parity(got, ref, f"chunk={chunk}"))


def test_slots_are_bitwise_independent():
    """Queries of several slots in one call, interleaved: each slot's rows equal a call with that
    slot's queries alone, bitwise (a query's kernel depends only on its own slot's queries), and
    each query alone matches the oracle (alone it may take the other partial kernel: here each
    slot's queries fill 4 or 6 matrix-core columns together, 2 alone)."""
    sid, pos = (1, 0, 1, 1, 0), (4000, 100, 4001, 1, 4095)
    ci = make_cache_inputs(2, 4096, 1, sid, pos, 16, 8, 256, True, seed_base=9200)
    dev = to_device(ci)
    batched = run_gpu_cache(ci, 0, dev_tensors=dev)
    ref = run_oracle_cache(ci, 0)
    for s_ in (0, 1):
        rows = [i for i in range(len(sid)) if sid[i] == s_]
        assert torch.equal(batched[rows], _sub_call(ci, dev, rows)), s_
    for i in range(len(sid)):
        assert_parity(_sub_call(ci, dev, [i]).cpu().numpy(), ref[i:i + 1], f"query {i} alone")


@pytest.mark.parametrize("i8", [False, True])
def test_linear_cache_matches_packed_entry_bitwise(i8):
    # the same rows in a [slot][kv][capacity][D] cache and packed back to back
    seq = (700, 2048, 1)
    cap = 2048
    inp = make_inputs(seq, 16, 8, 256, i8, seed_base=9300)
    d, nkv = 256, 8
    k = torch.zeros((3, nkv, cap, d), dtype=torch.float16)
    v = torch.zeros((3, nkv, cap, d), dtype=torch.int8 if i8 else torch.float16)
    vs = torch.zeros((3, nkv, cap, d // 32), dtype=torch.float16) if i8 else None
    off = 0
    for s, L in enumerate(seq):
        n = nkv * L * d
        k[s, :, :L] = inp.k[off:off + n].view(nkv, L, d)
        v[s, :, :L] = inp.v[off:off + n].view(nkv, L, d)
        if i8:
            vs[s, :, :L] = inp.v_scales[off // 32:(off + n) // 32].view(nkv, L, d // 32)
        off += n
    ci = CacheInputs(
        inp.q, k.reshape(-1), v.reshape(-1), None if vs is None else vs.reshape(-1), (0, 1, 2),
        tuple(L - 1 for L in seq), 3, cap, 0, 16, nkv, d, inp.scale)
    for W in (0, 500):
        packed = run_gpu(inp, W)
        cached = run_gpu_cache(ci, W)
        assert torch.equal(packed, cached), W


def test_cache_rejects_out_of_range_before_launch():
    ci = make_cache_inputs(2, 64, 0, (0,), (10,), 2, 1, 64, False, seed_base=9400)
    q, k, v, _ = to_device(ci)
    out = torch.empty((1, 2, 64), dtype=torch.float32, device=q.device)
    for sid, pos in (((2,), (10,)), ((0,), (64,)), ((0,), (-1,))):
        with pytest.raises(binding.AttnDecodeError):
            binding.attn_decode_cache(q, k, v, None, sid, pos, 1, 2, 64, 0, 0, out, 2, 1, 64, ci.scale)


def test_sliding_window_ring_at_serving_shape():
    # 8 slots, a 1024-position ring each (a sliding-window layer), tokens deep into long contexts
    pos = (131071, 90000, 1023, 1024, 50001, 77777, 2047, 300000)
    ci = make_cache_inputs(8, 1024, 1, tuple(range(8)), pos, 16, 8, 256, False, seed_base=9500)
    got = run_gpu_cache(ci, 0).cpu().numpy()
    ref = run_oracle_cache(ci, 0)
    _report("ring 8 x 1024", assert_parity(got, ref, "ring serving shape"))


def _sub_call(ci, dev, rows, W=0, chunk=0, path=0):
    """The queries `rows` of a cache call on their own."""
    one = CacheInputs(ci.q[rows].clone(), ci.k, ci.v, ci.v_scales, tuple(ci.slot_ids[i] for i in rows),
                      tuple(ci.positions[i] for i in rows), ci.n_cache_slots, ci.capacity, ci.ring, ci.n_q_heads,
                      ci.n_kv_heads, ci.head_dim, ci.scale)
    return run_gpu_cache(one, W, chunk=chunk, dev_tensors=(dev[0][rows].contiguous(), dev[1], dev[2], dev[3]),
                         path=path)


@pytest.mark.parametrize("nq,nkv,i8", [(16, 8, False), (8, 8, True), (4, 4, False), (16, 2, True)])
def test_draft_queries_share_a_workgroup_and_match_solo(nq, nkv, i8):
    # 4 consecutive draft positions per slot.  G = 1 makes 4 (draft, head) columns and G = 2
    # makes 8, a matrix-core workgroup either way (a single query needs 4 heads for that); G = 8
    # is on the matrix cores anyway and groups pairs.  Every query equals the oracle; each
    # slot's rows equal a call with that slot's queries alone bitwise (a query's kernel depends
    # only on its own slot's queries), and a single query's call too where grouping does not
    # change its kernel.  The same with the lane kernel forced, which groups up to 4 rows.
    sid = (0, 0, 0, 0, 1, 1, 1, 1, 2)
    pos = (3000, 3001, 3002, 3003, 700, 701, 702, 703, 50)
    G = nq // nkv
    ci = make_cache_inputs(3, 4096, 0, sid, pos, nq, nkv, 256, i8, seed_base=9600 + nq + nkv)
    dev = to_device(ci)
    got = run_gpu_cache(ci, 0, dev_tensors=dev)
    ref = run_oracle_cache(ci, 0)
    _report(f"drafts G={G}", assert_parity(got.cpu().numpy(), ref, "drafts"))
    for rows in ([0, 1, 2, 3], [4, 5, 6, 7], [8]):
        per_slot = _sub_call(ci, dev, rows)
        assert torch.equal(got[rows], per_slot), rows
    kernel_changes = G < 4      # the four drafts fill 4 matrix-core columns, a lone query does not
    for i in range(len(sid)):
        solo = _sub_call(ci, dev, [i])
        if kernel_changes and i < 8:
            assert_parity(solo.cpu().numpy(), ref[i:i + 1], f"solo {i}")
        else:
            assert torch.equal(got[i:i + 1], solo), i
    if G % 8:
        lanes = run_gpu_cache(ci, 0, dev_tensors=dev, path=1)
        _report(f"drafts G={G} lanes", assert_parity(lanes.cpu().numpy(), ref, "drafts on the lanes"))
        for rows in ([0, 1, 2, 3], [4, 5, 6, 7], [8]):
            assert torch.equal(lanes[rows], _sub_call(ci, dev, rows, path=1)), rows


DRAFT_CASES = [
    # n_q, n_kv, D, int8 V, ring, drafts per slot, forced chunk
    (16, 8, 256, False, 0, 4, 0),      # 2 heads x 4 drafts = 8 columns
    (16, 8, 128, True, 1, 8, 0),       # 2 x 8 = 16 columns, ring storage
    (16, 8, 256, False, 0, 5, 250),    # 10 columns; members end in different chunks
    (8, 8, 128, False, 0, 8, 0),       # 1 head x 8 drafts
    (16, 4, 512, False, 0, 2, 0),      # 4 heads x 2 drafts
    (16, 4, 256, True, 1, 4, 7),       # 4 x 4 = 16 columns, tiny chunks, ring
    (16, 2, 256, False, 0, 2, 0),      # 8 heads x 2 drafts (8 heads per kv head: pairs)
    (16, 8, 256, False, 0, 16, 0),     # 16 drafts: two groups of 8
    (16, 4, 512, True, 1, 2, 0),       # one-byte V at 512, where a group needs 8 columns
]


@pytest.mark.parametrize("case", DRAFT_CASES, ids=[f"d{i}" for i in range(len(DRAFT_CASES))])
def test_matrix_core_draft_groups(case):
    """Draft queries of a speculative-verify step as matrix-core columns (drafts x heads): each
    K and V row is read once for the whole group, each draft masked at its own position."""
    nq, nkv, d, i8, ring, nd, chunk = case
    cap = 2048
    base = (1999, 3100) if ring else (1999, 1500)
    sid = tuple(s for s in range(2) for _ in range(nd)) + (2,)
    pos = tuple(base[s] + t for s in range(2) for t in range(nd)) + (40,)
    ci = make_cache_inputs(3, cap, ring, sid, pos, nq, nkv, d, i8, seed_base=9700 + DRAFT_CASES.index(case))
    dev = to_device(ci)
    got = run_gpu_cache(ci, 0, chunk=chunk, dev_tensors=dev)
    ref = run_oracle_cache(ci, 0)
    _report(f"draft group {case}", assert_parity(got.cpu().numpy(), ref, f"{case}"))
    for s in range(3):
        rows = [i for i in range(len(sid)) if sid[i] == s]
        assert torch.equal(got[rows], _sub_call(ci, dev, rows, chunk=chunk)), f"slot {s}"


def test_draft_queries_with_forced_chunks_and_windows():
    # small forced chunks: members end in different chunks; a window gives each draft its own
    # start (no grouping), the full range groups them
    sid = (1, 1, 1, 1)
    pos = (1000, 1001, 1002, 1003)
    ci = make_cache_inputs(2, 2048, 0, sid, pos, 8, 8, 128, False, seed_base=9650)
    for W, chunk in ((0, 7), (0, 250), (300, 0), (300, 13)):
        got = run_gpu_cache(ci, W, chunk=chunk).cpu().numpy()
        ref = run_oracle_cache(ci, W)
        _report(f"drafts W={W} chunk={chunk}", assert_parity(got, ref, f"W={W} chunk={chunk}"))


@pytest.mark.parametrize("merge_mode", [0, 2])
def test_mixed_kernels_across_launch_groups(merge_mode):
    """20 slots: even slots verify 4 drafts (a matrix-core group at 2 heads per kv head), odd
    slots decode one token (lane kernel); 50 table entries span two launch groups of each
    kernel's own.  Every row matches the oracle, and each slot's rows equal a call with that
    slot's queries alone, bitwise, with the combine kernel or the in-kernel merge."""
    sid, pos = [], []
    for s in range(20):
        n = 4 if s % 2 == 0 else 1
        base = 300 + 37 * s
        sid += [s] * n
        pos += [base + t for t in range(n)]
    ci = make_cache_inputs(20, 1024, 0, tuple(sid), tuple(pos), 16, 8, 128, True, seed_base=9800 + merge_mode)
    dev = to_device(ci)
    got = run_gpu_cache(ci, 0, dev_tensors=dev, merge_mode=merge_mode)
    ref = run_oracle_cache(ci, 0)
    _report(f"mixed kernels merge_mode={merge_mode}", assert_parity(got.cpu().numpy(), ref, "mixed"))
    for s in (0, 1, 18, 19):
        rows = [i for i in range(len(sid)) if sid[i] == s]
        one = CacheInputs(ci.q[rows].clone(), ci.k, ci.v, ci.v_scales, tuple(sid[i] for i in rows),
                          tuple(pos[i] for i in rows), ci.n_cache_slots, ci.capacity, ci.ring, ci.n_q_heads,
                          ci.n_kv_heads, ci.head_dim, ci.scale)
        alone = run_gpu_cache(one, 0, dev_tensors=(dev[0][rows].contiguous(), dev[1], dev[2], dev[3]),
                              merge_mode=merge_mode)
        assert torch.equal(got[rows], alone), f"slot {s}"


def test_cache_call_of_many_queries():
    """130 query rows (two per slot over 65 ring slots, positions before and past the wrap) take the
    large query table: one launch, against the oracle."""
    rng = np.random.default_rng(9660)
    sid = tuple(s for s in range(65) for _ in range(2))
    pos = tuple(int(x) for x in rng.integers(0, 2000, size=130))
    ci = make_cache_inputs(65, 256, 1, sid, pos, 8, 4, 128, True, seed_base=9660)
    got = run_gpu_cache(ci, 0).cpu().numpy()
    ref = run_oracle_cache(ci, 0)
    _report("130 cache queries", assert_parity(got, ref, "130 cache queries"))


def test_per_call_chunk_floor_on_draft_groups():
    """The per-call chunk floor on a speculative-verify call (drafts grouped on the matrix cores and
    on the lanes) and a ring call: every output against the oracle."""
    for case in ((4, 4096, 0, tuple(s for s in range(4) for _ in range(4)),
                  tuple(4092 + t for _ in range(4) for t in range(4)), 16, 8, 256, False),
                 (4, 4096, 0, (0, 0, 1, 1, 2, 2, 3, 3), (4000, 4001) * 4, 4, 2, 128, True),
                 (8, 1024, 1, tuple(range(8)) * 2, tuple(range(5000, 5016)), 16, 8, 256, True)):
        nc, cap, ring, sid, pos, nq, nkv, d, i8 = case
        ci = make_cache_inputs(nc, cap, ring, sid, pos, nq, nkv, d, i8, seed_base=9670 + nq + ring)
        got = run_gpu_cache(ci, 0, chunk=binding.CHUNK_PER_CALL).cpu().numpy()
        _report(f"per-call floor {len(sid)} queries", assert_parity(got, run_oracle_cache(ci, 0), str(case[:3])))
