"""Pins of the oracle's fixed-capacity (linear / ring) cache entry point.

The cache layout keeps each (cache slot, kv head) in ``capacity`` rows; linear
storage puts position p in row p, ring storage in row p mod capacity, so only
the last ``capacity`` positions exist (mlx-native flash_attn_vec_hybrid.metal,
batched kernels: kv_seq_len = min(pos + 1, capacity) for the ring and the
logical-to-physical row remap).  The cache path is pinned to the packed path
(itself pinned in test_oracle_pins.py) by placing the same rows in a cache,
and by closed forms over the position values.
"""
import numpy as np
import pytest

from oracle import oracle_attn_decode, oracle_attn_decode_cache


def _rng(seed):
    return np.random.default_rng(seed)


def _packed_case(seed, seq_lens, n_q, n_kv, d, v_int8):
    r = _rng(seed)
    total = sum(seq_lens) * n_kv * d
    q = r.standard_normal((len(seq_lens), n_q, d)).astype(np.float16)
    k = r.standard_normal(total).astype(np.float16)
    if v_int8:
        v = r.integers(-127, 128, size=total).astype(np.int8)
        vs = r.uniform(0.001, 0.05, size=total // 32).astype(np.float16)
    else:
        v = r.standard_normal(total).astype(np.float16)
        vs = None
    return q, k, v, vs


def _to_cache(arr, seq_lens, n_kv, width, cap, ring, filler_seed, dtype, slot_of):
    """Place each packed slot into cache slot slot_of[s] (row p or p % cap); other rows random."""
    n_cache = max(slot_of) + 1
    r = _rng(filler_seed)
    if dtype == np.int8:
        cache = r.integers(-127, 128, size=(n_cache, n_kv, cap, width)).astype(np.int8)
    else:
        cache = r.standard_normal((n_cache, n_kv, cap, width)).astype(dtype)
    off = 0
    for s, L in enumerate(seq_lens):
        blk = arr[off:off + n_kv * L * width].reshape(n_kv, L, width)
        off += n_kv * L * width
        lo = max(L - cap, 0) if ring else 0
        for p in range(lo, L):
            cache[slot_of[s], :, p % cap if ring else p] = blk[:, p]
    return cache


@pytest.mark.parametrize("v_int8", [False, True])
@pytest.mark.parametrize("ring", [0, 1])
def test_cache_equals_packed_slots(v_int8, ring):
    seq_lens, n_q, n_kv, d, cap, W = (9, 30, 1, 17), 4, 2, 64, 20, 0
    if not ring:
        seq_lens = (9, 20, 1, 17)
    q, k, v, vs = _packed_case(11 + ring, seq_lens, n_q, n_kv, d, v_int8)
    slot_of = [3, 0, 2, 1]
    kc = _to_cache(k, seq_lens, n_kv, d, cap, ring, 1, np.float16, slot_of)
    vc = _to_cache(v, seq_lens, n_kv, d, cap, ring, 2, np.int8 if v_int8 else np.float16, slot_of)
    sc = None if vs is None else _to_cache(vs, seq_lens, n_kv, d // 32, cap, ring, 3, np.float16, slot_of)
    positions = [L - 1 for L in seq_lens]
    got = oracle_attn_decode_cache(q, kc, vc, sc, slot_of, positions, 4, cap, ring, W, n_q, n_kv, d, 0.3)
    # a ring holds the last `cap` positions: the packed slot with window `cap` attends the same rows
    ref = oracle_attn_decode(q, k, v, vs, seq_lens, cap if ring else W, n_q, n_kv, d, 0.3)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("pos,cap,ring,W", [
    (0, 8, 0, 0), (7, 8, 0, 0), (5, 8, 0, 3), (7, 8, 0, 100),
    (0, 8, 1, 0), (7, 8, 1, 0), (8, 8, 1, 0), (29, 8, 1, 0), (29, 8, 1, 3), (29, 8, 1, 20),
    (1000, 64, 1, 0), (1000, 64, 1, 17), (63, 64, 1, 64),
])
def test_position_values_give_the_attended_mean(pos, cap, ring, W):
    # q = 0: uniform weights over the attended positions; the row holding position p has V = p
    d, n_kv = 8, 1
    L = pos + 1
    v = np.full((1, n_kv, cap, d), -1.0)            # rows not holding a live position
    lo_store = max(L - cap, 0) if ring else 0
    for p in range(lo_store, L):
        v[0, 0, p % cap if ring else p] = p
    v = v.astype(np.float16)
    k = _rng(pos + cap).standard_normal((1, n_kv, cap, d)).astype(np.float16)
    q = np.zeros((1, 1, d), dtype=np.float16)
    got = oracle_attn_decode_cache(q, k, v, None, [0], [pos], 1, cap, ring, W, 1, n_kv, d, 1.0)
    lo = lo_store
    if W > 0:
        lo = max(lo, L - W)
    assert np.abs(got[0, 0] - (lo + L - 1) / 2).max() <= 1e-12 * L


def test_several_queries_of_one_slot_are_independent_rows():
    # speculative-verify shape: one cache slot, consecutive positions, each its own causal prefix
    n_q, n_kv, d, cap = 4, 2, 32, 64
    r = _rng(5)
    k = r.standard_normal((2, n_kv, cap, d)).astype(np.float16)
    v = r.standard_normal((2, n_kv, cap, d)).astype(np.float16)
    q = r.standard_normal((4, n_q, d)).astype(np.float16)
    sid, pos = [1, 1, 1, 0], [40, 41, 42, 10]
    multi = oracle_attn_decode_cache(q, k, v, None, sid, pos, 2, cap, 0, 0, n_q, n_kv, d, 0.2)
    for i in range(4):
        one = oracle_attn_decode_cache(q[i:i + 1], k, v, None, [sid[i]], [pos[i]], 2, cap, 0, 0,
                                       n_q, n_kv, d, 0.2)
        assert np.array_equal(multi[i], one[0])
    # and a later position sees strictly more keys: outputs differ
    assert not np.array_equal(multi[0], multi[1])


@pytest.mark.parametrize("kw", [
    dict(positions=[8]),            # linear cache: position past the capacity
    dict(slot_ids=[2]),             # slot out of range
    dict(positions=[-1]),
    dict(ring=2),
])
def test_cache_invalid_arguments(kw):
    a = dict(slot_ids=[0], positions=[3], ring=0)
    a.update(kw)
    k = np.zeros((2, 1, 8, 64), dtype=np.float16)
    q = np.zeros((1, 1, 64), dtype=np.float16)
    with pytest.raises(ValueError):
        oracle_attn_decode_cache(q, k, k, None, a["slot_ids"], a["positions"], 2, 8, a["ring"], 0,
                                 1, 1, 64, 1.0)
