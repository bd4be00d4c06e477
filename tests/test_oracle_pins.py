"""Pins of the CPU fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute: a library
routine (numpy's binary16 decoder, torch's CPU scaled_dot_product_attention in
float64), a closed form (uniform weights, two-key logistic weights, exact
rational dequantised means), an invariant of the definition (permutation of
keys, window == truncation, identical rows), or the hand-derived cases under
``tests/golden/``.  Together they fail on a dropped scale, a sign error in the
exponent, a missing normalisation, an off-by-one window, an interleaved GQA
map, a wrong slot offset or a wrong int8 block index.

The definition is the one the pages' decode kernels reach: mlx-native
flash_attn_vec_hybrid.metal (GQA map, window start, QK then scale, online
softmax, 1/S with S == 0 giving zeros) and tessl nn.rs flash_attn_decode
(window 0 is global attention).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import half_to_double, oracle_attn_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_case(seed, seq_lens, n_q, n_kv, d, v_int8=False):
    r = _rng(seed)
    total = sum(seq_lens) * n_kv * d
    q = r.standard_normal((len(seq_lens), n_q, d)).astype(np.float16)
    k = r.standard_normal(total).astype(np.float16)
    if v_int8:
        v = r.integers(-127, 128, size=total).astype(np.int8)
        vs = (r.uniform(0.001, 0.05, size=total // 32)).astype(np.float16)
    else:
        v = r.standard_normal(total).astype(np.float16)
        vs = None
    return q, k, v, vs


def _slot_view(arr, seq_lens, n_kv, width, s):
    """[n_kv, L_s, width] view of slot s in a packed ragged array."""
    off = sum(seq_lens[:s]) * n_kv * width
    L = seq_lens[s]
    return arr[off:off + n_kv * L * width].reshape(n_kv, L, width)


def _dequant(v, vs, d):
    if vs is None:
        return v.astype(np.float64)
    return v.astype(np.float64) * np.repeat(vs.astype(np.float64), 32)


def test_half_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero too
    assert math.copysign(1.0, half_to_double(0x8000)) == -1.0


SDPA_CASES = [
    # seq_lens, n_q, n_kv, d, window, v_int8
    ((5,), 1, 1, 8, 0, False),
    ((7,), 4, 2, 8, 0, False),
    ((3, 9, 1), 4, 1, 4, 0, False),
    ((6, 0, 11), 6, 3, 8, 4, False),
    ((13, 2), 8, 2, 8, 5, False),
    ((4, 10), 2, 2, 64, 3, True),
    ((17,), 8, 8, 32, 0, True),
]


@pytest.mark.parametrize("case", SDPA_CASES)
def test_matches_torch_sdpa_float64(case):
    seq_lens, n_q, n_kv, d, window, v_int8 = case
    q, k, v, vs = _random_case(hash(case) % 2**32, seq_lens, n_q, n_kv, d, v_int8)
    scale = float(np.float32(0.37))
    got = oracle_attn_decode(q, k, v, vs, seq_lens, window, n_q, n_kv, d, scale, threads=3)
    vdq = _dequant(v, vs, d)
    G = n_q // n_kv
    for s, L in enumerate(seq_lens):
        lo = L - window if (window > 0 and L > window) else 0
        if L == 0:
            assert np.all(got[s] == 0.0)
            continue
        K = torch.from_numpy(_slot_view(k, seq_lens, n_kv, d, s).astype(np.float64))[:, lo:L]
        V = torch.from_numpy(_slot_view(vdq, seq_lens, n_kv, d, s))[:, lo:L]
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        Q = torch.from_numpy(q[s].astype(np.float64)).unsqueeze(1)
        ref = F.scaled_dot_product_attention(Q, K, V, scale=scale).squeeze(1).numpy()
        err = np.abs(got[s] - ref).max() / max(np.abs(ref).max(), 1e-300)
        assert err <= 1e-12, (s, err)


def test_single_key_returns_its_row_exactly():
    d, n_kv, n_q = 16, 2, 4
    q, k, v, _ = _random_case(11, (1, 1), n_q, n_kv, d)
    got = oracle_attn_decode(q, k, v, None, (1, 1), 0, n_q, n_kv, d, 0.25)
    for s in range(2):
        Vs = _slot_view(v, (1, 1), n_kv, d, s).astype(np.float64)
        for h in range(n_q):
            assert np.array_equal(got[s, h], Vs[h // 2, 0])
    # window 1 on a longer cache keeps only the newest row
    q, k, v, _ = _random_case(12, (9,), n_q, n_kv, d)
    got = oracle_attn_decode(q, k, v, None, (9,), 1, n_q, n_kv, d, 0.25)
    Vs = _slot_view(v, (9,), n_kv, d, 0).astype(np.float64)
    for h in range(n_q):
        assert np.array_equal(got[0, h], Vs[h // 2, 8])


def test_single_key_int8_is_code_times_block_scale():
    d = 64
    q, k, v, vs = _random_case(13, (1,), 1, 1, d, v_int8=True)
    got = oracle_attn_decode(q, k, v, vs, (1,), 0, 1, 1, d, 0.125)
    exp = np.array([float(v[i]) * float(vs[i // 32]) for i in range(d)])
    assert np.array_equal(got[0, 0], exp)


def test_identical_value_rows_return_that_row():
    d, L, n_q, n_kv = 32, 50, 2, 1
    q, k, _, _ = _random_case(21, (L,), n_q, n_kv, d)
    row = _rng(22).standard_normal(d).astype(np.float16)
    v = np.tile(row, L * n_kv)
    got = oracle_attn_decode(q, k, v, None, (L,), 0, n_q, n_kv, d, 0.7)
    r = row.astype(np.float64)
    for h in range(n_q):
        assert np.abs(got[0, h] - r).max() <= 1e-15 * np.abs(r).max() * 4


def test_permuting_keys_with_their_values_changes_nothing():
    d, L, n_q, n_kv = 16, 40, 4, 2
    q, k, v, _ = _random_case(31, (L,), n_q, n_kv, d)
    perm = _rng(32).permutation(L)
    kp = k.reshape(n_kv, L, d)[:, perm].reshape(-1).copy()
    vp = v.reshape(n_kv, L, d)[:, perm].reshape(-1).copy()
    a = oracle_attn_decode(q, k, v, None, (L,), 0, n_q, n_kv, d, 0.3)
    b = oracle_attn_decode(q, kp, vp, None, (L,), 0, n_q, n_kv, d, 0.3)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max()


@pytest.mark.parametrize("v_int8", [False, True])
def test_window_equals_truncated_cache(v_int8):
    d, n_q, n_kv = 64, 4, 2
    seq_lens = (20, 7, 33)
    W = 8
    q, k, v, vs = _random_case(41, seq_lens, n_q, n_kv, d, v_int8)
    full = oracle_attn_decode(q, k, v, vs, seq_lens, W, n_q, n_kv, d, 0.2)
    for s, L in enumerate(seq_lens):
        lo = max(L - W, 0)
        kt = _slot_view(k, seq_lens, n_kv, d, s)[:, lo:].reshape(-1).copy()
        vt = _slot_view(v, seq_lens, n_kv, d, s)[:, lo:].reshape(-1).copy()
        st = None
        if vs is not None:
            st = _slot_view(vs, seq_lens, n_kv, d // 32, s)[:, lo:].reshape(-1).copy()
        one = oracle_attn_decode(q[s:s + 1], kt, vt, st, (L - lo,), 0, n_q, n_kv, d, 0.2)
        assert np.array_equal(full[s], one[0])


@pytest.mark.parametrize("L,W", [(10, 0), (10, 3), (10, 9), (10, 10), (10, 11), (10, 1),
                                 (1, 0), (300, 64), (2048, 1000)])
def test_uniform_weights_give_window_mean(L, W):
    # q = 0 makes every logit equal; V row j holds j, so the mean is (lo + L - 1)/2
    d = 8
    q = np.zeros((1, 1, d), dtype=np.float16)
    k = _rng(L + W).standard_normal(L * d).astype(np.float16)
    v = np.repeat(np.arange(L, dtype=np.float64), d).astype(np.float16)
    got = oracle_attn_decode(q, k, v, None, (L,), W, 1, 1, d, 1.0)
    lo = L - W if (W > 0 and L > W) else 0
    assert np.abs(got[0, 0] - (lo + L - 1) / 2).max() <= 1e-12 * L


def test_equal_keys_give_plain_mean():
    d, L = 16, 12
    q = _rng(51).standard_normal((1, 1, d)).astype(np.float16)
    krow = _rng(52).standard_normal(d).astype(np.float16)
    k = np.tile(krow, L)
    v = _rng(53).standard_normal(L * d).astype(np.float16)
    got = oracle_attn_decode(q, k, v, None, (L,), 0, 1, 1, d, 3.0)
    exp = v.reshape(L, d).astype(np.float64).mean(axis=0)
    assert np.abs(got[0, 0] - exp).max() <= 1e-14


@pytest.mark.parametrize("a,b,scale", [(1.5, 0.5, 1.0), (-2.0, 3.0, 0.25), (4.0, 4.0, 7.0),
                                       (0.125, -6.0, 2.5), (10.0, -10.0, 0.5)])
def test_two_keys_logistic_weights(a, b, scale):
    d = 4
    q = np.array([[[1, 0, 0, 0]]], dtype=np.float16)
    k = np.array([a, 1, 2, 3, b, -1, -2, -3], dtype=np.float16)
    v = np.array([2, 0, -1, 4, 0, 2, -1, -4], dtype=np.float16)
    scale32 = float(np.float32(scale))
    got = oracle_attn_decode(q, k, v, None, (2,), 0, 1, 1, d, scale32)
    w0 = 1.0 / (1.0 + math.exp(-scale32 * (a - b)))
    w1 = 1.0 / (1.0 + math.exp(-scale32 * (b - a)))
    exp = w0 * v[:4].astype(np.float64) + w1 * v[4:].astype(np.float64)
    assert np.abs(got[0, 0] - exp).max() <= 1e-14


@pytest.mark.parametrize("n_q,n_kv", [(8, 2), (6, 3), (4, 4), (16, 8), (5, 1)])
def test_gqa_map_uses_consecutive_heads(n_q, n_kv):
    d, seq_lens = 8, (5, 3)
    q, k, _, _ = _random_case(61, seq_lens, n_q, n_kv, d)
    # V of (slot s, kv head c) is the constant 10*s + c + 1
    parts = []
    for s, L in enumerate(seq_lens):
        for c in range(n_kv):
            parts.append(np.full(L * d, 10 * s + c + 1, dtype=np.float16))
    v = np.concatenate(parts)
    got = oracle_attn_decode(q, k, v, None, seq_lens, 0, n_q, n_kv, d, 0.5)
    G = n_q // n_kv
    for s in range(len(seq_lens)):
        for h in range(n_q):
            assert np.abs(got[s, h] - (10 * s + h // G + 1)).max() <= 1e-13


def test_int8_uniform_mean_is_exact_rational():
    # K = 0 gives uniform weights; the mean of code*scale is computed exactly
    d, L, n_kv = 96, 7, 2
    r = _rng(71)
    codes = r.integers(-127, 128, size=n_kv * L * d).astype(np.int8)
    scales = r.uniform(0.001, 0.09, size=n_kv * L * d // 32).astype(np.float16)
    q = r.standard_normal((1, 2, d)).astype(np.float16)
    k = np.zeros(n_kv * L * d, dtype=np.float16)
    got = oracle_attn_decode(q, k, codes, scales, (L,), 0, 2, n_kv, d, 0.3)
    for h in range(2):
        for dd in range(d):
            tot = Fraction(0)
            for j in range(L):
                e = (h * L + j) * d + dd
                tot += Fraction(int(codes[e])) * Fraction(float(scales[e // 32]))
            exact = float(tot / L)
            assert abs(got[0, h, dd] - exact) <= 1e-15 * max(abs(exact), 1e-3)


def test_empty_slot_gives_zeros_and_leaves_neighbours_alone():
    d, n_q, n_kv = 16, 2, 1
    seq_lens = (4, 0, 6)
    q, k, v, _ = _random_case(81, seq_lens, n_q, n_kv, d)
    got = oracle_attn_decode(q, k, v, None, seq_lens, 0, n_q, n_kv, d, 0.4)
    assert np.all(got[1] == 0.0)
    for s in (0, 2):
        L = seq_lens[s]
        ks = _slot_view(k, seq_lens, n_kv, d, s).reshape(-1).copy()
        vv = _slot_view(v, seq_lens, n_kv, d, s).reshape(-1).copy()
        one = oracle_attn_decode(q[s:s + 1], ks, vv, None, (L,), 0, n_q, n_kv, d, 0.4)
        assert np.array_equal(got[s], one[0])


def test_row_subset_equals_full_rows():
    seq_lens, n_q, n_kv, d = (9, 4, 12), 4, 2, 32
    q, k, v, vs = _random_case(91, seq_lens, n_q, n_kv, d, v_int8=True)
    full = oracle_attn_decode(q, k, v, vs, seq_lens, 5, n_q, n_kv, d, 0.3)
    rows = [11, 0, 5, 7]
    sub = oracle_attn_decode(q, k, v, vs, seq_lens, 5, n_q, n_kv, d, 0.3, rows=rows)
    for i, r in enumerate(rows):
        assert np.array_equal(sub[i], full.reshape(-1, d)[r])


def _golden_array(spec, n, dtype):
    if isinstance(spec, str) and spec == "zeros":
        return np.zeros(n, dtype=dtype)
    return np.asarray(spec, dtype=dtype)


def test_golden_closed_form_cases():
    with open(GOLDEN) as fh:
        doc = json.load(fh)
    for c in doc["cases"]:
        seq, nq, nkv, d = tuple(c["seq_lens"]), c["n_q"], c["n_kv"], c["head_dim"]
        total = sum(seq) * nkv * d
        q = _golden_array(c["q"], len(seq) * nq * d, np.float16).reshape(len(seq), nq, d)
        k = _golden_array(c["k"], total, np.float16)
        if c["v_scales"] is None:
            v = _golden_array(c["v"], total, np.float16)
            vs = None
        else:
            blk = c["v"]["per_block"]
            v = np.concatenate([np.repeat(np.asarray(r, dtype=np.int8), blk) for r in c["v"]["rows"]])
            vs = np.asarray(c["v_scales"], dtype=np.float16)
        exp = c["expected"]
        if isinstance(exp, dict):
            exp = np.repeat(np.asarray(exp["per_block_values"], dtype=np.float64), exp["per_block"])
        exp = np.asarray(exp, dtype=np.float64).reshape(len(seq), nq, d)
        got = oracle_attn_decode(q, k, v, vs, seq, c["window"], nq, nkv, d,
                                 float(np.float32(c["scale"])))
        assert np.abs(got - exp).max() <= c["tol"], c["name"]


def test_invalid_arguments_are_rejected():
    q = np.zeros((1, 3, 8), dtype=np.float16)
    k = np.zeros(2 * 8 * 2, dtype=np.float16)
    with pytest.raises(ValueError):  # 3 q heads over 2 kv heads
        oracle_attn_decode(q, k, k, None, (2,), 0, 3, 2, 8, 1.0)
