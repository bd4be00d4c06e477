"""Pins of the oracle's codebook encode, its codebook-V append into a
fixed-capacity cache, and its cache-layout attention over codebook V.

The encode (the hybrid regime's KV encode: hf2q gemma4 batched_body.rs, the
FWHT-V encode per slot and position; mlx-native flash_attn_vec_hybrid.metal,
the TQ-HB layout it fills) rotates a row, y = H (s * v) / sqrt(D), takes one
norm per block of B = min(D, 256) coordinates, and stores the index of the
level nearest to u = y * sqrt(B) / norm.

* Closed forms: a scaled unit vector rotates to +-c / sqrt(D) in every
  coordinate with the sign pattern of a Hadamard row, so u = +-1 exactly and
  the norm is |c| (or |c| / sqrt(2) per block at D = 512).
* scipy's Hadamard matrix, a plain numpy norm and an argmin over the levels
  recompute the whole encode independently.
* Invariances: scaling v by a power of two scales the norms and leaves every
  code alone; negating v mirrors the codes on a symmetric table.
* Decoding the codes and undoing the rotation gives v back to the Lloyd-Max
  distortion, and a table with the wrong levels is shown to fail that.
* The append puts K (fp16, as the fp16 append does) and the encoded V into
  the row of each (slot, position), linear and ring, and nowhere else.
* Cache attention over codebook V agrees with the already pinned fp16-V cache
  oracle when the table and norms make every V value a known fp16 number,
  and with the packed-slot codebook oracle on the same rows.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from decode_attention_kv_02_amd.workloads import codebook_levels, make_signs
from oracle import (oracle_attn_decode_cache, oracle_attn_decode_cache_cb, oracle_attn_decode_cb,
                    oracle_codebook_encode, oracle_fwht_undo, oracle_kv_append, oracle_kv_append_cb)

SYM4 = np.array([-1.5, -0.5, 0.5, 1.5], dtype=np.float32)


def _rng(seed):
    return np.random.default_rng(seed)


def _signs(d, seed):
    return make_signs(d, seed).numpy()


# ---------------------------------------------------------------- encode

@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("k", [0, 5, 63])
def test_scaled_unit_vector_rotates_to_a_signed_hadamard_row(d, k):
    s = _signs(d, 11 + k)
    c = -2.5
    v = np.zeros((1, d), dtype=np.float32)
    v[0, k] = c
    table = np.array([-1.2, -0.3, 0.4, 1.1], dtype=np.float32)   # +-1 is nearest to 1.1 and -1.2, no tie
    codes, norms, u = oracle_codebook_encode(v, s, table, 2)
    pattern = np.array([(-1) ** bin(i & k).count("1") for i in range(d)], dtype=np.float64)
    want_u = np.sign(c) * s[k] * pattern
    assert np.allclose(u[0], want_u, atol=1e-12, rtol=0)
    assert np.array_equal(codes[0], np.where(want_u > 0, 3, 0))
    B = min(d, 256)
    assert np.allclose(norms[0], abs(c) * math.sqrt(B / d), rtol=1e-7, atol=0)


@pytest.mark.parametrize("d,bits", [(64, 5), (128, 8), (256, 6), (512, 8)])
def test_encode_matches_scipy_hadamard_and_argmin(d, bits):
    r = _rng(100 + d)
    v = r.standard_normal((20, d)).astype(np.float32)
    s = _signs(d, 200 + d)
    cb = codebook_levels(bits).numpy()
    codes, norms, u = oracle_codebook_encode(v, s, cb, bits)
    y = (scipy.linalg.hadamard(d).astype(np.float64) @ (s[:, None] * v.T.astype(np.float64))).T / math.sqrt(d)
    B = min(d, 256)
    yb = y.reshape(20, d // B, B)
    nb = np.sqrt((yb ** 2).sum(-1))
    assert np.allclose(norms, nb, rtol=1e-7, atol=0)
    ub = (yb * (math.sqrt(B) / nb)[..., None]).reshape(20, d)
    assert np.allclose(u, ub, rtol=0, atol=1e-12)
    want = np.abs(ub[..., None] - cb.astype(np.float64)).argmin(-1)
    assert np.array_equal(codes, want.astype(np.uint8))


def test_power_of_two_scale_changes_norms_only():
    d = 256
    r = _rng(7)
    v = r.standard_normal((16, d)).astype(np.float32)
    s = _signs(d, 8)
    cb = codebook_levels(8).numpy()
    c1, n1, u1 = oracle_codebook_encode(v, s, cb, 8)
    c4, n4, u4 = oracle_codebook_encode(v * 4, s, cb, 8)
    assert np.array_equal(c1, c4)
    assert np.array_equal(n4, n1 * 4)
    assert np.array_equal(u1, u4)


@pytest.mark.parametrize("d", [128, 512])
def test_negation_mirrors_codes_on_a_symmetric_table(d):
    r = _rng(9)
    v = r.standard_normal((8, d)).astype(np.float32)
    s = _signs(d, 10)
    c, n, _ = oracle_codebook_encode(v, s, SYM4, 2)
    cm, nm, _ = oracle_codebook_encode(-v, s, SYM4, 2)
    assert np.array_equal(cm, 3 - c)
    assert np.array_equal(n, nm)


def test_zero_row_gives_code_zero_and_norm_zero():
    codes, norms, u = oracle_codebook_encode(np.zeros((2, 512), np.float32), _signs(512, 1), SYM4, 2)
    assert not codes.any() and not norms.any() and not u.any()


def _decode(codes, norms, cb):
    d = codes.shape[-1]
    B = min(d, 256)
    lv = cb.astype(np.float64)[codes]
    return (lv.reshape(*codes.shape[:-1], d // B, B) * (norms.astype(np.float64) / math.sqrt(B))[..., None]
            ).reshape(codes.shape)


@pytest.mark.parametrize("bits,d,bound", [(8, 256, 0.02), (8, 512, 0.02), (6, 128, 0.05), (5, 64, 0.1)])
def test_decode_and_undo_give_v_back_to_the_quantiser_distortion(bits, d, bound):
    r = _rng(300 + bits)
    v = r.standard_normal((64, d)).astype(np.float32)
    s = _signs(d, 301)
    cb = codebook_levels(bits).numpy()
    codes, norms, _ = oracle_codebook_encode(v, s, cb, bits)
    back = oracle_fwht_undo(_decode(codes, norms, cb), s)
    err = np.linalg.norm(back - v) / np.linalg.norm(v)
    assert err < bound
    # a table with the wrong levels (every level halved) encodes far worse
    codes2, norms2, _ = oracle_codebook_encode(v, s, cb * 0.5, bits)
    back2 = oracle_fwht_undo(_decode(codes2, norms2, cb), s)
    assert np.linalg.norm(back2 - v) / np.linalg.norm(v) > 5 * bound


def test_encode_rejects_invalid_arguments():
    with pytest.raises(ValueError):
        oracle_codebook_encode(np.zeros((1, 96), np.float32), np.ones(96), SYM4, 2)   # not a power of two
    with pytest.raises(ValueError):
        oracle_codebook_encode(np.zeros((1, 64), np.float32), np.ones(64), np.zeros(512, np.float32), 9)


# ---------------------------------------------------------------- append

def _empty_cache(n_slots, n_kv, cap, d, fill=0):
    B = min(d, 256)
    kc = np.full(n_slots * n_kv * cap * d, fill, dtype=np.float16)
    vc = np.full(n_slots * n_kv * cap * d, 0xAB, dtype=np.uint8)
    vn = np.full(n_slots * n_kv * cap * d // B, -1.0, dtype=np.float32)
    return kc, vc, vn


@pytest.mark.parametrize("ring", [0, 1])
@pytest.mark.parametrize("d", [64, 512])
def test_append_places_each_row_and_touches_nothing_else(ring, d):
    n_slots, n_kv, cap, bits = 3, 2, 16, 8
    B = min(d, 256)
    sid = [2, 0, 2, 1]
    pos = [5, 15, 22, 0] if ring else [5, 15, 6, 0]
    r = _rng(400 + d + ring)
    kn = r.standard_normal((4, n_kv, d)).astype(np.float32)
    vn_ = r.standard_normal((4, n_kv, d)).astype(np.float32)
    s = _signs(d, 401)
    cb = codebook_levels(bits).numpy()
    kc, vc, nm = _empty_cache(n_slots, n_kv, cap, d)
    k2, v2, n2, u = oracle_kv_append_cb(kn, vn_, s, cb, bits, kc, vc, nm, sid, pos, n_slots, cap, ring, n_kv, d)
    # K exactly as the (pinned) fp16 append writes it
    kf, _, _ = oracle_kv_append(kn, vn_, kc, np.zeros(kc.size, np.float16), None, sid, pos, n_slots, cap,
                                ring, n_kv, d)
    assert np.array_equal(k2.view(np.uint16), kf.view(np.uint16))
    codes, norms, uu = oracle_codebook_encode(vn_.reshape(-1, d), s, cb, bits)
    touched = np.zeros(n_slots * n_kv * cap, dtype=bool)
    for i in range(4):
        phys = pos[i] % cap if ring else pos[i]
        for h in range(n_kv):
            row = (sid[i] * n_kv + h) * cap + phys
            touched[row] = True
            assert np.array_equal(v2[row * d:(row + 1) * d], codes[i * n_kv + h])
            assert np.array_equal(n2[row * (d // B):(row + 1) * (d // B)], norms[i * n_kv + h])
            assert np.array_equal(u[i, h], uu[i * n_kv + h])
    rows = np.repeat(~touched, d)
    assert np.all(v2[rows] == 0xAB) and np.all(n2[np.repeat(~touched, d // B)] == -1.0)


def test_append_rejects_collisions_and_bad_bits():
    kc, vc, nm = _empty_cache(1, 1, 8, 64)
    kn = np.zeros((2, 1, 64), np.float32)
    s = np.ones(64, np.float32)
    with pytest.raises(ValueError):   # 3 and 11 share ring row 3
        oracle_kv_append_cb(kn, kn, s, SYM4, 2, kc, vc, nm, [0, 0], [3, 11], 1, 8, 1, 1, 64)
    with pytest.raises(ValueError):
        oracle_kv_append_cb(kn, kn, s, np.zeros(512, np.float32), 9, kc, vc, nm, [0, 0], [1, 2], 1, 8, 0, 1, 64)
    with pytest.raises(ValueError):   # linear position past the capacity
        oracle_kv_append_cb(kn, kn, s, SYM4, 2, kc, vc, nm, [0, 0], [1, 8], 1, 8, 0, 1, 64)


# ---------------------------------------------------------------- cache attention over codebook V

def _exact_codebook_cache(r, n_slots, n_kv, cap, d):
    """Codes, norms and a 4-bit table whose decoded values are exact fp16 numbers: levels k/8 and
    norms sqrt(B) * 2^-e, so a V element is (k/8) * 2^-e (sqrt(B) exact: B = 64 or 256).  The
    stored bytes carry random high bits, which a 4-bit read must ignore."""
    B = min(d, 256)
    cb = (np.arange(16, dtype=np.float32) - 7.5) / 8
    low = r.integers(0, 16, n_slots * n_kv * cap * d)
    codes = (low + 16 * r.integers(0, 16, low.size)).astype(np.uint8)
    e = r.integers(0, 3, n_slots * n_kv * cap * d // B)
    norms = (math.sqrt(B) * 2.0 ** -e).astype(np.float32)
    vals = (cb.astype(np.float64)[low].reshape(-1, B) * (norms.astype(np.float64) / math.sqrt(B))[:, None])
    v16 = vals.reshape(-1).astype(np.float16)
    assert np.array_equal(v16.astype(np.float64), vals.reshape(-1))
    return cb, codes, norms, v16


@pytest.mark.parametrize("d,ring,window", [(64, 0, 0), (256, 1, 0), (512, 0, 0), (64, 1, 5)])
def test_cache_codebook_equals_cache_fp16_with_the_same_values(d, ring, window):
    r = _rng(500 + d)
    n_slots, n_kv, cap, nq = 3, 2, 24, 4
    cb, codes, norms, v16 = _exact_codebook_cache(r, n_slots, n_kv, cap, d)
    k = (r.standard_normal(n_slots * n_kv * cap * d) * 0.5).astype(np.float16)
    sid = [1, 0, 2, 1]
    pos = [23, 0, 40, 7] if ring else [23, 0, 12, 7]
    q = r.standard_normal((4, nq, d)).astype(np.float16)
    scale = 1 / math.sqrt(d)
    got = oracle_attn_decode_cache_cb(q, k, codes, norms, cb, 4, sid, pos, n_slots, cap, ring, window, nq,
                                      n_kv, d, scale)
    want = oracle_attn_decode_cache(q, k, v16, None, sid, pos, n_slots, cap, ring, window, nq, n_kv, d, scale)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("d", [128, 512])
def test_cache_codebook_equals_packed_codebook_on_the_same_rows(d):
    # a linear cache whose query i sits at the last stored position of its own slot
    r = _rng(600 + d)
    n_kv, nq, cap = 2, 8, 40
    B = min(d, 256)
    seq = [40, 13, 1]
    cb = codebook_levels(8).numpy()
    codes = r.integers(0, 256, 3 * n_kv * cap * d).astype(np.uint8)
    norms = r.uniform(0.5, 20, 3 * n_kv * cap * d // B).astype(np.float32)
    k = (r.standard_normal(3 * n_kv * cap * d) * 0.5).astype(np.float16)
    q = r.standard_normal((3, nq, d)).astype(np.float16)
    got = oracle_attn_decode_cache_cb(q, k, codes, norms, cb, 8, [0, 1, 2], [L - 1 for L in seq], 3, cap, 0,
                                      0, nq, n_kv, d, 0.0625)
    # the same rows packed: slot s, head h, positions [0, L_s)
    kk, cc, nn = [], [], []
    for s_, L in enumerate(seq):
        for h in range(n_kv):
            row0 = (s_ * n_kv + h) * cap
            kk.append(k[row0 * d:(row0 + L) * d])
            cc.append(codes[row0 * d:(row0 + L) * d])
            nn.append(norms[row0 * (d // B):(row0 + L) * (d // B)])
    want = oracle_attn_decode_cb(q, np.concatenate(kk), np.concatenate(cc), np.concatenate(nn), cb, 8, seq, 0,
                                 nq, n_kv, d, 0.0625)
    assert np.array_equal(got, want)
