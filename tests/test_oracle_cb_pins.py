"""Pins of the oracle's codebook-V pieces: attention over codebook V and the
undo of the sign-randomised Walsh-Hadamard rotation.

Codebook V (mlx-native flash_attn_vec_hybrid.metal, the hybrid dequant; hf2q
gemma4 batched_body.rs, the KV encode and the FWHT sign-undo): each V element
is a byte index into a table of levels, with one fp32 norm per block of
B = min(D, 256) coordinates, and is worth level * norm / sqrt(B).  V lives in
the rotated basis v_rot = H (s * v) / sqrt(D), so the attention result comes
out rotated and the undo multiplies by s * H / sqrt(D).

* The undo is checked against hand-written closed forms (D = 1, 2, 4),
  scipy's Hadamard matrix, and the inverse of the input generator's butterfly
  transform (an independent implementation).
* The dequant is checked by a constant table (the output must equal that
  constant times norm / sqrt(B) whatever the weights are), by agreement with
  the fp16-V oracle when the table and norms make every V value a known
  number, with a different norm in each block at D = 512, and by the index
  mask (codes above 2**bits - 1 read the low bits only).
* The whole chain encode -> attend -> undo is checked against plain fp16-V
  attention on the unrotated V, to the accuracy the Lloyd-Max quantiser's
  distortion allows, and a wrong sign convention is shown to fail it.
* The input generator's Lloyd-Max levels are checked against their closed
  form (1 bit: +-sqrt(2/pi)) and the classical 2-bit table.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from decode_attention_kv_02_amd.workloads import (fwht_rows, lloyd_max_gaussian, make_codebook_inputs,
                                                   make_signs)
from oracle import oracle_attn_decode, oracle_attn_decode_cb, oracle_fwht_undo
import torch


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- FWHT undo

def test_undo_d1_is_the_sign():
    x = np.array([[3.5], [-2.0]])
    assert np.array_equal(oracle_fwht_undo(x, [-1.0]), -x)


def test_undo_d2_closed_form():
    a, b = 1.25, -0.5
    got = oracle_fwht_undo(np.array([[a, b]]), [1.0, -1.0])[0]
    r = 1 / math.sqrt(2)
    assert got[0] == pytest.approx((a + b) * r, abs=1e-15)
    assert got[1] == pytest.approx(-(a - b) * r, abs=1e-15)


def test_undo_d4_hand_matrix():
    H = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64)
    x = np.array([[1.0, 2.0, -3.0, 0.5]])
    s = np.array([1.0, -1.0, -1.0, 1.0])
    want = s * (H @ x[0]) / 2
    assert np.allclose(oracle_fwht_undo(x, s)[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d", [8, 64, 256, 512])
def test_undo_matches_scipy_hadamard(d):
    r = _rng(d)
    x = r.standard_normal((3, d))
    s = np.where(r.random(d) < 0.5, -1.0, 1.0)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    want = s * (x @ H.T) / math.sqrt(d)
    assert np.allclose(oracle_fwht_undo(x, s), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 256, 512])
def test_undo_inverts_the_generators_rotation(d):
    r = _rng(d + 1)
    v = r.standard_normal((5, d))
    s = make_signs(d, 99).double()
    rot = fwht_rows(torch.from_numpy(v) * s) / math.sqrt(d)
    back = oracle_fwht_undo(rot.numpy(), s.numpy())
    assert np.allclose(back, v, rtol=0, atol=1e-12)


def test_undo_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle_fwht_undo(np.zeros((1, 96)), np.ones(96))


# ---------------------------------------------------------------- dequant

def _random_qk(r, seq_lens, n_q, n_kv, d):
    n = sum(seq_lens) * n_kv * d
    q = r.standard_normal(len(seq_lens) * n_q * d).astype(np.float16)
    k = r.standard_normal(n).astype(np.float16)
    return q, k


@pytest.mark.parametrize("d", [64, 256, 512])
def test_constant_codebook_gives_constant_times_norm_over_sqrt_b(d):
    r = _rng(5)
    seq, n_q, n_kv = (33, 1, 70), 4, 2
    B = min(d, 256)
    q, k = _random_qk(r, seq, n_q, n_kv, d)
    n_rows = sum(seq) * n_kv
    codes = r.integers(0, 256, n_rows * d).astype(np.uint8)
    norms = np.full(n_rows * d // B, 2.0 * math.sqrt(B), dtype=np.float32)
    cb = np.full(256, 0.375, dtype=np.float32)
    out = oracle_attn_decode_cb(q, k, codes, norms, cb, 8, seq, 0, n_q, n_kv, d, 1 / math.sqrt(d))
    want = 0.375 * float(np.float32(2.0 * math.sqrt(B))) / math.sqrt(B)
    assert np.allclose(out, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("d,window", [(64, 0), (256, 0), (512, 0), (256, 40)])
def test_codebook_v_equals_fp16_v_with_the_same_values(d, window):
    """Levels (i - 128) / 8 and norms sqrt(B) * 2^m make each V value (i - 128) / 8 * 2^m,
    exact in fp16; the fp16-V oracle over those values must agree to rounding."""
    r = _rng(d + window)
    seq, n_q, n_kv = (1, 100, 0, 257), 8, 2
    B = min(d, 256)
    q, k = _random_qk(r, seq, n_q, n_kv, d)
    n_rows = sum(seq) * n_kv
    codes = r.integers(0, 256, n_rows * d).astype(np.uint8)
    m = r.integers(-3, 4, n_rows * d // B)       # a different power of two per block
    norms = (math.sqrt(B) * np.exp2(m)).astype(np.float32)
    cb = ((np.arange(256) - 128) / 8).astype(np.float32)
    v16 = ((np.arange(256)[codes] - 128) / 8 * np.exp2(np.repeat(m, B))).astype(np.float16)
    got = oracle_attn_decode_cb(q, k, codes, norms, cb, 8, seq, window, n_q, n_kv, d, 1 / math.sqrt(d))
    want = oracle_attn_decode(q, k, v16, None, seq, window, n_q, n_kv, d, 1 / math.sqrt(d))
    # the norm sqrt(B) * 2^m is rounded to fp32 (exact for B = 64, 256), so agreement is to ~1e-7
    assert np.allclose(got, want, rtol=2e-7, atol=1e-12)


def test_index_is_masked_to_the_codebook_bits():
    r = _rng(11)
    seq, n_q, n_kv, d = (50, 9), 4, 4, 128
    q, k = _random_qk(r, seq, n_q, n_kv, d)
    n_rows = sum(seq) * n_kv
    codes = r.integers(0, 256, n_rows * d).astype(np.uint8)
    norms = r.uniform(5, 15, n_rows * d // 128).astype(np.float32)
    cb = r.standard_normal(256).astype(np.float32)
    five = oracle_attn_decode_cb(q, k, codes, norms, cb[:32], 5, seq, 0, n_q, n_kv, d, 0.1)
    low = oracle_attn_decode_cb(q, k, codes & 31, norms, cb, 8, seq, 0, n_q, n_kv, d, 0.1)
    assert np.array_equal(five, low)
    full = oracle_attn_decode_cb(q, k, codes, norms, cb, 8, seq, 0, n_q, n_kv, d, 0.1)
    assert not np.allclose(five, full)


def test_empty_slot_gives_zeros():
    r = _rng(12)
    seq, n_q, n_kv, d = (0, 5), 2, 1, 64
    q, k = _random_qk(r, seq, n_q, n_kv, d)
    codes = r.integers(0, 256, 5 * d).astype(np.uint8)
    norms = np.ones(5, dtype=np.float32)
    out = oracle_attn_decode_cb(q, k, codes, norms, np.ones(256, np.float32), 8, seq, 0, n_q, n_kv, d, 0.1)
    assert np.array_equal(out[0], np.zeros((n_q, d)))
    assert np.all(np.abs(out[1]) > 0)


def test_invalid_arguments_are_rejected():
    q = np.zeros(64, np.float16)
    k = np.zeros(64, np.float16)
    codes = np.zeros(64, np.uint8)
    norms = np.ones(1, np.float32)
    cb = np.zeros(256, np.float32)
    with pytest.raises(ValueError):
        oracle_attn_decode_cb(q, k, codes, norms, cb, 9, (1,), 0, 1, 1, 64, 0.1)
    with pytest.raises(ValueError):
        oracle_attn_decode_cb(q, k, codes, norms, cb, 0, (1,), 0, 1, 1, 64, 0.1)
    with pytest.raises(ValueError):
        oracle_attn_decode_cb(q, k, codes, norms, cb[:16], 5, (1,), 0, 1, 1, 64, 0.1)


# ---------------------------------------------------------------- whole chain

def _chain_error(bits, d, signs_override=None):
    seq, n_q, n_kv = (700, 300), 4, 2
    ci = make_codebook_inputs(seq, n_q, n_kv, d, bits, 4242, keep_plain=True)
    rot = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), bits, seq, 0, n_q, n_kv, d, ci.scale)
    s = ci.signs.numpy() if signs_override is None else signs_override
    got = oracle_fwht_undo(rot, s)
    # fp16 V is within 2^-11 relative of the fp32 draw: far below the quantiser's error
    want = oracle_attn_decode(ci.q.numpy(), ci.k.numpy(), ci.v_plain.numpy().astype(np.float16), None, seq, 0,
                              n_q, n_kv, d, ci.scale)
    return np.linalg.norm(got - want) / np.linalg.norm(want)


@pytest.mark.parametrize("bits,d,bound", [(8, 256, 0.03), (8, 512, 0.03), (4, 256, 0.3)])
def test_encode_attend_undo_approximates_plain_attention(bits, d, bound):
    """Lloyd-Max distortion for N(0, 1) is about 2.7 * 4^-bits (Panter-Dite): rms error 0.0064
    at 8 bits, 0.10 at 4 bits, per coordinate; the attention average keeps the ratio."""
    err = _chain_error(bits, d)
    assert err < bound, err


def test_chain_fails_with_the_wrong_signs():
    d = 256
    err = _chain_error(8, d, signs_override=np.ones(d, np.float32))
    assert err > 0.5, err


# ---------------------------------------------------------------- generator levels

def test_lloyd_max_one_bit_is_mean_of_half_normal():
    c = lloyd_max_gaussian(1).numpy()
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-6)


def test_lloyd_max_two_bit_matches_the_classical_table():
    c = lloyd_max_gaussian(2).numpy()
    assert np.allclose(c, [-1.510, -0.4528, 0.4528, 1.510], rtol=0, atol=1e-3)


@pytest.mark.parametrize("bits,tol", [(3, 1e-6), (5, 2e-6), (8, 2e-4)])
def test_lloyd_max_is_a_fixed_point(bits, tol):
    """Each level is the mean of N(0, 1) on its cell (midpoints between neighbours)."""
    from scipy.stats import norm
    c = lloyd_max_gaussian(bits).numpy().astype(np.float64)
    b = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
    means = (norm.pdf(b[:-1]) - norm.pdf(b[1:])) / (norm.cdf(b[1:]) - norm.cdf(b[:-1]))
    assert np.allclose(c, means, rtol=0, atol=tol)
    assert np.allclose(c, -c[::-1], atol=1e-6)
