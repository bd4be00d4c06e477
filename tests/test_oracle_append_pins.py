"""Pins of the oracle's KV-append pieces: float32 -> fp16 rounding, the
block-int8 quantiser, and the append itself.

* fp16 rounding is checked against numpy's float32 -> float16 conversion
  (round to nearest even) on every fp16 value, the exact midpoints between
  neighbours (ties) and one float32 ulp either side, and random floats over
  the whole range.
* The quantiser is checked bit for bit against the independent torch
  implementation used to generate the int8 workloads
  (decode_attention_kv_02_amd.workloads.quantize_int8_blocks): same
  definition, scale = fp16(max|v| / 127), code = round-half-even(v / scale).
* The append is checked by placement: rows land at position p (linear) or
  p mod capacity (ring) of their slot, nothing else changes, and colliding
  rows are rejected.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd.workloads import quantize_int8_blocks
from oracle import float_to_half_bits, oracle_kv_append, quantize_blocks


def _np_half_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def test_float_to_half_on_every_half_and_every_tie():
    halves = np.arange(0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16)  # finite, >= 0
    h32 = halves.astype(np.float32)
    nxt = np.append(halves[1:].astype(np.float32), np.float32(65520.0))  # rounding boundary to inf
    mid = ((h32.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    cand = np.concatenate([h32, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)),
                           -h32, -mid, np.float32([np.inf, -np.inf, 1e30, -1e30, 0.0, -0.0])])
    want = _np_half_bits(cand)
    got = np.array([float_to_half_bits(x) for x in cand], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(cand[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_float_to_half_on_random_floats():
    r = np.random.default_rng(1)
    x = (r.standard_normal(20000) * np.exp2(r.uniform(-30, 18, 20000))).astype(np.float32)
    got = np.array([float_to_half_bits(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, _np_half_bits(x))


def _torch_quant(v):
    codes, sc = quantize_int8_blocks(torch.from_numpy(np.asarray(v, dtype=np.float32)))
    return codes.numpy().reshape(-1), sc.numpy().reshape(-1)


@pytest.mark.parametrize("kind", ["normal", "tiny", "large", "ties", "zeros", "mixed"])
def test_quantiser_matches_the_independent_torch_quantiser(kind):
    r = np.random.default_rng(hash(kind) % 2**32)
    n = 32 * 512
    if kind == "normal":
        v = r.standard_normal(n)
    elif kind == "tiny":
        v = r.standard_normal(n) * 1e-6          # fp16 subnormal scales
    elif kind == "large":
        v = r.standard_normal(n) * 3e4
    elif kind == "ties":
        # amax = 127 gives scale 1 exactly, so v = k + 0.5 is an exact tie
        v = r.integers(-126, 126, n) + 0.5
        v.reshape(-1, 32)[:, 0] = 127.0
    elif kind == "zeros":
        v = np.zeros(n)
        v[32 * 7 + 3] = 0.25
    else:
        v = r.standard_normal(n) * np.repeat(np.exp2(r.uniform(-20, 10, n // 32)), 32)
    v = v.astype(np.float32).reshape(-1, 32)
    codes, scales = quantize_blocks(v)
    tc, ts = _torch_quant(v)
    assert np.array_equal(codes, tc)
    assert np.array_equal(scales.view(np.uint16), ts.view(np.uint16))


def test_quantiser_closed_form():
    # a block with max 127 has scale 1 and codes equal to round-half-even(v)
    v = np.array([127.0, -127.0, 2.5, 3.5, -2.5, 0.49, -0.5, 1.5] + [0.0] * 24, dtype=np.float32)
    codes, scales = quantize_blocks(v)
    assert float(scales[0]) == 1.0
    assert list(codes[:8]) == [127, -127, 2, 4, -2, 0, 0, 2]


@pytest.mark.parametrize("ring", [0, 1])
@pytest.mark.parametrize("v_int8", [False, True])
def test_append_places_rows_and_touches_nothing_else(ring, v_int8):
    n_slots, n_kv, cap, d = 3, 2, 16, 64
    r = np.random.default_rng(7)
    k = r.standard_normal((n_slots, n_kv, cap, d)).astype(np.float16)
    if v_int8:
        v = r.integers(-127, 128, (n_slots, n_kv, cap, d)).astype(np.int8)
        vs = r.uniform(0.01, 0.1, (n_slots, n_kv, cap, d // 32)).astype(np.float16)
    else:
        v = r.standard_normal((n_slots, n_kv, cap, d)).astype(np.float16)
        vs = None
    sid = [2, 0, 2]
    pos = [5, 15, 40] if ring else [5, 15, 9]
    kn = r.standard_normal((3, n_kv, d)).astype(np.float32)
    vn = r.standard_normal((3, n_kv, d)).astype(np.float32)
    kc, vc, sc = oracle_kv_append(kn, vn, k, v, vs, sid, pos, n_slots, cap, ring, n_kv, d)
    kc = kc.reshape(k.shape)
    vc = vc.reshape(v.shape)
    touched = set()
    for i in range(3):
        row = pos[i] % cap if ring else pos[i]
        touched.add((sid[i], row))
        assert np.array_equal(kc[sid[i], :, row], kn[i].astype(np.float16))
        if v_int8:
            codes, scales = quantize_blocks(vn[i])
            assert np.array_equal(vc[sid[i], :, row].reshape(-1), codes)
            assert np.array_equal(sc.reshape(vs.shape)[sid[i], :, row].reshape(-1).view(np.uint16),
                                  scales.view(np.uint16))
        else:
            assert np.array_equal(vc[sid[i], :, row], vn[i].astype(np.float16))
    for s in range(n_slots):
        for row in range(cap):
            if (s, row) not in touched:
                assert np.array_equal(kc[s, :, row], k[s, :, row])
                assert np.array_equal(vc[s, :, row], v[s, :, row])


@pytest.mark.parametrize("sid,pos,ring", [
    ([0, 0], [3, 3], 0),       # same row twice
    ([1, 1], [3, 19], 1),      # ring: 19 mod 16 == 3
    ([0], [16], 0),            # linear cache full
    ([2], [0], 0),             # slot out of range
])
def test_append_rejects_collisions_and_out_of_range(sid, pos, ring):
    k = np.zeros((2, 1, 16, 64), dtype=np.float16)
    kn = np.zeros((len(sid), 1, 64), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_kv_append(kn, kn, k, k, None, sid, pos, 2, 16, ring, 1, 64)
