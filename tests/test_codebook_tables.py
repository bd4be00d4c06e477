"""Pins of the codebook levels the codebook-V inputs use.

The pages' hybrid V indexes three fixed tables of N(0, 1) levels, 32, 64 and
256 entries (mlx-native 0.21.1 flash_attn_vec_hybrid.metal: CODEBOOK_HB_5BIT,
CODEBOOK_HB_6BIT and CODEBOOK_HB_8BIT, read by dequant_hb_single and
dequant_hb_float4).  tests/golden/codebook_hb_tables.json holds them as the
page prints them; the input generator carries its own transcription
(workloads.PAGE_CODEBOOKS), and every codebook preset and test at 5, 6 and 8
bits takes its levels from there.

* The generator's tables equal the golden transcription in float32, level by
  level (a misread digit, a dropped or swapped level fails).
* The presets and generators hand out exactly those tables.
* What the page states about them holds: strictly increasing (the encoder's
  nearest-level search needs it), symmetric about 0, the 8-bit range
  +-5.0652659.
* As quantisers of N(0, 1) they are close to Lloyd-Max: the 5-bit table is a
  fixed point of Lloyd's map, and every table's mean-square error lies within
  1% of a 2000-step Lloyd iteration (lloyd_max_gaussian) and well below a uniform
  quantiser's over the same range.
"""
import json
import os

import numpy as np
import pytest
from scipy.stats import norm

from decode_attention_kv_02_amd.workloads import (CODEBOOK_WORKLOADS, PAGE_CODEBOOKS, codebook_levels,
                                                   codebook_workload_inputs, lloyd_max_gaussian,
                                                   make_cache_codebook_inputs, make_codebook_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codebook_hb_tables.json")


def _golden():
    with open(GOLDEN) as fh:
        d = json.load(fh)
    return {int(b): np.array([float(x) for x in v], dtype=np.float32) for b, v in d["tables"].items()}


def _mse(c):
    """E[(X - q(X))^2] for X ~ N(0, 1) and the nearest-level quantiser with levels c (exact)."""
    c = np.asarray(c, dtype=np.float64)
    b = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
    lo, hi = b[:-1], b[1:]
    p = norm.cdf(hi) - norm.cdf(lo)
    m1 = norm.pdf(lo) - norm.pdf(hi)                      # int x phi
    xphi = lambda x: np.where(np.isfinite(x), x * norm.pdf(np.where(np.isfinite(x), x, 0.0)), 0.0)
    m2 = p + xphi(lo) - xphi(hi)                          # int x^2 phi
    return float(np.sum(m2 - 2 * c * m1 + c * c * p))


def test_golden_holds_the_three_printed_tables():
    g = _golden()
    assert sorted(g) == [5, 6, 8]
    for bits, c in g.items():
        assert c.shape == (1 << bits,)


@pytest.mark.parametrize("bits", [5, 6, 8])
def test_generator_tables_equal_the_golden_transcription(bits):
    want = _golden()[bits]
    got = np.array(PAGE_CODEBOOKS[bits], dtype=np.float32)
    assert got.shape == want.shape
    assert np.abs(got.astype(np.float64) - want.astype(np.float64)).max() <= 1e-7
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits", [5, 6, 8])
def test_inputs_use_the_printed_tables(bits):
    want = _golden()[bits]
    assert np.array_equal(codebook_levels(bits).numpy(), want)
    ci = make_codebook_inputs((5, 3), 4, 2, 64, bits, 11)
    assert np.array_equal(ci.codebook.numpy(), want)
    cc = make_cache_codebook_inputs(2, 8, 0, (0, 1), (3, 7), 4, 2, 64, bits, 12)
    assert np.array_equal(cc.codebook.numpy(), want)


def test_codebook_presets_use_the_8bit_table():
    want = _golden()[8]
    for cfg in CODEBOOK_WORKLOADS:
        assert cfg.bits == 8
    # the preset's levels without drawing its full cache
    assert np.array_equal(codebook_levels(CODEBOOK_WORKLOADS[0].bits).numpy(), want)
    assert callable(codebook_workload_inputs)


def test_other_widths_use_the_lloyd_iteration():
    assert np.array_equal(codebook_levels(4).numpy(), lloyd_max_gaussian(4).numpy())


@pytest.mark.parametrize("bits", [5, 6, 8])
def test_printed_tables_increase_and_are_symmetric(bits):
    c = _golden()[bits]
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])


def test_eight_bit_range():
    c = _golden()[8]
    assert c[0] == np.float32(-5.0652659) and c[-1] == np.float32(5.0652659)


def test_five_bit_table_is_a_lloyd_fixed_point():
    c = _golden()[5].astype(np.float64)
    b = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
    means = (norm.pdf(b[:-1]) - norm.pdf(b[1:])) / (norm.cdf(b[1:]) - norm.cdf(b[:-1]))
    assert np.abs(c - means).max() < 2e-5


@pytest.mark.parametrize("bits", [5, 6, 8])
def test_printed_tables_quantise_nearly_as_well_as_lloyd_max(bits):
    n = 1 << bits
    page = _mse(_golden()[bits])
    ours = _mse(lloyd_max_gaussian(bits).numpy())
    assert abs(page - ours) <= 0.01 * ours, (page, ours)
    # and far better than a uniform quantiser over the same range
    u = np.linspace(_golden()[bits][0], _golden()[bits][-1], n)
    assert page < 0.8 * _mse(u)
