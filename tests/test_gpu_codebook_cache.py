"""Codebook V on the fixed-capacity cache, through the C ABI: the encode of new
rows (attn_kv_append_cb), attention over the cache (attn_decode_cache_cb) and
the whole serving loop (append, attend, undo), each against the CPU fp64 oracle.

The encode decides an integer (the level index) from floating point.  The
kernel takes that decision in fp32, the oracle in fp64, and their rotated
coordinates differ by rounding, so the code is unique only away from the
midpoints between neighbouring levels.  The check is exact wherever the
oracle's normalised coordinate u lies farther than EPS from every midpoint;
nearer than that, either neighbour is a correct result.  EPS bounds the fp32
error of u: log2(D) + 1 roundings in each rotated coordinate of a row of norm
|v|, each at most 2^-24 |v|, scaled by sqrt(B) / norm, plus the norm's own
relative error times |u| <= 4 -- under 1e-4 at D = 512 -- doubled for margin.
Norms are compared to a relative NORM_RTOL from the same bound.

The serving-loop test draws V rows whose coordinates all sit at least 4 EPS
from every midpoint, so every code is unique and the GPU cache must equal the
oracle's bit for bit, step after step.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import codebook_levels, make_cache_codebook_inputs, make_signs
from oracle import oracle_attn_decode_cache_cb, oracle_codebook_encode, oracle_fwht_undo, oracle_kv_append_cb

from gpu_util import assert_parity

pytestmark = pytest.mark.gpu

EPS = 2e-4
NORM_RTOL = 5e-5
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(f"[cb-cache] {msg}", flush=True)


def _mids(cb):
    c = np.asarray(cb, dtype=np.float64)
    return (c[1:] + c[:-1]) / 2


def check_codes(got, ref, u, cb, bits, what):
    """Exact away from the level midpoints; within EPS of one, either neighbour.
    Returns the number of coordinates where the two differ."""
    got = np.asarray(got).astype(np.int64)
    ref = np.asarray(ref).astype(np.int64)
    assert got.max(initial=0) < (1 << bits), f"{what}: code out of range"
    diff = got != ref
    n = int(diff.sum())
    if n:
        assert np.all(np.abs(got[diff] - ref[diff]) == 1), f"{what}: codes differ by more than one level"
        c = np.asarray(cb, dtype=np.float64)
        m = (c[np.minimum(got[diff], ref[diff])] + c[np.maximum(got[diff], ref[diff])]) / 2
        worst = float(np.abs(u[diff] - m).max())
        assert worst <= EPS, f"{what}: a code differs {worst:.2e} from the midpoint (bound {EPS})"
    return n


def check_norms(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    zero = ref == 0
    assert np.all(got[zero] == 0), f"{what}: zero norm"
    rel = np.abs(got[~zero] - ref[~zero]) / ref[~zero]
    assert rel.max(initial=0) <= NORM_RTOL, f"{what}: norm rel err {rel.max():.2e}"


# ---------------------------------------------------------------- append

def _rows(n_rows, n_slots, cap, ring):
    sid = [i % n_slots for i in range(n_rows)]
    pos = [(5000 if ring else 1) + 3 * (i // n_slots) for i in range(n_rows)]
    if not ring:
        assert max(pos) < cap
    return sid, pos


APPEND_CASES = [  # D, bits, ring
    (64, 5, 0), (128, 6, 1), (256, 8, 0), (512, 8, 1), (256, 4, 1), (512, 1, 0), (128, 8, 0),
]


@pytest.mark.parametrize("d,bits,ring", APPEND_CASES, ids=[f"d{c[0]}b{c[1]}r{c[2]}" for c in APPEND_CASES])
def test_codebook_append_matches_oracle(d, bits, ring):
    n_slots, n_kv, cap, n_rows = 5, 2, 48, 37
    B = min(d, 256)
    r = np.random.default_rng(9000 + d + bits + ring)
    sid, pos = _rows(n_rows, n_slots, cap, ring)
    kn = (r.standard_normal((n_rows, n_kv, d)) * 2).astype(np.float32)
    vn = (r.standard_normal((n_rows, n_kv, d)) * 3).astype(np.float32)
    vn[3, 1] = 0.0                                      # a zero row: code 0, norm 0
    s = make_signs(d, 9100 + d).numpy()
    cb = codebook_levels(bits).numpy()
    total = n_slots * n_kv * cap * d
    k0 = r.standard_normal(total).astype(np.float16)
    c0 = r.integers(0, 256, total).astype(np.uint8)
    n0 = np.full(total // B, -1.0, dtype=np.float32)
    _say(f"append D={d} bits={bits} ring={ring} rows={n_rows}")
    kc, vc, nm = (torch.from_numpy(a.copy()).to(DEV) for a in (k0, c0, n0))
    binding.attn_kv_append_cb(torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV), kc, vc, nm,
                              torch.from_numpy(s).to(DEV), torch.from_numpy(cb).to(DEV), bits, sid, pos, n_rows,
                              n_slots, cap, ring, n_kv, d)
    torch.cuda.synchronize()
    rk, rc, rn, u = oracle_kv_append_cb(kn, vn, s, cb, bits, k0, c0, n0, sid, pos, n_slots, cap, ring, n_kv, d)
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), rk.view(np.uint16)), "K"
    gc, gn = vc.cpu().numpy(), nm.cpu().numpy()
    touched = np.zeros(n_slots * n_kv * cap, dtype=bool)
    codes_g, codes_r, norms_g, norms_r, us = [], [], [], [], []
    for i in range(n_rows):
        phys = pos[i] % cap if ring else pos[i]
        for h in range(n_kv):
            row = (sid[i] * n_kv + h) * cap + phys
            touched[row] = True
            codes_g.append(gc[row * d:(row + 1) * d])
            codes_r.append(rc[row * d:(row + 1) * d])
            norms_g.append(gn[row * (d // B):(row + 1) * (d // B)])
            norms_r.append(rn[row * (d // B):(row + 1) * (d // B)])
            us.append(u[i, h])
    untouched = np.repeat(~touched, d)
    assert np.array_equal(gc[untouched], c0[untouched]), "codes of rows not appended changed"
    assert np.array_equal(gn[np.repeat(~touched, d // B)], n0[np.repeat(~touched, d // B)])
    n_diff = check_codes(np.concatenate(codes_g), np.concatenate(codes_r), np.concatenate(us), cb, bits, "codes")
    check_norms(np.concatenate(norms_g), np.concatenate(norms_r), "norms")
    n_all = n_rows * n_kv * d
    _say(f"  codes at a midpoint: {n_diff} of {n_all}")
    assert n_diff <= n_all // 100


def test_codebook_append_rejections():
    d = 64
    z = torch.zeros((1, 1, d), dtype=torch.float32, device=DEV)
    kc = torch.zeros(4 * d, dtype=torch.float16, device=DEV)
    vc = torch.zeros(4 * d, dtype=torch.uint8, device=DEV)
    nm = torch.zeros(4, dtype=torch.float32, device=DEV)
    s = torch.ones(d, dtype=torch.float32, device=DEV)
    cb = torch.zeros(512, dtype=torch.float32, device=DEV)
    with pytest.raises(binding.AttnDecodeError):
        binding.attn_kv_append_cb(z, z, kc, vc, nm, s, cb[:2], 0, [0], [0], 1, 1, 4, 0, 1, d)
    with pytest.raises(binding.AttnDecodeError):
        binding.attn_kv_append_cb(z, z, kc, vc, nm, s, cb[:4], 2, [0], [4], 1, 1, 4, 0, 1, d)   # past capacity
    two = torch.zeros((2, 1, d), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.AttnDecodeError) as ei:
        binding.attn_kv_append_cb(two, two, kc, vc, nm, s, cb[:4], 2, [0, 0], [1, 5], 2, 1, 4, 1, 1, d)
    assert "same cache row" in ei.value.message


# ---------------------------------------------------------------- attention over the cache

ATTN_CASES = [
    # n_cache_slots, capacity, ring, slot_ids, positions, n_q, n_kv, D, bits, window
    (4, 1536, 0, (0, 1, 2, 3), (1535, 200, 1000, 0), 16, 2, 256, 8, 0),
    (3, 1024, 1, (0, 1, 2, 0), (5000, 1023, 77, 5001), 32, 2, 512, 8, 0),
    (2, 700, 1, (1, 0, 1), (2000, 699, 2001), 8, 8, 128, 6, 100),
    (2, 4096, 0, (1, 1, 1, 1), (4092, 4093, 4094, 4095), 16, 8, 64, 5, 0),
    (2, 2048, 0, (0, 1), (2047, 10), 16, 2, 512, 8, 0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[f"a{i}" for i in range(len(ATTN_CASES))])
def test_cache_codebook_attention_matches_oracle(case):
    ns, cap, ring, sid, pos, nq, nkv, d, bits, W = case
    ci = make_cache_codebook_inputs(ns, cap, ring, sid, pos, nq, nkv, d, bits, seed_base=9300 + 7 * ATTN_CASES.index(case))
    _say(f"attend {case}")
    ref = oracle_attn_decode_cache_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                      ci.codebook.numpy(), bits, sid, pos, ns, cap, ring, W, nq, nkv, d, ci.scale)
    q, k, vc, vn, cb, sg = (t.to(DEV) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook, ci.signs))
    G = nq // nkv
    paths = (1, 2) if (G % 8 == 0 and d >= 128) else (1,)
    for path in (0,) + paths:
        out = torch.full((len(sid), nq, d), float("nan"), dtype=torch.float32, device=DEV)
        binding.attn_decode_cache_cb(q, k, vc, vn, cb, bits, sid, pos, len(sid), ns, cap, ring, W, out, nq, nkv,
                                     d, ci.scale, path=path)
        torch.cuda.synchronize()
        err = assert_parity(out.cpu().numpy(), ref, f"path {path}")
        _say(f"  path {path}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}")
    binding.attn_fwht_undo(out, sg, out)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle_fwht_undo(ref, ci.signs.numpy()), "undo")


# ---------------------------------------------------------------- the serving loop

def _v_away_from_midpoints(r, n, d, cb, signs, margin):
    """float32 V rows whose rotated, normalised coordinates all lie >= margin from every
    level midpoint: drawn in the rotated basis, pushed off the midpoints, rotated back."""
    B = min(d, 256)
    mids = _mids(cb)
    y = r.standard_normal((n, d))
    for _ in range(6):
        yb = y.reshape(n, d // B, B)
        nb = np.sqrt((yb ** 2).sum(-1, keepdims=True))
        u = yb * math.sqrt(B) / nb
        j = np.searchsorted(mids, u)                 # mids[j - 1] < u <= mids[j]
        lo = mids[np.clip(j - 1, 0, len(mids) - 1)]
        hi = mids[np.clip(j, 0, len(mids) - 1)]
        m = np.where(np.abs(u - lo) <= np.abs(u - hi), lo, hi)
        near = np.abs(u - m) < margin
        u = np.where(near, m + np.where(u >= m, margin, -margin), u)
        y = (u * nb / math.sqrt(B)).reshape(n, d)
    v = oracle_fwht_undo(y, signs).astype(np.float32)
    _, _, uu = oracle_codebook_encode(v, signs, cb, int(math.log2(len(cb))))
    gap = np.abs(uu[..., None] - mids).min(-1)
    assert gap.min() >= margin / 2, "inputs too near a midpoint"
    return v


@pytest.mark.parametrize("d,bits,nq,nkv", [(256, 8, 16, 2), (512, 8, 32, 2), (128, 5, 8, 8)])
def test_serving_loop_append_attend_undo(d, bits, nq, nkv):
    """A ring cache of 32 rows per slot; 40 steps, each appending one token per slot and
    attending from it, so the ring wraps.  The GPU cache stays bit-identical to the oracle's."""
    ns, cap = 3, 32
    B = min(d, 256)
    r = np.random.default_rng(9500 + d)
    s = make_signs(d, 9600 + d).numpy()
    cb = codebook_levels(bits).numpy()
    total = ns * nkv * cap * d
    k_host = np.zeros(total, np.float16)
    c_host = np.zeros(total, np.uint8)
    n_host = np.zeros(total // B, np.float32)
    kc = torch.zeros(total, dtype=torch.float16, device=DEV)
    vc = torch.zeros(total, dtype=torch.uint8, device=DEV)
    nm = torch.zeros(total // B, dtype=torch.float32, device=DEV)
    sg, cbt = torch.from_numpy(s).to(DEV), torch.from_numpy(cb).to(DEV)
    start = (0, 5, 17)          # each slot's first position
    scale = 1 / math.sqrt(d)
    worst = (0.0, 0.0)
    _say(f"loop D={d} bits={bits} G={nq // nkv}")
    for t in range(40):
        sid = [0, 1, 2]
        pos = [p + t for p in start]
        kn = r.standard_normal((ns, nkv, d)).astype(np.float32)
        vn = _v_away_from_midpoints(r, ns * nkv, d, cb, s, 4 * EPS).reshape(ns, nkv, d)
        q = r.standard_normal((ns, nq, d)).astype(np.float16)
        binding.attn_kv_append_cb(torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV), kc, vc, nm, sg, cbt,
                                  bits, sid, pos, ns, ns, cap, 1, nkv, d)
        out = torch.full((ns, nq, d), float("nan"), dtype=torch.float32, device=DEV)
        binding.attn_decode_cache_cb(torch.from_numpy(q).to(DEV), kc, vc, nm, cbt, bits, sid, pos, ns, ns, cap, 1,
                                     0, out, nq, nkv, d, scale)
        binding.attn_fwht_undo(out, sg, out)
        k_host, c_host, n_host, _ = oracle_kv_append_cb(kn, vn, s, cb, bits, k_host, c_host, n_host, sid, pos, ns,
                                                        cap, 1, nkv, d)
        ref = oracle_fwht_undo(oracle_attn_decode_cache_cb(q, k_host, c_host, n_host, cb, bits, sid, pos, ns, cap,
                                                           1, 0, nq, nkv, d, scale), s)
        torch.cuda.synchronize()
        assert np.array_equal(kc.cpu().numpy().view(np.uint16), k_host.view(np.uint16)), f"K at step {t}"
        assert np.array_equal(vc.cpu().numpy(), c_host), f"codes at step {t}"
        check_norms(nm.cpu().numpy(), n_host, f"norms at step {t}")
        err = assert_parity(out.cpu().numpy(), ref, f"step {t}")
        worst = (max(worst[0], err[0]), max(worst[1], err[1]))
    _say(f"  40 steps: worst max-abs {worst[0]:.3e} rel-L2 {worst[1]:.3e}")
