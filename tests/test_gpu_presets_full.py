"""Bench presets at their full sizes, in the launch configuration bench.py times, checked over
their whole output tensors against the CPU fp64 oracle (every row, on all host cores):

* the D = 512 global layer with 8-bit codebook V (16 q / 2 kv heads, 8 x 32768): the
  matrix-core kernel, plus the undo of the rotation;
* speculative verify (4 slots x 4 drafts over a 32768-row cache): matrix-core draft groups;
* the codebook serving steps (append each slot's token, attend, undo) over 8 x 32768 and on
  8 rings of 1024 rows;
* the KV appends (one decode step for 8 slots; 4096 tokens into one slot), bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import (APPEND_WORKLOADS, CACHE_WORKLOADS, CODEBOOK_WORKLOADS,
                                                   SERVE_STEP_WORKLOADS, append_new_rows, cache_workload_inputs,
                                                   codebook_workload_inputs, serve_step_inputs)
from oracle import (oracle_attn_decode_cache, oracle_attn_decode_cache_cb, oracle_attn_decode_cb,
                    oracle_fwht_undo, oracle_kv_append, oracle_kv_append_cb)

from gpu_util import assert_parity

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(f"[presets] {msg}", flush=True)


def test_global_d512_codebook_preset_full_output():
    cfg = next(c for c in CODEBOOK_WORKLOADS if c.head_dim == 512)
    ci = codebook_workload_inputs(cfg)
    _say(f"{cfg.name}: generated")
    q, k, vc, vn, cb, sg = (t.to(DEV) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook, ci.signs))
    out = torch.full((ci.n_slots, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    binding.attn_decode_cb(q, k, vc, vn, cb, ci.codebook_bits, ci.seq_lens, cfg.window, out, ci.n_slots,
                           ci.n_q_heads, ci.n_kv_heads, ci.head_dim, ci.scale)
    rot = out.clone()
    binding.attn_fwht_undo(out, sg, out)
    torch.cuda.synchronize()
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), ci.codebook_bits, ci.seq_lens, cfg.window, ci.n_q_heads,
                                ci.n_kv_heads, ci.head_dim, ci.scale).reshape(-1, ci.head_dim)
    got_rot = rot.cpu().numpy().reshape(-1, ci.head_dim)
    assert got_rot.shape == ref.shape == (ci.n_slots * ci.n_q_heads, ci.head_dim)
    err = assert_parity(got_rot, ref, "rotated basis")
    _say(f"{cfg.name}: rotated max-abs {err[0]:.3e} rel-L2 {err[1]:.3e} (all {ref.shape[0]} rows)")
    got = out.cpu().numpy().reshape(-1, ci.head_dim)
    err = assert_parity(got, oracle_fwht_undo(ref, ci.signs.numpy()), "undone")
    _say(f"{cfg.name}: undone max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}")


@pytest.mark.parametrize("prefix", ["verify", "batch128"])
def test_cache_preset_full_output(prefix):
    """The speculative-verify preset and the 128-slot serving batch (one launch on the large query
    table and the single-buffer lane kernel), every output row against the oracle."""
    cfg = next(c for c in CACHE_WORKLOADS if c.name.startswith(prefix))
    ci = cache_workload_inputs(cfg)
    _say(f"{cfg.name}: generated")
    q, k, v = ci.q.to(DEV), ci.k.to(DEV), ci.v.to(DEV)
    vs = None if ci.v_scales is None else ci.v_scales.to(DEV)
    out = torch.full((ci.n_queries, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    binding.attn_decode_cache(q, k, v, vs, ci.slot_ids, ci.positions, ci.n_queries, ci.n_cache_slots, ci.capacity,
                              ci.ring, cfg.window, out, ci.n_q_heads, ci.n_kv_heads, ci.head_dim, ci.scale)
    torch.cuda.synchronize()
    ref = oracle_attn_decode_cache(ci.q.numpy(), ci.k.numpy(), ci.v.numpy(),
                                   None if ci.v_scales is None else ci.v_scales.numpy(), ci.slot_ids, ci.positions,
                                   ci.n_cache_slots, ci.capacity, ci.ring, cfg.window, ci.n_q_heads, ci.n_kv_heads,
                                   ci.head_dim, ci.scale)
    got = out.cpu().numpy()
    assert got.shape == ref.shape
    err = assert_parity(got, ref, cfg.name)
    _say(f"{cfg.name}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e} (all {ci.n_queries * ci.n_q_heads} rows)")


@pytest.mark.parametrize("cfg", SERVE_STEP_WORKLOADS, ids=[c.name for c in SERVE_STEP_WORKLOADS])
def test_serving_step_preset_full_output(cfg):
    """Append (fp16 K, codebook V) then attend and undo, on the bench's serving-step presets.  The
    codes the GPU writes are checked against the oracle's fp64 decision (a code may differ only
    where the normalised coordinate lies within 2e-4 of a level midpoint); the outputs, which weigh
    the new token like any other, against the oracle over the oracle's own cache."""
    ci, kn, vn = serve_step_inputs(cfg)
    _say(f"{cfg.name}: generated")
    B = min(ci.head_dim, 256)
    k_d, vc_d, nm_d = ci.k.to(DEV), ci.v_codes.to(DEV), ci.v_norms.to(DEV)
    q, cb, sg = ci.q.to(DEV), ci.codebook.to(DEV), ci.signs.to(DEV)
    out = torch.full((ci.n_queries, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    binding.attn_kv_append_cb(kn.to(DEV), vn.to(DEV), k_d, vc_d, nm_d, sg, cb, ci.codebook_bits, ci.slot_ids,
                              ci.positions, ci.n_queries, ci.n_cache_slots, ci.capacity, ci.ring, ci.n_kv_heads,
                              ci.head_dim)
    binding.attn_decode_cache_cb(q, k_d, vc_d, nm_d, cb, ci.codebook_bits, ci.slot_ids, ci.positions, ci.n_queries,
                                 ci.n_cache_slots, ci.capacity, ci.ring, 0, out, ci.n_q_heads, ci.n_kv_heads,
                                 ci.head_dim, ci.scale)
    binding.attn_fwht_undo(out, sg, out)
    torch.cuda.synchronize()
    k_h, c_h, n_h, u = oracle_kv_append_cb(kn.numpy(), vn.numpy(), ci.signs.numpy(), ci.codebook.numpy(),
                                           ci.codebook_bits, ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                           ci.slot_ids, ci.positions, ci.n_cache_slots, ci.capacity, ci.ring,
                                           ci.n_kv_heads, ci.head_dim)
    # the appended rows: K exact, codes by the midpoint rule, norms to 5e-5
    cap, d = ci.capacity, ci.head_dim
    gk, gc, gn = k_d.cpu().numpy(), vc_d.cpu().numpy(), nm_d.cpu().numpy()
    cbd = ci.codebook.numpy().astype(np.float64)
    n_diff = 0
    for i, (s, p) in enumerate(zip(ci.slot_ids, ci.positions)):
        for h in range(ci.n_kv_heads):
            row = (s * ci.n_kv_heads + h) * cap + (p % cap if ci.ring else p)
            sl = slice(row * d, (row + 1) * d)
            assert np.array_equal(gk[sl].view(np.uint16), k_h[sl].view(np.uint16))
            g_codes, r_codes = gc[sl].astype(np.int64), c_h[sl].astype(np.int64)
            diff = g_codes != r_codes
            if diff.any():
                assert np.all(np.abs(g_codes[diff] - r_codes[diff]) == 1)
                mid = (cbd[np.minimum(g_codes[diff], r_codes[diff])] + cbd[np.maximum(g_codes[diff], r_codes[diff])]) / 2
                assert np.abs(u[i, h][diff] - mid).max() <= 2e-4
                n_diff += int(diff.sum())
            nsl = slice(row * (d // B), (row + 1) * (d // B))
            assert np.allclose(gn[nsl], n_h[nsl], rtol=5e-5, atol=0)
    ref = oracle_fwht_undo(oracle_attn_decode_cache_cb(ci.q.numpy(), k_h, c_h, n_h, ci.codebook.numpy(),
                                                       ci.codebook_bits, ci.slot_ids, ci.positions,
                                                       ci.n_cache_slots, cap, ci.ring, 0, ci.n_q_heads,
                                                       ci.n_kv_heads, d, ci.scale).reshape(-1, d),
                           ci.signs.numpy())
    got = out.cpu().numpy().reshape(-1, d)
    assert got.shape == ref.shape == (ci.n_queries * ci.n_q_heads, d)
    err = assert_parity(got, ref, cfg.name)
    _say(f"{cfg.name}: codes at a midpoint {n_diff}; max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}")


@pytest.mark.parametrize("cfg", APPEND_WORKLOADS, ids=[c.name for c in APPEND_WORKLOADS])
def test_append_preset_bit_exact(cfg):
    d = cfg.head_dim
    el = cfg.n_cache_slots * cfg.n_kv_heads * cfg.capacity * d
    kc = torch.zeros(el, dtype=torch.float16, device=DEV)
    vc = torch.zeros(el, dtype=torch.int8 if cfg.v_int8 else torch.float16, device=DEV)
    sc = torch.zeros(el // 32, dtype=torch.float16, device=DEV) if cfg.v_int8 else None
    kn, vn = append_new_rows(cfg)
    binding.attn_kv_append(kn.to(DEV), vn.to(DEV), kc, vc, sc, cfg.slot_ids, cfg.positions, cfg.n_rows,
                           cfg.n_cache_slots, cfg.capacity, cfg.ring, cfg.n_kv_heads, d)
    torch.cuda.synchronize()
    rk, rv, rs = oracle_kv_append(kn.numpy(), vn.numpy(), np.zeros(el, np.float16),
                                  np.zeros(el, np.int8 if cfg.v_int8 else np.float16),
                                  np.zeros(el // 32, np.float16) if cfg.v_int8 else None, cfg.slot_ids,
                                  cfg.positions, cfg.n_cache_slots, cfg.capacity, cfg.ring, cfg.n_kv_heads, d)
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), rk.view(np.uint16)), "K"
    if cfg.v_int8:
        assert np.array_equal(vc.cpu().numpy(), rv), "V codes"
        assert np.array_equal(sc.cpu().numpy().view(np.uint16), rs.view(np.uint16)), "V scales"
    else:
        assert np.array_equal(vc.cpu().numpy().view(np.uint16), rv.view(np.uint16)), "V"
    _say(f"{cfg.name}: bit-exact")
