"""Helpers shared by the GPU tests: run the HIP path on seeded inputs and compare
with the oracle to the acceptance bar (max-abs <= 2e-3, relative L2 <= 1e-3
over the whole output, fp32 outputs against the fp64 oracle)."""
import numpy as np
import torch

from decode_attention_kv_02_amd import binding
from oracle import oracle_attn_decode, oracle_attn_decode_cache

MAX_ABS = 2e-3
REL_L2 = 1e-3


def to_device(inp, dev="cuda:0"):
    d = torch.device(dev)
    return (inp.q.to(d), inp.k.to(d), inp.v.to(d),
            None if inp.v_scales is None else inp.v_scales.to(d))


def run_gpu(inp, window, chunk=0, dev_tensors=None, stream=None, poison=True, merge_mode=0):
    q, k, v, vs = dev_tensors if dev_tensors is not None else to_device(inp)
    out = torch.empty((inp.n_slots, inp.n_q_heads, inp.head_dim), dtype=torch.float32, device=q.device)
    if poison:
        out.fill_(float("nan"))
    binding.attn_decode_ex(q, k, v, vs, inp.seq_lens, window, out, inp.n_slots, inp.n_q_heads,
                           inp.n_kv_heads, inp.head_dim, inp.scale, stream=stream, chunk=chunk,
                           merge_mode=merge_mode)
    torch.cuda.synchronize()
    return out


def run_oracle(inp, window, rows=None):
    return oracle_attn_decode(
        inp.q.numpy(), inp.k.numpy(), inp.v.numpy(),
        None if inp.v_scales is None else inp.v_scales.numpy(),
        inp.seq_lens, window, inp.n_q_heads, inp.n_kv_heads, inp.head_dim, inp.scale, rows=rows)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else 0.0
    return max_abs, rel


def assert_parity(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    max_abs, rel = errors(got, ref)
    if ref.size and np.linalg.norm(ref) == 0:
        assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs:.3e}"
    else:
        assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max-abs {max_abs:.3e}, rel-L2 {rel:.3e}"
    return max_abs, rel


def run_gpu_cache(ci, window, chunk=0, dev_tensors=None, merge_mode=0, path=0):
    q, k, v, vs = dev_tensors if dev_tensors is not None else to_device(ci)
    out = torch.full((ci.n_queries, ci.n_q_heads, ci.head_dim), float("nan"), dtype=torch.float32,
                     device=q.device)
    binding.attn_decode_cache(q, k, v, vs, ci.slot_ids, ci.positions, ci.n_queries, ci.n_cache_slots,
                              ci.capacity, ci.ring, window, out, ci.n_q_heads, ci.n_kv_heads,
                              ci.head_dim, ci.scale, chunk=chunk, merge_mode=merge_mode, path=path)
    torch.cuda.synchronize()
    return out


def run_oracle_cache(ci, window, rows=None):
    return oracle_attn_decode_cache(
        ci.q.numpy(), ci.k.numpy(), ci.v.numpy(),
        None if ci.v_scales is None else ci.v_scales.numpy(),
        ci.slot_ids, ci.positions, ci.n_cache_slots, ci.capacity, ci.ring, window,
        ci.n_q_heads, ci.n_kv_heads, ci.head_dim, ci.scale, rows=rows)
