"""V magnitudes across the range the ABI documents, on the matrix-core kernel (which carries
int8 values, codebook levels and norm-scaled weights as exact pairs of fp16 values) and on the
lane kernel (fp32), against the CPU fp64 oracle.

The stated tolerance (max-abs 2e-3, relative-L2 1e-3) is for N(0, 1)-scale data.  For V scaled
up by a factor F the same relative accuracy is max-abs 2e-3 F, and that is the bound used there;
relative-L2 1e-3 holds at every scale, the small ones included.
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_codebook_inputs, make_inputs
from oracle import oracle_attn_decode_cb

from gpu_util import errors, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _check(got, ref, factor, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    print(f"[ranges] {what}: max |ref| {np.abs(ref).max():.3e}, max-abs {max_abs:.3e}, rel-L2 {rel:.3e}",
          flush=True)
    assert max_abs <= 2e-3 * max(factor, 1.0) and rel <= 1e-3, f"{what}: max-abs {max_abs:.3e}, rel-L2 {rel:.3e}"


# int8 V: scales multiplied by the factor.  N(0, 1) sources give scales of about 0.03 and codes up
# to 127, so 1.2e4 puts |code * scale| near 5e4, close to fp16's 65504; 1e-3 puts scales among
# fp16's subnormals.
@pytest.mark.parametrize("d,factor", [(256, 1.2e4), (512, 1.2e4), (256, 1e-3), (128, 300.0)])
def test_int8_v_magnitudes(d, factor):
    seq = (1500, 700)
    inp = make_inputs(seq, 16, 2, d, True, seed_base=8800 + d)
    inp.v_scales.copy_((inp.v_scales.float() * factor).half())
    assert torch.isfinite(inp.v_scales.float()).all()
    vmax = (inp.v.float().abs().reshape(-1, 32) * inp.v_scales.float().reshape(-1, 1)).max().item()
    assert vmax <= 65504.0, vmax
    ref = run_oracle(inp, 0)
    dev = to_device(inp)
    for path in (2, 1):
        out = torch.full((len(seq), 16, d), float("nan"), dtype=torch.float32, device=DEV)
        q, k, v, vs = dev
        binding.attn_decode_ex(q, k, v, vs, inp.seq_lens, 0, out, len(seq), 16, 2, d, inp.scale, path=path)
        torch.cuda.synchronize()
        _check(out.cpu().numpy(), ref, factor, f"int8 D={d} x{factor:g} path {path} (|v| <= {vmax:.3g})")


# codebook V: block norms multiplied by the factor.  N(0, 1) rows have norms near sqrt(B) = 16 at
# B = 256, so 500 gives about 8000 (the documented bound is 16376), 0.1 about 1.6 and 1e-3 about
# 0.016, where the weights of the less likely keys lose relative precision gradually.
@pytest.mark.parametrize("d,factor", [(256, 500.0), (512, 500.0), (256, 0.1), (256, 1e-3), (128, 1e-3)])
def test_codebook_v_magnitudes(d, factor):
    seq = (1500, 700)
    ci = make_codebook_inputs(seq, 16, 2, d, 8, 8900 + d)
    ci.v_norms.mul_(factor)
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), 8, seq, 0, 16, 2, d, ci.scale)
    q, k, vc, vn, cb = (t.to(DEV) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook))
    for path in (2, 1):
        out = torch.full((len(seq), 16, d), float("nan"), dtype=torch.float32, device=DEV)
        binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq, 0, out, len(seq), 16, 2, d, ci.scale, path=path)
        torch.cuda.synchronize()
        _check(out.cpu().numpy(), ref, factor, f"codebook D={d} x{factor:g} path {path}")
