"""attn_kv_append (the step before decode attention) against the oracle, bit for bit.

New tokens' K become fp16 and V fp16 or block-int8 codes + fp16 scales, in
the cache row of their (slot, position); integer and byte results must be
bit-exact, so both sides make every rounding decision in fp32 with correctly
rounded divisions (scale = fp16(max|v| / 127), code = rint(v / scale)).
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import CacheInputs, make_cache_inputs
from oracle import oracle_kv_append

from gpu_util import assert_parity, run_gpu_cache, run_oracle_cache, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _new_rows(seed, n, n_kv, d, kind="normal"):
    g = torch.Generator("cpu").manual_seed(seed)
    k = torch.randn((n, n_kv, d), generator=g, dtype=torch.float32)
    v = torch.randn((n, n_kv, d), generator=g, dtype=torch.float32)
    if kind == "scaled":
        f = torch.exp2(torch.empty((n, n_kv, d // 32, 1)).uniform_(-24, 12, generator=g))
        v = (v.view(n, n_kv, d // 32, 32) * f).view(n, n_kv, d)
        k = k * 1000.0
    elif kind == "ties":
        v = torch.randint(-126, 126, (n, n_kv, d), generator=g).float() + 0.5
        v.view(n, n_kv, d // 32, 32)[..., 0] = 127.0
    return k, v


def _append_both(ci, k_new, v_new, sid, pos):
    dev = torch.device("cuda:0")
    kc, vc, sc = to_device(ci)[1:]
    binding.attn_kv_append(k_new.to(dev), v_new.to(dev), kc, vc, sc, sid, pos, len(sid), ci.n_cache_slots,
                           ci.capacity, ci.ring, ci.n_kv_heads, ci.head_dim)
    torch.cuda.synchronize()
    rk, rv, rs = oracle_kv_append(k_new.numpy(), v_new.numpy(), ci.k.numpy(), ci.v.numpy(),
                                  None if ci.v_scales is None else ci.v_scales.numpy(), sid, pos,
                                  ci.n_cache_slots, ci.capacity, ci.ring, ci.n_kv_heads, ci.head_dim)
    return (kc, vc, sc), (rk, rv, rs)


CASES = [
    # n_cache_slots, capacity, ring, D, v_int8, kind, slot_ids, positions
    (3, 64, 0, 64, True, "normal", (0, 2, 1), (0, 63, 17)),
    (2, 128, 1, 128, True, "scaled", (1, 0, 1), (129, 5, 500)),
    (4, 256, 0, 256, True, "ties", (3, 2, 1, 0), (1, 2, 3, 255)),
    (2, 64, 1, 512, True, "scaled", (0, 1), (1000, 64)),
    (2, 100, 0, 256, False, "scaled", (1, 0), (99, 0)),
    (2, 16, 1, 64, False, "normal", (0, 1), (33, 15)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"a{i}" for i in range(len(CASES))])
def test_append_is_bit_exact(case):
    nc, cap, ring, d, i8, kind, sid, pos = case
    n_kv = 2
    ci = make_cache_inputs(nc, cap, ring, (0,), (0,), 2, n_kv, d, i8, seed_base=9700 + CASES.index(case))
    k_new, v_new = _new_rows(97 + CASES.index(case), len(sid), n_kv, d, kind)
    (kc, vc, sc), (rk, rv, rs) = _append_both(ci, k_new, v_new, sid, pos)
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), rk.view(np.uint16))
    if i8:
        assert np.array_equal(vc.cpu().numpy(), rv)
        assert np.array_equal(sc.cpu().numpy().view(np.uint16), rs.view(np.uint16))
    else:
        assert np.array_equal(vc.cpu().numpy().view(np.uint16), rv.view(np.uint16))


def test_append_many_rows_spans_several_launches():
    n_slots, cap, n_kv, d = 4, 512, 8, 256
    sid = tuple(s for s in range(n_slots) for _ in range(150))
    pos = tuple(p for _ in range(n_slots) for p in range(200, 350))
    ci = make_cache_inputs(n_slots, cap, 0, (0,), (0,), 2, n_kv, d, True, seed_base=9800)
    k_new, v_new = _new_rows(98, len(sid), n_kv, d)
    (kc, vc, sc), (rk, rv, rs) = _append_both(ci, k_new, v_new, sid, pos)
    assert np.array_equal(kc.cpu().numpy().view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(vc.cpu().numpy(), rv)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), rs.view(np.uint16))


@pytest.mark.parametrize("ring", [0, 1])
def test_append_then_attend_is_one_decode_step(ring):
    # tokens at positions p are appended, then each slot's query at p attends up to p
    n_slots, cap, n_kv, nq, d = 3, 1024, 8, 16, 256
    pos = (1023, 400, 7) if not ring else (5000, 1023, 1024)
    sid = (0, 1, 2)
    ci = make_cache_inputs(n_slots, cap, ring, sid, pos, nq, n_kv, d, True, seed_base=9900 + ring)
    k_new, v_new = _new_rows(99, 3, n_kv, d)
    (kc, vc, sc), (rk, rv, rs) = _append_both(ci, k_new, v_new, sid, pos)
    after = CacheInputs(ci.q, torch.from_numpy(rk), torch.from_numpy(rv), torch.from_numpy(rs), sid, pos,
                        n_slots, cap, ring, nq, n_kv, d, ci.scale)
    got = run_gpu_cache(after, 0, dev_tensors=(ci.q.to(kc.device), kc, vc, sc)).cpu().numpy()
    ref = run_oracle_cache(after, 0)
    assert_parity(got, ref, "append then attend")


def test_append_rejects_collisions():
    ci = make_cache_inputs(2, 16, 1, (0,), (0,), 2, 1, 64, False, seed_base=9950)
    dev = torch.device("cuda:0")
    kc, vc, _ = to_device(ci)[1:]
    k_new = torch.zeros((2, 1, 64), dtype=torch.float32, device=dev)
    with pytest.raises(binding.AttnDecodeError):
        binding.attn_kv_append(k_new, k_new, kc, vc, None, (1, 1), (3, 19), 2, 2, 16, 1, 1, 64)
