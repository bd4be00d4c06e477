"""Seeded random shapes through the C ABI against the fp64 oracle, over the whole output.

Each case draws a head_dim (64..512), query heads per kv head (1..16, odd counts included), kv
heads, a V format (fp16, int8 blocks, codebook of 5, 6 or 8 bits), a batch of slot lengths that
mixes empty, one-position, chunk-edge and long slots, a window, a merge mode and, where it
applies, a forced kernel path; a third of the cases are cache calls (fixed-capacity or ring, with
positions past the wrap).  The shapes are sized so the oracle finishes each in about a second.
Every output element is compared with the oracle; for packed calls a slot drawn at random is also
called alone and must give the same bits (the chunks of a slot depend on its own length only).
Twelve more cases draw codebook V on the fixed-capacity or ring cache (attn_decode_cache_cb).
"""
import numpy as np
import pytest
import torch

from decode_attention_kv_02_amd import binding
from decode_attention_kv_02_amd.workloads import make_cache_inputs, make_codebook_inputs, make_inputs

from gpu_util import assert_parity, run_gpu, run_gpu_cache, run_oracle, run_oracle_cache, to_device

pytestmark = pytest.mark.gpu

N_CASES = 40
LENGTHS = (0, 1, 63, 64, 65, 127, 700, 2048, 4097)
WORK_LIMIT = 4e8   # attended positions x query heads x head_dim per case


def _draw(i):
    r = np.random.default_rng(8100 + i)
    while True:
        d = int(r.choice([64, 128, 256, 512]))
        G = int(r.choice([1, 2, 3, 4, 5, 6, 8, 16]))
        nkv = int(r.choice([1, 2, 4, 8]))
        fmt = str(r.choice(["fp16", "int8", "cb"]))
        cache = r.random() < 1 / 3 and fmt != "cb"
        n = int(r.integers(1, 7))
        seq = [int(r.choice(LENGTHS)) if r.random() < 0.6 else int(r.integers(0, 9000)) for _ in range(n)]
        W = 0 if r.random() < 0.6 else int(r.integers(1, 3000))
        mm = int(r.choice([0, 1, 2]))
        paths = [0, 1] + ([2] if G % 8 == 0 and d >= 128 else [])
        path = int(r.choice(paths))
        bits = int(r.choice([5, 6, 8]))
        ring = int(r.integers(0, 2))
        if sum(seq) * G * nkv * d <= WORK_LIMIT and G * nkv <= 64:
            return dict(d=d, G=G, nkv=nkv, fmt=fmt, cache=cache, seq=seq, W=W, mm=mm, path=path,
                        bits=bits, ring=ring, seed=8100 + i)


CASES = [_draw(i) for i in range(N_CASES)]


def _id(c):
    kind = "cache" if c["cache"] else "packed"
    return f"{kind}-D{c['d']}-G{c['G']}-kv{c['nkv']}-{c['fmt']}-W{c['W']}-mm{c['mm']}-p{c['path']}"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _say(c, err):
    print(f"[random] {_id(c)} seq={c['seq']}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)


def _packed(c):
    d, G, nkv, seq, W = c["d"], c["G"], c["nkv"], c["seq"], c["W"]
    nq = G * nkv
    inp = make_inputs(seq, nq, nkv, d, c["fmt"] == "int8", seed_base=c["seed"])
    got = run_gpu(inp, W, merge_mode=c["mm"]) if c["path"] == 0 else _run_path(inp, W, c)
    _say(c, assert_parity(got.cpu().numpy(), run_oracle(inp, W), _id(c)))
    # one slot alone gives the same bits
    s = int(np.random.default_rng(c["seed"] + 1).integers(0, len(seq)))
    off = sum(seq[:s]) * nkv * d
    m = seq[s] * nkv * d
    vs = None if inp.v_scales is None else inp.v_scales[off // 32:(off + m) // 32].clone()
    alone = type(inp)(inp.q[s:s + 1].clone(), inp.k[off:off + m].clone(), inp.v[off:off + m].clone(), vs,
                      (seq[s],), nq, nkv, d, inp.scale)
    solo = run_gpu(alone, W, merge_mode=c["mm"]) if c["path"] == 0 else _run_path(alone, W, c)
    assert torch.equal(got[s:s + 1], solo), f"{_id(c)}: slot {s} alone differs from the batch"


def _run_path(inp, W, c):
    q, k, v, vs = to_device(inp)
    out = torch.full((inp.n_slots, inp.n_q_heads, inp.head_dim), float("nan"), dtype=torch.float32, device=q.device)
    binding.attn_decode_ex(q, k, v, vs, inp.seq_lens, W, out, inp.n_slots, inp.n_q_heads, inp.n_kv_heads,
                           inp.head_dim, inp.scale, merge_mode=c["mm"], path=c["path"])
    torch.cuda.synchronize()
    return out


def _codebook(c):
    from oracle import oracle_attn_decode_cb
    d, G, nkv, seq, W, bits = c["d"], c["G"], c["nkv"], c["seq"], c["W"], c["bits"]
    nq = G * nkv
    ci = make_codebook_inputs(seq, nq, nkv, d, bits, c["seed"])
    dev = torch.device("cuda:0")
    out = torch.full((len(seq), nq, d), float("nan"), dtype=torch.float32, device=dev)
    binding.attn_decode_cb(ci.q.to(dev), ci.k.to(dev), ci.v_codes.to(dev), ci.v_norms.to(dev), ci.codebook.to(dev),
                           bits, seq, W, out, len(seq), nq, nkv, d, ci.scale, merge_mode=c["mm"], path=c["path"])
    torch.cuda.synchronize()
    ref = oracle_attn_decode_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                ci.codebook.numpy(), bits, seq, W, nq, nkv, d, ci.scale)
    _say(c, assert_parity(out.cpu().numpy(), ref, _id(c)))


def _cache(c):
    d, G, nkv, W, ring = c["d"], c["G"], c["nkv"], c["W"], c["ring"]
    nq = G * nkv
    r = np.random.default_rng(c["seed"] + 2)
    cap = int(r.choice([256, 1000, 4096]))
    n_cache = int(r.integers(1, 4))
    n_queries = int(r.integers(1, 6))
    sid = tuple(int(x) for x in r.integers(0, n_cache, size=n_queries))
    hi = 3 * cap if ring else cap
    pos = tuple(int(x) for x in r.integers(0, hi, size=n_queries))
    if n_queries * min(cap, max(pos) + 1) * nq * d > WORK_LIMIT:
        pos = tuple(min(p, 2000) for p in pos)
    ci = make_cache_inputs(n_cache, cap, ring, sid, pos, nq, nkv, d, c["fmt"] == "int8", seed_base=c["seed"])
    got = run_gpu_cache(ci, W, merge_mode=c["mm"], path=c["path"])
    _say(c, assert_parity(got.cpu().numpy(), run_oracle_cache(ci, W), _id(c) + f" cap={cap} ring={ring}"))


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_matches_the_oracle(case):
    print(f"[random] start {_id(case)} seq={case['seq']}", flush=True)
    if case["fmt"] == "cb":
        _codebook(case)
    elif case["cache"]:
        _cache(case)
    else:
        _packed(case)


def _draw_cb_cache(i):
    """Codebook V on the fixed-capacity or ring cache (attn_decode_cache_cb)."""
    r = np.random.default_rng(8300 + i)
    while True:
        d = int(r.choice([64, 128, 256, 512]))
        G = int(r.choice([1, 2, 3, 4, 6, 8, 16]))
        nkv = int(r.choice([1, 2, 4, 8]))
        bits = int(r.choice([5, 6, 8]))
        cap = int(r.choice([300, 1024, 4096]))
        ring = int(r.integers(0, 2))
        n_cache = int(r.integers(1, 4))
        nqu = int(r.integers(1, 6))
        sid = tuple(int(x) for x in r.integers(0, n_cache, size=nqu))
        pos = tuple(int(x) for x in r.integers(0, 3 * cap if ring else cap, size=nqu))
        W = 0 if r.random() < 0.6 else int(r.integers(1, 3000))
        mm = int(r.choice([0, 1, 2]))
        path = int(r.choice([0, 1] + ([2] if G % 8 == 0 and d >= 128 else [])))
        if nqu * cap * G * nkv * d <= WORK_LIMIT and G * nkv <= 64:
            return dict(d=d, G=G, nkv=nkv, bits=bits, cap=cap, ring=ring, n_cache=n_cache, sid=sid, pos=pos, W=W,
                        mm=mm, path=path, seed=8300 + i)


CB_CACHE_CASES = [_draw_cb_cache(i) for i in range(12)]


def _cb_id(c):
    return (f"cbcache-D{c['d']}-G{c['G']}-kv{c['nkv']}-b{c['bits']}-cap{c['cap']}-r{c['ring']}-W{c['W']}"
            f"-mm{c['mm']}-p{c['path']}")


@pytest.mark.parametrize("case", CB_CACHE_CASES, ids=[_cb_id(c) for c in CB_CACHE_CASES])
def test_random_codebook_cache_matches_the_oracle(case):
    from decode_attention_kv_02_amd.workloads import make_cache_codebook_inputs
    from oracle import oracle_attn_decode_cache_cb
    c = case
    d, G, nkv, bits = c["d"], c["G"], c["nkv"], c["bits"]
    nq = G * nkv
    print(f"[random] start {_cb_id(c)} sid={c['sid']} pos={c['pos']}", flush=True)
    ci = make_cache_codebook_inputs(c["n_cache"], c["cap"], c["ring"], c["sid"], c["pos"], nq, nkv, d, bits,
                                    seed_base=c["seed"])
    dev = torch.device("cuda:0")
    q, k, vc, vn, cb = (t.to(dev) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook))
    out = torch.full((len(c["sid"]), nq, d), float("nan"), dtype=torch.float32, device=dev)
    binding.attn_decode_cache_cb(q, k, vc, vn, cb, bits, c["sid"], c["pos"], len(c["sid"]), c["n_cache"], c["cap"],
                                 c["ring"], c["W"], out, nq, nkv, d, ci.scale, merge_mode=c["mm"], path=c["path"])
    torch.cuda.synchronize()
    ref = oracle_attn_decode_cache_cb(ci.q.numpy(), ci.k.numpy(), ci.v_codes.numpy(), ci.v_norms.numpy(),
                                      ci.codebook.numpy(), bits, c["sid"], c["pos"], c["n_cache"], c["cap"],
                                      c["ring"], c["W"], nq, nkv, d, ci.scale)
    err = assert_parity(out.cpu().numpy(), ref, _cb_id(c))
    print(f"[random] {_cb_id(c)}: max-abs {err[0]:.3e} rel-L2 {err[1]:.3e}", flush=True)
