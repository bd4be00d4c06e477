"""ctypes front end of the C fp64 oracle (test infrastructure only).

``oracle_attn_decode`` computes, for each (slot, query head) row, the plain
softmax attention of one fp16 query over that slot's packed KV cache:

    out[s, h, :] = sum_j softmax_j(scale * q[s,h,:] . K[s,kvh,j,:]) * V[s,kvh,j,:]

with ``kvh = h // (n_q // n_kv)`` and ``j`` over the last ``window`` positions
(all positions when ``window`` is 0 or at least ``L_s``).  See the C source
for the citations of each step on the pages (mlx-native
flash_attn_vec_hybrid.metal; tessl nn.rs, flash_attn_decode).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_decode_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_attn_decode.so")

_lock = threading.Lock()
_lib = None


def oracle_library_path() -> str:
    return _LIB


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double: no fast-math, no contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        _SRC, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_oracle()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_attn_decode_cb_f64.restype = ctypes.c_int
        lib.oracle_attn_decode_cb_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int32]
        lib.oracle_fwht_undo_f64.restype = ctypes.c_int
        lib.oracle_fwht_undo_f64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int32]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_quantize_blocks.restype = None
        lib.oracle_quantize_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_kv_append.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.oracle_attn_decode_cache_f64.restype = ctypes.c_int
        lib.oracle_attn_decode_cache_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
        ]
        lib.oracle_codebook_encode_f64.restype = ctypes.c_int
        lib.oracle_codebook_encode_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_kv_append_cb.restype = ctypes.c_int
        lib.oracle_kv_append_cb.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_void_p]
        lib.oracle_attn_decode_cache_cb_f64.restype = ctypes.c_int
        lib.oracle_attn_decode_cache_cb_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int32]
        lib.oracle_attn_decode_f64.restype = ctypes.c_int
        lib.oracle_attn_decode_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
        ]
        _lib = lib
        return lib


def half_to_double(bits: int) -> float:
    """The oracle's own fp16 bit-pattern decoder (exposed so it can be pinned)."""
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def _as_c(arr: np.ndarray, dtype) -> np.ndarray:
    arr = np.asarray(arr)
    if arr.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {arr.dtype}")
    return np.ascontiguousarray(arr)


def _ptr(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def oracle_attn_decode(q, k, v, v_scales, seq_lens, window, n_q, n_kv, head_dim,
                       scale, rows=None, threads=None) -> np.ndarray:
    """Plain fp64 decode attention.

    q: float16 [n_slots, n_q, D]; k: float16 packed [sum_s n_kv*L_s*D];
    v: float16 (``v_scales is None``) or int8, same layout as k;
    v_scales: float16 [sum_s n_kv*L_s*D/32] or None; seq_lens: ints.
    rows: optional iterable of flat row ids ``s*n_q + h``.
    Returns float64 ``[n_slots, n_q, D]``, or ``[len(rows), D]`` when rows is given.
    """
    lib = _load()
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    n_slots = int(seq.shape[0])
    q16 = _as_c(q, np.float16)
    if q16.size != n_slots * n_q * head_dim:
        raise ValueError("q has the wrong number of elements")
    total = int(seq.astype(np.int64).sum()) * n_kv * head_dim
    k16 = _as_c(k, np.float16).reshape(-1)
    if k16.size != total:
        raise ValueError("k has the wrong number of elements")
    if v_scales is None:
        vv = _as_c(v, np.float16).reshape(-1)
        sc = None
    else:
        vv = _as_c(v, np.int8).reshape(-1)
        sc = _as_c(v_scales, np.float16).reshape(-1)
        if sc.size != total // 32:
            raise ValueError("v_scales has the wrong number of elements")
    if vv.size != total:
        raise ValueError("v has the wrong number of elements")
    if rows is None:
        rows_arr = None
        n_rows = n_slots * n_q
        out = np.zeros((n_slots, n_q, head_dim), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        n_rows = int(rows_arr.shape[0])
        out = np.zeros((n_rows, head_dim), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = lib.oracle_attn_decode_f64(
        _ptr(q16), _ptr(k16), _ptr(vv), _ptr(sc), _ptr(seq), int(window), _ptr(out),
        n_slots, int(n_q), int(n_kv), int(head_dim), float(scale),
        _ptr(rows_arr), n_rows, int(threads),
    )
    if rc != 0:
        raise ValueError(f"oracle_attn_decode_f64 returned {rc}")
    return out


def oracle_attn_decode_cache(q, k, v, v_scales, slot_ids, positions, n_cache_slots, capacity, ring,
                             window, n_q, n_kv, head_dim, scale, rows=None, threads=None) -> np.ndarray:
    """Plain fp64 decode attention over a fixed-capacity (linear or ring) cache.

    q: float16 [n_queries, n_q, D]; k: float16 [n_cache_slots, n_kv, capacity, D]
    (any shape with that many elements); v: float16 or int8 like k; v_scales:
    float16 [n_cache_slots, n_kv, capacity, D/32] or None.  Query i reads cache
    slot ``slot_ids[i]`` and attends positions up to ``positions[i]``; linear
    storage keeps position p in row p, ring storage in row p % capacity.
    Returns float64 ``[n_queries, n_q, D]`` (or ``[len(rows), D]``).
    """
    lib = _load()
    sid = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    nqry = int(sid.shape[0])
    if pos.shape[0] != nqry:
        raise ValueError("slot_ids and positions differ in length")
    q16 = _as_c(q, np.float16)
    if q16.size != nqry * n_q * head_dim:
        raise ValueError("q has the wrong number of elements")
    total = int(n_cache_slots) * n_kv * int(capacity) * head_dim
    k16 = _as_c(k, np.float16).reshape(-1)
    if k16.size != total:
        raise ValueError("k has the wrong number of elements")
    if v_scales is None:
        vv = _as_c(v, np.float16).reshape(-1)
        sc = None
    else:
        vv = _as_c(v, np.int8).reshape(-1)
        sc = _as_c(v_scales, np.float16).reshape(-1)
        if sc.size != total // 32:
            raise ValueError("v_scales has the wrong number of elements")
    if vv.size != total:
        raise ValueError("v has the wrong number of elements")
    if rows is None:
        rows_arr = None
        n_rows = nqry * n_q
        out = np.zeros((nqry, n_q, head_dim), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        n_rows = int(rows_arr.shape[0])
        out = np.zeros((n_rows, head_dim), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = lib.oracle_attn_decode_cache_f64(
        _ptr(q16), _ptr(k16), _ptr(vv), _ptr(sc), _ptr(sid), _ptr(pos), nqry, int(n_cache_slots),
        int(capacity), int(ring), int(window), _ptr(out), int(n_q), int(n_kv), int(head_dim),
        float(scale), _ptr(rows_arr), n_rows, int(threads),
    )
    if rc != 0:
        raise ValueError(f"oracle_attn_decode_cache_f64 returned {rc}")
    return out


def float_to_half_bits(x: float) -> int:
    """The oracle's own float32 -> binary16 (round to nearest even), as bits."""
    return int(_load().oracle_float_to_half(float(np.float32(x))))


def quantize_blocks(v) -> tuple:
    """The oracle's block-int8 quantiser on float32 values (length a multiple of 32)."""
    lib = _load()
    vv = _as_c(np.asarray(v, dtype=np.float32), np.float32).reshape(-1)
    if vv.size % 32:
        raise ValueError("length must be a multiple of 32")
    codes = np.zeros(vv.size, dtype=np.int8)
    scales = np.zeros(vv.size // 32, dtype=np.uint16)
    lib.oracle_quantize_blocks(_ptr(vv), vv.size // 32, _ptr(codes), _ptr(scales))
    return codes, scales.view(np.float16)


def oracle_kv_append(k_new, v_new, k_cache, v_cache, v_scales, slot_ids, positions, n_cache_slots,
                     capacity, ring, n_kv, head_dim):
    """Writes new tokens into copies of the cache arrays; returns (k_cache, v_cache, v_scales).

    k_new, v_new: float32 [n_rows, n_kv, D]; caches as for oracle_attn_decode_cache.
    """
    lib = _load()
    sid = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    n_rows = int(sid.shape[0])
    kn = _as_c(np.asarray(k_new), np.float32)
    vn = _as_c(np.asarray(v_new), np.float32)
    if kn.size != n_rows * n_kv * head_dim or vn.size != kn.size:
        raise ValueError("k_new / v_new have the wrong number of elements")
    kc = np.array(k_cache, dtype=np.float16, copy=True).reshape(-1)
    vc = np.array(v_cache, copy=True).reshape(-1)
    sc = None if v_scales is None else np.array(v_scales, dtype=np.float16, copy=True).reshape(-1)
    if v_scales is None and vc.dtype != np.float16:
        raise TypeError("fp16 V cache expected")
    if v_scales is not None and vc.dtype != np.int8:
        raise TypeError("int8 V cache expected")
    rc = lib.oracle_kv_append(_ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), _ptr(sc), _ptr(sid), _ptr(pos),
                              n_rows, int(n_cache_slots), int(capacity), int(ring), int(n_kv), int(head_dim))
    if rc != 0:
        raise ValueError(f"oracle_kv_append returned {rc}")
    return kc, vc, sc


def oracle_attn_decode_cb(q, k, v_codes, v_norms, codebook, codebook_bits, seq_lens, window, n_q, n_kv,
                          head_dim, scale, rows=None, threads=None) -> np.ndarray:
    """Plain fp64 decode attention over packed slots with codebook V (result in the rotated basis).

    v_codes: uint8 packed like k; v_norms: float32 [rows_total * D / B], B = min(D, 256);
    codebook: float32 [2**codebook_bits].
    """
    lib = _load()
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    n_slots = int(seq.shape[0])
    q16 = _as_c(q, np.float16)
    if q16.size != n_slots * n_q * head_dim:
        raise ValueError("q has the wrong number of elements")
    B = min(head_dim, 256)
    total = int(seq.astype(np.int64).sum()) * n_kv * head_dim
    k16 = _as_c(k, np.float16).reshape(-1)
    vc = _as_c(v_codes, np.uint8).reshape(-1)
    vn = _as_c(v_norms, np.float32).reshape(-1)
    cb = _as_c(codebook, np.float32).reshape(-1)
    if k16.size != total or vc.size != total or vn.size != total // B:
        raise ValueError("k / v_codes / v_norms have the wrong number of elements")
    if cb.size < (1 << int(codebook_bits)):
        raise ValueError("codebook is shorter than 2**codebook_bits")
    if rows is None:
        rows_arr = None
        n_rows = n_slots * n_q
        out = np.zeros((n_slots, n_q, head_dim), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        n_rows = int(rows_arr.shape[0])
        out = np.zeros((n_rows, head_dim), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = lib.oracle_attn_decode_cb_f64(
        _ptr(q16), _ptr(k16), _ptr(vc), _ptr(vn), _ptr(cb), int(codebook_bits), _ptr(seq), int(window),
        _ptr(out), n_slots, int(n_q), int(n_kv), int(head_dim), float(scale), _ptr(rows_arr), n_rows,
        int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_decode_cb_f64 returned {rc}")
    return out


def oracle_fwht_undo(x, signs) -> np.ndarray:
    """signs * (H x) / sqrt(D) per row of x (float64 [..., D]), H the Walsh-Hadamard matrix."""
    lib = _load()
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    d = xx.shape[-1]
    sg = _as_c(np.asarray(signs, dtype=np.float32), np.float32).reshape(-1)
    if sg.size != d:
        raise ValueError("signs must have head_dim entries")
    y = np.empty_like(xx)
    rc = lib.oracle_fwht_undo_f64(_ptr(xx), _ptr(sg), _ptr(y), xx.size // d, d)
    if rc != 0:
        raise ValueError(f"oracle_fwht_undo_f64 returned {rc}")
    return y


def _codebook_args(signs, codebook, bits, head_dim):
    sg = _as_c(np.asarray(signs, dtype=np.float32), np.float32).reshape(-1)
    cb = _as_c(np.asarray(codebook, dtype=np.float32), np.float32).reshape(-1)
    if sg.size != head_dim:
        raise ValueError("signs must have head_dim entries")
    if cb.size < (1 << int(bits)):
        raise ValueError("codebook is shorter than 2**bits")
    return sg, cb


def oracle_codebook_encode(v, signs, codebook, bits):
    """The oracle's codebook encode of rows of float32 V (last axis D):
    returns (codes uint8 like v, norms float32 [..., D / B], u float64 like v)."""
    lib = _load()
    vv = _as_c(np.asarray(v, dtype=np.float32), np.float32)
    d = vv.shape[-1]
    B = min(d, 256)
    sg, cb = _codebook_args(signs, codebook, bits, d)
    n = vv.size // d
    codes = np.zeros(vv.shape, dtype=np.uint8)
    norms = np.zeros(vv.shape[:-1] + (d // B,), dtype=np.float32)
    u = np.zeros(vv.shape, dtype=np.float64)
    rc = lib.oracle_codebook_encode_f64(_ptr(vv), _ptr(sg), _ptr(cb), int(bits), n, d, _ptr(codes),
                                        _ptr(norms), _ptr(u))
    if rc != 0:
        raise ValueError(f"oracle_codebook_encode_f64 returned {rc}")
    return codes, norms, u


def oracle_kv_append_cb(k_new, v_new, signs, codebook, bits, k_cache, v_codes, v_norms, slot_ids,
                        positions, n_cache_slots, capacity, ring, n_kv, head_dim):
    """Writes new tokens into copies of a codebook-V cache; returns (k_cache, v_codes, v_norms, u)
    with u float64 [n_rows, n_kv, D] the normalised coordinates each code was chosen for."""
    lib = _load()
    sid = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    n_rows = int(sid.shape[0])
    kn = _as_c(np.asarray(k_new), np.float32)
    vn = _as_c(np.asarray(v_new), np.float32)
    if kn.size != n_rows * n_kv * head_dim or vn.size != kn.size:
        raise ValueError("k_new / v_new have the wrong number of elements")
    sg, cb = _codebook_args(signs, codebook, bits, head_dim)
    kc = np.array(k_cache, dtype=np.float16, copy=True).reshape(-1)
    vc = np.array(v_codes, dtype=np.uint8, copy=True).reshape(-1)
    nm = np.array(v_norms, dtype=np.float32, copy=True).reshape(-1)
    if vc.size != kc.size or nm.size != kc.size // min(head_dim, 256):
        raise ValueError("cache arrays have inconsistent sizes")
    u = np.zeros((n_rows, n_kv, head_dim), dtype=np.float64)
    rc = lib.oracle_kv_append_cb(_ptr(kn), _ptr(vn), _ptr(sg), _ptr(cb), int(bits), _ptr(kc), _ptr(vc),
                                 _ptr(nm), _ptr(sid), _ptr(pos), n_rows, int(n_cache_slots), int(capacity),
                                 int(ring), int(n_kv), int(head_dim), _ptr(u))
    if rc != 0:
        raise ValueError(f"oracle_kv_append_cb returned {rc}")
    return kc, vc, nm, u


def oracle_attn_decode_cache_cb(q, k, v_codes, v_norms, codebook, codebook_bits, slot_ids, positions,
                                n_cache_slots, capacity, ring, window, n_q, n_kv, head_dim, scale,
                                rows=None, threads=None) -> np.ndarray:
    """oracle_attn_decode_cache with codebook V (result in the rotated basis).

    v_codes: uint8 like k; v_norms: float32 [n_cache_slots, n_kv, capacity, D / B], B = min(D, 256).
    """
    lib = _load()
    sid = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32))
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    nqry = int(sid.shape[0])
    if pos.shape[0] != nqry:
        raise ValueError("slot_ids and positions differ in length")
    q16 = _as_c(q, np.float16)
    if q16.size != nqry * n_q * head_dim:
        raise ValueError("q has the wrong number of elements")
    total = int(n_cache_slots) * n_kv * int(capacity) * head_dim
    k16 = _as_c(k, np.float16).reshape(-1)
    vc = _as_c(v_codes, np.uint8).reshape(-1)
    vn = _as_c(v_norms, np.float32).reshape(-1)
    cb = _as_c(codebook, np.float32).reshape(-1)
    if k16.size != total or vc.size != total or vn.size != total // min(head_dim, 256):
        raise ValueError("k / v_codes / v_norms have the wrong number of elements")
    if cb.size < (1 << int(codebook_bits)):
        raise ValueError("codebook is shorter than 2**codebook_bits")
    if rows is None:
        rows_arr = None
        n_rows = nqry * n_q
        out = np.zeros((nqry, n_q, head_dim), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int32))
        n_rows = int(rows_arr.shape[0])
        out = np.zeros((n_rows, head_dim), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = lib.oracle_attn_decode_cache_cb_f64(
        _ptr(q16), _ptr(k16), _ptr(vc), _ptr(vn), _ptr(cb), int(codebook_bits), _ptr(sid), _ptr(pos),
        nqry, int(n_cache_slots), int(capacity), int(ring), int(window), _ptr(out), int(n_q), int(n_kv),
        int(head_dim), float(scale), _ptr(rows_arr), n_rows, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_decode_cache_cb_f64 returned {rc}")
    return out
