"""Thin ctypes binding of ``libattn_decode.so`` (argument marshalling only).

Every entry point has the name of the C function it calls (declared in
``include/attn_decode.h``).  Tensors are passed as device pointers; torch is
used only for device memory and the current stream.  Before a pointer is
handed to the library the binding checks that each tensor lives on the
current GPU, is contiguous and has the dtype and element count the C ABI
expects, so a host pointer can never reach a kernel.  There is no fallback:
if the library is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn_decode.so")

ATTN_DECODE_OK = 0
ATTN_DECODE_EINVAL = -1
ATTN_DECODE_ENOMEM = -2
ATTN_DECODE_EHIP = -3

EXPORTED_SYMBOLS = (
    "attn_decode",
    "attn_decode_cache",
    "attn_decode_cache_cb",
    "attn_decode_cb",
    "attn_decode_ex",
    "attn_decode_noalloc",
    "attn_decode_plan",
    "attn_decode_cache_plan",
    "attn_decode_last_error",
    "attn_decode_release",
    "attn_fwht_undo",
    "attn_kv_append",
    "attn_kv_append_cb",
)


class AttnDecodeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"attn_decode error {code}: {message}")
        self.code = code
        self.message = message


# attn_decode_ex(chunk=CHUNK_PER_CALL): the per-call chunk floor (ATTN_DECODE_CHUNK_PER_CALL)
CHUNK_PER_CALL = -1


class _Options(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int32),
        ("merge_mode", ctypes.c_int32),
        ("ev_partial_begin", ctypes.c_void_p),
        ("ev_partial_end", ctypes.c_void_p),
        ("path", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m decode_attention_kv_02_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(_LIB_PATH)
        common = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
        lib.attn_decode.restype = ctypes.c_int
        lib.attn_decode.argtypes = common
        lib.attn_decode_ex.restype = ctypes.c_int
        lib.attn_decode_ex.argtypes = common + [ctypes.POINTER(_Options)]
        lib.attn_decode_noalloc.restype = ctypes.c_int
        lib.attn_decode_noalloc.argtypes = common + [ctypes.POINTER(_Options)]
        lib.attn_decode_cache.restype = ctypes.c_int
        lib.attn_decode_cache.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(_Options)]
        lib.attn_decode_cb.restype = ctypes.c_int
        lib.attn_decode_cb.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
            ctypes.POINTER(_Options)]
        lib.attn_fwht_undo.restype = ctypes.c_int
        lib.attn_fwht_undo.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_void_p]
        lib.attn_kv_append.restype = ctypes.c_int
        lib.attn_kv_append.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        lib.attn_decode_cache_cb.restype = ctypes.c_int
        lib.attn_decode_cache_cb.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(_Options)]
        lib.attn_kv_append_cb.restype = ctypes.c_int
        lib.attn_kv_append_cb.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_void_p]
        lib.attn_decode_plan.restype = ctypes.c_int
        lib.attn_decode_plan.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.attn_decode_cache_plan.restype = ctypes.c_int
        lib.attn_decode_cache_plan.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.attn_decode_last_error.restype = ctypes.c_char_p
        lib.attn_decode_last_error.argtypes = []
        lib.attn_decode_release.restype = ctypes.c_int
        lib.attn_decode_release.argtypes = []
        _lib = lib
        return lib


def _raise(lib, rc: int):
    msg = lib.attn_decode_last_error()
    raise AttnDecodeError(rc, msg.decode() if msg else "")


class _HostInts:
    """A host int32 array for the C ABI; numpy int32 arrays are passed without a copy."""

    def __init__(self, values):
        if (isinstance(values, np.ndarray) and values.dtype == np.int32 and values.ndim == 1 and values.size
                and values.flags.c_contiguous):
            # the common case (a decode loop passing its own int32 array): no conversion
            self.arr = values
            self.n = int(values.size)
            self._as_parameter_ = ctypes.c_void_p(values.__array_interface__["data"][0])
            return
        if isinstance(values, torch.Tensor):
            values = values.detach().cpu().numpy()
        arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32).reshape(-1))
        self.arr = arr if arr.size else np.zeros(1, dtype=np.int32)
        self.n = int(arr.size)
        self._as_parameter_ = ctypes.c_void_p(self.arr.ctypes.data)

    def __iter__(self):
        return iter(self.arr[:self.n].tolist())


def _seq_array(seq_lens):
    h = _HostInts(seq_lens)
    return h, h.n


def _cuda_index(t, name: str) -> int:
    """Device index of a CUDA tensor; ValueError for anything else."""
    d = t.get_device() if isinstance(t, torch.Tensor) else -1
    if d < 0:
        raise ValueError(f"{name} must be a CUDA tensor")
    return d


def _dev_ptr(t, name: str, dtype, numel: int, device_index: int):
    """Device pointer of a tensor after the marshalling checks (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.get_device() != device_index:        # -1 for host tensors
        raise ValueError(f"{name} must be on cuda:{device_index}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr() if numel else None


def _marshal(q, k_cache, v_cache, v_scales, seq_lens, out, n_slots, n_q_heads, n_kv_heads, head_dim,
             check_v=True):
    seq_arr, n = _seq_array(seq_lens)
    if n_slots is None:
        n_slots = n
    if n_slots != n:
        raise ValueError("n_slots does not match len(seq_lens)")
    if n and int(seq_arr.arr[:n].min()) < 0:
        # the library rejects this too; checked here because sizes below depend on it
        raise AttnDecodeError(ATTN_DECODE_EINVAL, "seq_lens must be >= 0")
    dev = _cuda_index(out, "out")
    kv = int(seq_arr.arr[:n].astype(np.int64).sum()) * n_kv_heads * head_dim
    int8 = v_scales is not None
    ptrs = (
        _dev_ptr(q, "q", torch.float16, n_slots * n_q_heads * head_dim, dev),
        _dev_ptr(k_cache, "k_cache", torch.float16, kv, dev),
        _dev_ptr(v_cache, "v_cache", torch.int8 if int8 else torch.float16, kv, dev) if check_v else None,
        _dev_ptr(v_scales, "v_scales", torch.float16, kv // 32, dev) if int8 else None,
        _dev_ptr(out, "out", torch.float32, n_slots * n_q_heads * head_dim, dev),
    )
    return seq_arr, n_slots, dev, ptrs


# torch's current stream of a device as a raw handle, without building a Stream object (about 2 us
# per call less); the public route where this accessor does not exist
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, dev: int):
    if stream is None:
        if _current_raw_stream is not None:
            return _current_raw_stream(dev)
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def attn_decode(q, k_cache, v_cache, v_scales, seq_lens, window: int, out,
                n_slots: Optional[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                scale: float, stream=None) -> None:
    """Enqueue decode attention on ``stream`` (default: torch's current stream)."""
    lib = load_library()
    seq_arr, n_slots, dev, (pq, pk, pv, ps, po) = _marshal(
        q, k_cache, v_cache, v_scales, seq_lens, out, n_slots, n_q_heads, n_kv_heads, head_dim)
    rc = lib.attn_decode(pq, pk, pv, ps, seq_arr, int(window), po, int(n_slots), int(n_q_heads),
                         int(n_kv_heads), int(head_dim), float(scale), _stream_handle(stream, dev))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_decode_ex(q, k_cache, v_cache, v_scales, seq_lens, window: int, out,
                   n_slots: Optional[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                   scale: float, stream=None, chunk: int = 0, merge_mode: int = 0,
                   ev_partial_begin: Optional[int] = None, ev_partial_end: Optional[int] = None,
                   path: int = 0) -> None:
    """attn_decode with a forced chunk size, a merge mode (0 automatic, 1 combine kernel,
    2 single launch), raw hipEvent_t handles around the partial kernel, and/or a forced
    partial kernel (path: 0 automatic, 1 lanes, 2 matrix cores)."""
    lib = load_library()
    seq_arr, n_slots, dev, (pq, pk, pv, ps, po) = _marshal(
        q, k_cache, v_cache, v_scales, seq_lens, out, n_slots, n_q_heads, n_kv_heads, head_dim)
    opts = _Options(int(chunk), int(merge_mode), ev_partial_begin or None, ev_partial_end or None, int(path))
    rc = lib.attn_decode_ex(pq, pk, pv, ps, seq_arr, int(window), po, int(n_slots), int(n_q_heads),
                            int(n_kv_heads), int(head_dim), float(scale), _stream_handle(stream, dev),
                            ctypes.byref(opts))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_decode_noalloc(q, k_cache, v_cache, v_scales, seq_lens, window: int, out,
                        n_slots: Optional[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                        scale: float, stream=None, chunk: int = 0, merge_mode: int = 0,
                        ev_partial_begin: Optional[int] = None, ev_partial_end: Optional[int] = None,
                        path: int = 0) -> None:
    """attn_decode_ex whose partials go to the library's fixed device scratch (no allocation;
    calls that overlap in time on one GPU race)."""
    lib = load_library()
    seq_arr, n_slots, dev, (pq, pk, pv, ps, po) = _marshal(
        q, k_cache, v_cache, v_scales, seq_lens, out, n_slots, n_q_heads, n_kv_heads, head_dim)
    opts = _Options(int(chunk), int(merge_mode), ev_partial_begin or None, ev_partial_end or None, int(path))
    rc = lib.attn_decode_noalloc(pq, pk, pv, ps, seq_arr, int(window), po, int(n_slots), int(n_q_heads),
                                 int(n_kv_heads), int(head_dim), float(scale), _stream_handle(stream, dev),
                                 ctypes.byref(opts))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_decode_cb(q, k_cache, v_codes, v_norms, codebook, codebook_bits: int, seq_lens, window: int, out,
                   n_slots: Optional[int], n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float,
                   stream=None, chunk: int = 0, merge_mode: int = 0,
                   ev_partial_begin: Optional[int] = None, ev_partial_end: Optional[int] = None,
                   path: int = 0) -> None:
    """Decode attention with codebook V (uint8 indices, fp32 norms per min(D, 256) dims, fp32
    codebook of 2**codebook_bits levels); out is in the rotated basis (see attn_fwht_undo)."""
    lib = load_library()
    seq_arr, n_slots, dev, (pq, pk, _, _, po) = _marshal(
        q, k_cache, None, None, seq_lens, out, n_slots, n_q_heads, n_kv_heads, head_dim, check_v=False)
    kv = int(seq_arr.arr[:seq_arr.n].astype(np.int64).sum()) * n_kv_heads * head_dim
    B = min(head_dim, 256)
    pv = _dev_ptr(v_codes, "v_codes", torch.uint8, kv, dev)
    pn = _dev_ptr(v_norms, "v_norms", torch.float32, kv // B, dev)
    bits = int(codebook_bits)
    if not 1 <= bits <= 8:
        raise AttnDecodeError(ATTN_DECODE_EINVAL, "codebook_bits must be in 1..8")
    pc = _dev_ptr(codebook, "codebook", torch.float32, 1 << bits, dev)
    opts = _Options(int(chunk), int(merge_mode), ev_partial_begin or None, ev_partial_end or None, int(path))
    rc = lib.attn_decode_cb(pq, pk, pv, pn, pc, bits, seq_arr, int(window), po, int(n_slots), int(n_q_heads),
                            int(n_kv_heads), int(head_dim), float(scale), _stream_handle(stream, dev),
                            ctypes.byref(opts))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_fwht_undo(x, signs, y, stream=None) -> None:
    """y = signs * (H x) / sqrt(D) per row of x (fp32 [..., D]); y may be x."""
    lib = load_library()
    dev = _cuda_index(y, "y")
    d = int(x.shape[-1])
    n_rows = x.numel() // d if d else 0
    px = _dev_ptr(x, "x", torch.float32, n_rows * d, dev)
    py = _dev_ptr(y, "y", torch.float32, n_rows * d, dev)
    ps = _dev_ptr(signs, "signs", torch.float32, d, dev)
    rc = lib.attn_fwht_undo(px, ps, py, int(n_rows), d, _stream_handle(stream, dev))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_decode_cache(q, k_cache, v_cache, v_scales, slot_ids, positions, n_queries: Optional[int],
                      n_cache_slots: int, capacity: int, ring: int, window: int, out, n_q_heads: int,
                      n_kv_heads: int, head_dim: int, scale: float, stream=None, chunk: int = 0,
                      merge_mode: int = 0, ev_partial_begin: Optional[int] = None,
                      ev_partial_end: Optional[int] = None, path: int = 0) -> None:
    """Enqueue decode attention over a fixed-capacity (linear or ring) cache."""
    lib = load_library()
    sid, n = _seq_array(slot_ids)
    pos, n2 = _seq_array(positions)
    if n_queries is None:
        n_queries = n
    if n != n_queries or n2 != n_queries:
        raise ValueError("slot_ids / positions do not match n_queries")
    dev = _cuda_index(out, "out")
    kv = int(n_cache_slots) * int(n_kv_heads) * int(capacity) * int(head_dim)
    int8 = v_scales is not None
    pq = _dev_ptr(q, "q", torch.float16, n_queries * n_q_heads * head_dim, dev)
    pk = _dev_ptr(k_cache, "k_cache", torch.float16, kv, dev)
    pv = _dev_ptr(v_cache, "v_cache", torch.int8 if int8 else torch.float16, kv, dev)
    ps = _dev_ptr(v_scales, "v_scales", torch.float16, kv // 32, dev) if int8 else None
    po = _dev_ptr(out, "out", torch.float32, n_queries * n_q_heads * head_dim, dev)
    opts = _Options(int(chunk), int(merge_mode), ev_partial_begin or None, ev_partial_end or None, int(path))
    rc = lib.attn_decode_cache(pq, pk, pv, ps, sid, pos, int(n_queries), int(n_cache_slots),
                               int(capacity), int(ring), int(window), po, int(n_q_heads),
                               int(n_kv_heads), int(head_dim), float(scale),
                               _stream_handle(stream, dev), ctypes.byref(opts))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_kv_append(k_new, v_new, k_cache, v_cache, v_scales, slot_ids, positions, n_rows: Optional[int],
                   n_cache_slots: int, capacity: int, ring: int, n_kv_heads: int, head_dim: int,
                   stream=None) -> None:
    """Enqueue the write of new tokens' K (fp16) and V (fp16 or block-int8) into the cache."""
    lib = load_library()
    sid, n = _seq_array(slot_ids)
    pos, n2 = _seq_array(positions)
    if n_rows is None:
        n_rows = n
    if n != n_rows or n2 != n_rows:
        raise ValueError("slot_ids / positions do not match n_rows")
    dev = _cuda_index(k_cache, "k_cache")
    kv = int(n_cache_slots) * int(n_kv_heads) * int(capacity) * int(head_dim)
    int8 = v_scales is not None
    pkn = _dev_ptr(k_new, "k_new", torch.float32, n_rows * n_kv_heads * head_dim, dev)
    pvn = _dev_ptr(v_new, "v_new", torch.float32, n_rows * n_kv_heads * head_dim, dev)
    pk = _dev_ptr(k_cache, "k_cache", torch.float16, kv, dev)
    pv = _dev_ptr(v_cache, "v_cache", torch.int8 if int8 else torch.float16, kv, dev)
    ps = _dev_ptr(v_scales, "v_scales", torch.float16, kv // 32, dev) if int8 else None
    rc = lib.attn_kv_append(pkn, pvn, pk, pv, ps, sid, pos, int(n_rows), int(n_cache_slots), int(capacity),
                            int(ring), int(n_kv_heads), int(head_dim), _stream_handle(stream, dev))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def _cache_rows(slot_ids, positions, n_queries):
    sid, n = _seq_array(slot_ids)
    pos, n2 = _seq_array(positions)
    if n_queries is None:
        n_queries = n
    if n != n_queries or n2 != n_queries:
        raise ValueError("slot_ids / positions do not match the number of rows")
    return sid, pos, n_queries


def _codebook_ptr(codebook, codebook_bits, dev):
    bits = int(codebook_bits)
    if not 1 <= bits <= 8:
        raise AttnDecodeError(ATTN_DECODE_EINVAL, "codebook_bits must be in 1..8")
    return bits, _dev_ptr(codebook, "codebook", torch.float32, 1 << bits, dev)


def attn_decode_cache_cb(q, k_cache, v_codes, v_norms, codebook, codebook_bits: int, slot_ids, positions,
                         n_queries: Optional[int], n_cache_slots: int, capacity: int, ring: int, window: int,
                         out, n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float, stream=None,
                         chunk: int = 0, merge_mode: int = 0, path: int = 0) -> None:
    """attn_decode_cache with codebook V (uint8 indices and fp32 norms per min(D, 256) dims, laid out
    like the cache); out is in the rotated basis (see attn_fwht_undo)."""
    lib = load_library()
    sid, pos, n_queries = _cache_rows(slot_ids, positions, n_queries)
    dev = _cuda_index(out, "out")
    kv = int(n_cache_slots) * int(n_kv_heads) * int(capacity) * int(head_dim)
    pq = _dev_ptr(q, "q", torch.float16, n_queries * n_q_heads * head_dim, dev)
    pk = _dev_ptr(k_cache, "k_cache", torch.float16, kv, dev)
    pv = _dev_ptr(v_codes, "v_codes", torch.uint8, kv, dev)
    pn = _dev_ptr(v_norms, "v_norms", torch.float32, kv // min(head_dim, 256), dev)
    bits, pc = _codebook_ptr(codebook, codebook_bits, dev)
    po = _dev_ptr(out, "out", torch.float32, n_queries * n_q_heads * head_dim, dev)
    opts = _Options(int(chunk), int(merge_mode), None, None, int(path))
    rc = lib.attn_decode_cache_cb(pq, pk, pv, pn, pc, bits, sid, pos, int(n_queries), int(n_cache_slots),
                                  int(capacity), int(ring), int(window), po, int(n_q_heads), int(n_kv_heads),
                                  int(head_dim), float(scale), _stream_handle(stream, dev), ctypes.byref(opts))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_kv_append_cb(k_new, v_new, k_cache, v_codes, v_norms, signs, codebook, codebook_bits: int, slot_ids,
                      positions, n_rows: Optional[int], n_cache_slots: int, capacity: int, ring: int,
                      n_kv_heads: int, head_dim: int, stream=None) -> None:
    """Enqueue the write of new tokens' K (fp16) and codebook-encoded V (rotated with ``signs``,
    nearest level of ``codebook``, fp32 norms per min(D, 256) dims) into the cache."""
    lib = load_library()
    sid, pos, n_rows = _cache_rows(slot_ids, positions, n_rows)
    dev = _cuda_index(k_cache, "k_cache")
    kv = int(n_cache_slots) * int(n_kv_heads) * int(capacity) * int(head_dim)
    pkn = _dev_ptr(k_new, "k_new", torch.float32, n_rows * n_kv_heads * head_dim, dev)
    pvn = _dev_ptr(v_new, "v_new", torch.float32, n_rows * n_kv_heads * head_dim, dev)
    pk = _dev_ptr(k_cache, "k_cache", torch.float16, kv, dev)
    pv = _dev_ptr(v_codes, "v_codes", torch.uint8, kv, dev)
    pn = _dev_ptr(v_norms, "v_norms", torch.float32, kv // min(head_dim, 256), dev)
    ps = _dev_ptr(signs, "signs", torch.float32, int(head_dim), dev)
    bits, pc = _codebook_ptr(codebook, codebook_bits, dev)
    rc = lib.attn_kv_append_cb(pkn, pvn, pk, pv, pn, ps, pc, bits, sid, pos, int(n_rows), int(n_cache_slots),
                               int(capacity), int(ring), int(n_kv_heads), int(head_dim),
                               _stream_handle(stream, dev))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def attn_kv_append_cb_raw(k_new, v_new, k_cache, v_codes, v_norms, signs, codebook, codebook_bits, slot_ids,
                          positions, n_rows, n_cache_slots, capacity, ring, n_kv_heads, head_dim,
                          stream_ptr=None) -> int:
    """Direct call with raw pointers (tests of the C-side validation); returns the C return code."""
    lib = load_library()
    sid, _ = _seq_array(slot_ids)
    pos, _ = _seq_array(positions)
    return lib.attn_kv_append_cb(k_new, v_new, k_cache, v_codes, v_norms, signs, codebook, int(codebook_bits),
                                 sid, pos, int(n_rows), int(n_cache_slots), int(capacity), int(ring),
                                 int(n_kv_heads), int(head_dim), stream_ptr)


def attn_decode_cache_raw(q_ptr, k_ptr, v_ptr, vs_ptr, slot_ids, positions, n_queries, n_cache_slots,
                          capacity, ring, window, out_ptr, n_q_heads, n_kv_heads, head_dim, scale,
                          stream_ptr=None) -> int:
    """Direct call with raw pointers (tests of the C-side validation); returns the C return code."""
    lib = load_library()
    sid, _ = _seq_array(slot_ids)
    pos, _ = _seq_array(positions)
    return lib.attn_decode_cache(q_ptr, k_ptr, v_ptr, vs_ptr, sid, pos, int(n_queries), int(n_cache_slots),
                                 int(capacity), int(ring), int(window), out_ptr, int(n_q_heads),
                                 int(n_kv_heads), int(head_dim), float(scale), stream_ptr, None)


def attn_decode_raw(q_ptr, k_ptr, v_ptr, vs_ptr, seq_lens, window, out_ptr, n_slots, n_q_heads,
                    n_kv_heads, head_dim, scale, stream_ptr=None) -> int:
    """Direct call with raw pointers (tests of the C-side validation); returns the C return code."""
    lib = load_library()
    seq_arr, _ = _seq_array(seq_lens)
    return lib.attn_decode(q_ptr, k_ptr, v_ptr, vs_ptr, seq_arr, int(window), out_ptr, int(n_slots),
                           int(n_q_heads), int(n_kv_heads), int(head_dim), float(scale), stream_ptr)


def attn_decode_plan(seq_lens, window: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                     v_int8: bool = False, chunk: int = 0) -> dict:
    """The host planner alone (no GPU needed)."""
    lib = load_library()
    seq_arr, n = _seq_array(seq_lens)
    ck = np.zeros(max(n, 1), dtype=np.int32)
    nc = np.zeros(max(n, 1), dtype=np.int32)
    ws = ctypes.c_int64(0)
    items = ctypes.c_int64(0)
    rc = lib.attn_decode_plan(seq_arr, n, int(window), int(n_q_heads), int(n_kv_heads), int(head_dim),
                              int(bool(v_int8)), int(chunk), ck.ctypes.data_as(ctypes.c_void_p),
                              nc.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ws), ctypes.byref(items))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)
    return {"chunk": ck[:n].tolist(), "n_chunks": nc[:n].tolist(), "workspace_bytes": ws.value,
            "partial_workgroups": items.value}


_V_FORMATS = {"fp16": 0, "int8": 1, "codebook": 2}


def attn_decode_cache_plan(slot_ids, positions, n_cache_slots: int, capacity: int, ring: int, window: int,
                           n_q_heads: int, n_kv_heads: int, head_dim: int, v_format: str = "fp16",
                           chunk: int = 0) -> dict:
    """The host planner alone for a cache call (no GPU needed): per query its chunk, chunk count,
    partial kernel ("lanes" or "matrix") and query-group leader."""
    lib = load_library()
    if v_format not in _V_FORMATS:
        raise ValueError(f"v_format must be one of {sorted(_V_FORMATS)}")
    sid, n = _seq_array(slot_ids)
    pos, n2 = _seq_array(positions)
    if n != n2:
        raise ValueError("slot_ids / positions differ in length")
    ck, nc, kern, lead = (np.zeros(max(n, 1), dtype=np.int32) for _ in range(4))
    ws = ctypes.c_int64(0)
    items = ctypes.c_int64(0)
    rc = lib.attn_decode_cache_plan(sid, pos, n,
                                    int(n_cache_slots), int(capacity), int(ring), int(window), int(n_q_heads),
                                    int(n_kv_heads), int(head_dim), _V_FORMATS[v_format], int(chunk),
                                    ck.ctypes.data_as(ctypes.c_void_p), nc.ctypes.data_as(ctypes.c_void_p),
                                    kern.ctypes.data_as(ctypes.c_void_p), lead.ctypes.data_as(ctypes.c_void_p),
                                    ctypes.byref(ws), ctypes.byref(items))
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)
    return {"chunk": ck[:n].tolist(), "n_chunks": nc[:n].tolist(),
            "kernel": ["matrix" if k else "lanes" for k in kern[:n]], "group_leader": lead[:n].tolist(),
            "workspace_bytes": ws.value, "partial_workgroups": items.value}


def attn_decode_release() -> None:
    lib = load_library()
    rc = lib.attn_decode_release()
    if rc != ATTN_DECODE_OK:
        _raise(lib, rc)


def last_error() -> str:
    msg = load_library().attn_decode_last_error()
    return msg.decode() if msg else ""
