#!/usr/bin/env python3
"""Decode-attention benchmark: effective KV GB/s (fraction of HBM peak) and us/call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--quick]

A step is one ``attn_decode`` call (partial kernel + combine kernel) over the
whole batch of the workload, with every input already resident in HBM.  The
headline workload is the hybrid KV regime at 8 slots x 32768 positions (fp16
K, int8 V in blocks of 32 with fp16 scales, 16 q / 8 kv heads, head_dim 256):
1.64 GB of KV per call, far above the 256 MB Infinity Cache, so back-to-back
steps stream from HBM.  The K steps are bracketed by device synchronisation;
``value`` = algorithmic KV bytes per step / wall time per step.

Algorithmic bytes (what the method must move) = every K, V and V-scale byte of
each slot's attended range, read once:
    sum_s n_s * n_kv * (2*D + bytes_V),  bytes_V = 2*D (fp16) or D + 2*D/32 (int8).

One JSON line is printed.  Besides the contract fields it carries
  * ``roofline``: the partial kernel's algorithmic bytes / its average launch
    duration against the 8 TB/s HBM peak.  The duration comes from HIP event
    pairs (timing-only events, created with hipEventDisableSystemFence) that the
    library records around the partial-kernel launch, on the call's stream, on
    every ``--event-every``-th step of the timed region (an event between two
    kernels leaves the GPU idle for a few microseconds, so they are not recorded
    on every step).  ``traffic`` comes from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary when that summary was taken on
    the current kernel source, else null;
  * ``cpu_baseline``: the CPU fp64 oracle timed on a bounded sample of the same
    workload on this host's cores;
  * ``per_config``: every workload preset, warm (back-to-back calls, wall clock
    between device synchronisations), cold (the same with a 1 GiB read of
    another buffer before every call, minus the time of those reads alone) and
    graph (20 calls captured into one HIP graph and replayed: the GPU time per
    call without the Python and launch cost on the host, as a decode loop that
    captures its step sees it) and flushed events (50 reps of the 1 GiB read
    followed by one call between two events on its stream: median, p10, p90,
    and the median of the same pairs with nothing between them; once with
    default events and once with timing-only ones, which skip the system-scope
    cache writeback and invalidation a default event performs),
    with the CPU fp64 oracle over all query rows of the preset on all cores
    (and on one core for the three smallest presets), and the graph figure again
    with ``chunk = CHUNK_PER_CALL`` (``*_chunk_per_call``: chunks raised to the
    per-call floor, which gives up the per-slot bitwise contract; small calls keep
    their chunks),
    plus the codebook-V presets (``attn_decode_cb`` followed by ``attn_fwht_undo``
    in place; bytes = fp16 K, one index byte per V element and the fp32 norms),
    the fixed-capacity cache presets (``attn_decode_cache``: a
    sliding-window ring layer and a speculative-verify shape; rates and
    fractions count ``kv_bytes``, each cache row once, while
    ``kv_bytes_per_query`` counts every query's own rows), and the KV-append presets
    (``attn_kv_append``; ``bytes`` = fp32 K and V read plus the fp16 K and the
    fp16 or int8 V and scales written);
  * ``device_copy_gbs``: a plain 1 GiB device copy, read plus written bytes per
    second, timed for about 0.3 s right before the warm-up steps (context, not
    a ceiling; it also lets the GPU's clocks settle before the timed steps).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(ROOT, "decode_attention_kv_02_amd", "csrc", "attn_decode_kernels.hpp")
MFMA_KERNEL_SRC = os.path.join(ROOT, "decode_attention_kv_02_amd", "csrc", "attn_mfma_kernels.hpp")
TRAFFIC_SUMMARY_DIR = os.path.join(ROOT, "profiles")
METRIC = "decode-attention effective KV GB/s (% of HBM peak) + µs/call per config"
HEADLINE = "hybrid_int8v_8x32768"


def attended(L: int, window: int) -> int:
    return L - (L - window if (window > 0 and L > window) else 0)


def kv_bytes(seq_lens, window, n_kv, d, v_int8) -> int:
    per_row = 2 * d + (d + 2 * (d // 32) if v_int8 else 2 * d)
    return sum(attended(L, window) for L in seq_lens) * n_kv * per_row


def cb_kv_bytes(seq_lens, window, n_kv, d) -> int:
    """Codebook V: fp16 K, one index byte per V element and one fp32 norm per min(D, 256) dims."""
    per_row = 2 * d + d + 4 * (d // min(d, 256))
    return sum(attended(L, window) for L in seq_lens) * n_kv * per_row


def cache_attended(pos: int, capacity: int, ring: int, window: int) -> int:
    L = pos + 1
    lo = L - capacity if (ring and L > capacity) else 0
    if window > 0 and L - window > lo:
        lo = L - window
    return L - lo


def cache_kv_bytes(cfg) -> tuple:
    """(bytes counted per query: every query's own attended rows, as if nothing were shared,
        unique bytes: each cache row counted once however many queries read it)."""
    d = cfg.head_dim
    per_row = 2 * d + (d + 2 * (d // 32) if cfg.v_int8 else 2 * d)
    read = sum(cache_attended(p, cfg.capacity, cfg.ring, cfg.window)
               for p in cfg.positions) * cfg.n_kv_heads * per_row
    spans = {}
    for sid, p in zip(cfg.slot_ids, cfg.positions):
        L = p + 1
        lo = L - cache_attended(p, cfg.capacity, cfg.ring, cfg.window)
        a, b = spans.get(sid, (lo, L))
        spans[sid] = (min(a, lo), max(b, L))
    unique = sum(min(b - a, cfg.capacity) for a, b in spans.values()) * cfg.n_kv_heads * per_row
    return read, unique


def kernel_source_digest(kernel: str = "attn_partial_kernel") -> str:
    """First 16 hex digits of the sha256 of the kernels' source headers (the lane kernel's, and the
    matrix-core kernel's, which includes it), so a summary taken on other kernel code never matches."""
    h = hashlib.sha256()
    for path in (KERNEL_SRC, MFMA_KERNEL_SRC):
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, window: int, kernel: str = "attn_partial_kernel"):
    """HBM bytes per partial-kernel launch from the committed PMC summary, or None when there is
    none or it was taken from another version of the kernel's source."""
    path = os.path.join(TRAFFIC_SUMMARY_DIR, f"traffic_{workload}_w{window}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            vals[m.group(1)] = m.group(2)
    if vals.get("kernel_source_sha256_16") != kernel_source_digest(kernel):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--quick", action="store_true", help="headline workload only (no per_config, no cpu_baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=50, help="calls per timing sample for per_config")
    ap.add_argument("--event-every", type=int, default=8,
                    help="time the partial kernel with HIP events on every N-th timed step")
    ap.add_argument("--chunk", type=int, default=0, help="forced chunk size (tuning only)")
    ap.add_argument("--merge-mode", type=int, default=0, choices=(0, 1, 2),
                    help="merge of split slots: 0 automatic, 1 combine kernel, 2 single launch")
    ap.add_argument("--window", type=int, default=-1,
                    help="attention window of the timed workload (default: the workload's first window)")
    ap.add_argument("--gqa-sweep", action="store_true",
                    help="only time the lane and the matrix-core partial kernels on groups of 8 and 16 "
                         "query heads per kv head (graph-replayed calls, one JSON line per shape)")
    ap.add_argument("--only", default="", help="with --gqa-sweep: comma-separated shape names to run")
    ap.add_argument("--torch-reductions", action="store_true",
                    help="time torch's own sum / amax reading 1-4 GiB (a reference streaming read) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args(argv)


def calibrate_copy(nbytes: int) -> int:
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "copies": 5}), flush=True)
    return 0


def measured_copy_gbs(dev, nbytes: int = 1 << 30, seconds: float = 0.3, keep: list = None):
    """(bytes moved per second, read + written, by a plain device-to-device copy of `nbytes`,
    back to back on the current stream for about `seconds`; the seconds it ran).  Context for
    the partial kernel's rate, not a ceiling.  It runs right before the headline's warm-up
    steps: after an idle spell the GPU takes some 10 ms of streaming to settle (calls 10-40 of
    a fresh loop ran up to 7% slower than later ones), and this copy is that much streaming
    work of its own.  With `keep` (a list), the two buffers are appended to it instead of
    being freed: calls right after a large free ran about 2% slower (measured over 60 calls),
    so the caller frees them after its timed region."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 0
    while True:
        for _ in range(10):
            dst.copy_(src)
        reps += 10
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if keep is not None:
        keep.extend((src, dst))
    else:
        del src, dst
        torch.cuda.empty_cache()
    return 2 * nbytes * reps / el / 1e9, el


class TimingEvent:
    """A hipEvent for timing only, created with hipEventDisableSystemFence: HIP documents that
    such an event skips the system-scope cache writeback and invalidation that a default event
    performs when it is recorded, which makes the interval between two of them more precise.
    Used where the bench times GPU work between events; nothing on the host reads results
    through them."""
    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, stream):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._c = ctypes
        self.handle = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.handle), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.record(stream)   # a recorded event, as torch's own new_event() gives

    @property
    def cuda_event(self) -> int:
        return self.handle.value

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.handle, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both complete)."""
        ms = self._c.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        hip = type(self)._hip   # the class stays reachable at interpreter exit, its module name may not
        if hip is not None and self.handle:
            hip.hipEventDestroy(self.handle)


def torch_reductions() -> int:
    """GB/s of torch's own reductions reading 1, 2 and 4 GiB once (sum and amax over fp16 and fp32),
    10 calls captured into a graph and replayed: a streaming read written by someone else, for
    comparison with the partial kernel's rate."""
    import torch
    dev = torch.device("cuda:0")
    for gib in (1, 2, 4):
        for dtype in (torch.float16, torch.float32):
            x = torch.ones((gib << 30) // torch.tensor([], dtype=dtype).element_size(), dtype=dtype, device=dev)
            for name, fn in (("sum", lambda: x.sum()), ("amax", lambda: x.amax())):
                side = torch.cuda.Stream(device=dev)
                side.wait_stream(torch.cuda.current_stream(dev))
                with torch.cuda.stream(side):
                    fn()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=side):
                    for _ in range(10):
                        fn()
                torch.cuda.synchronize()
                samples = []
                for _ in range(5):
                    t0 = time.perf_counter()
                    graph.replay()
                    torch.cuda.synchronize()
                    samples.append((time.perf_counter() - t0) / 10)
                s_per = statistics.median(samples)
                gbs = (gib << 30) / s_per / 1e9
                print(json.dumps({"read": f"{name} {str(dtype).replace('torch.', '')}", "bytes": gib << 30,
                                  "us_per_call": round(s_per * 1e6, 2), "gbs": round(gbs, 1),
                                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
                del graph
            del x
            torch.cuda.empty_cache()
    return 0


# Shapes with 8 or 16 query heads per kv head (gemma4's global layers have 8 at head_dim 512),
# inputs drawn on the GPU (timing only): name, slots x length, q heads, kv heads, head_dim, V format
GQA_SHAPES = (
    ("g8_d512_fp16_4x32768", (32768,) * 4, 16, 2, 512, "fp16"),
    ("g8_d512_codebook_4x32768", (32768,) * 4, 16, 2, 512, "codebook"),
    ("g8_d512_int8_4x32768", (32768,) * 4, 16, 2, 512, "int8"),
    ("g8_d512_codebook_8x32768", (32768,) * 8, 16, 2, 512, "codebook"),
    ("g8_d512_int8_8x32768", (32768,) * 8, 16, 2, 512, "int8"),
    ("g8_d256_fp16_4x32768", (32768,) * 4, 16, 2, 256, "fp16"),
    ("g8_d256_codebook_4x32768", (32768,) * 4, 16, 2, 256, "codebook"),
    ("g8_d128_fp16_8x8192", (8192,) * 8, 64, 8, 128, "fp16"),
    ("g8_d128_int8_8x8192", (8192,) * 8, 64, 8, 128, "int8"),
    ("g8_d128_codebook_8x8192", (8192,) * 8, 64, 8, 128, "codebook"),
    ("g16_d512_fp16_4x16384", (16384,) * 4, 32, 2, 512, "fp16"),
    ("g16_d256_fp16_4x16384", (16384,) * 4, 32, 2, 256, "fp16"),
    ("g16_d256_int8_4x16384", (16384,) * 4, 32, 2, 256, "int8"),
    ("g16_d128_fp16_8x8192", (8192,) * 8, 64, 4, 128, "fp16"),
)


def oracle_per_config(inp, W: int, one_thread: bool) -> dict:
    """The CPU fp64 oracle over every query row of a preset, one pass: µs per call and KV GB/s on
    all of this host's cores (`oracle_*`) and, when asked, on one core (`oracle_1thread_*`)."""
    from oracle import oracle_attn_decode
    threads = len(os.sched_getaffinity(0))
    rows = list(range(inp.n_slots * inp.n_q_heads))
    nb = kv_bytes(inp.seq_lens, W, inp.n_kv_heads, inp.head_dim, inp.v_int8)
    sn = None if inp.v_scales is None else inp.v_scales.numpy()
    res = {"oracle_threads": threads}
    for key, t in (("oracle", threads),) + ((("oracle_1thread", 1),) if one_thread else ()):
        t0 = time.perf_counter()
        oracle_attn_decode(inp.q.numpy(), inp.k.numpy(), inp.v.numpy(), sn, inp.seq_lens, W, inp.n_q_heads,
                           inp.n_kv_heads, inp.head_dim, inp.scale, rows=rows, threads=t)
        dt = time.perf_counter() - t0
        res[key + "_us_per_call"] = round(dt * 1e6, 1)
        res[key + "_gbs"] = round(nb / dt / 1e9, 3)
    return res


def partial_kernel_name(G: int, head_dim: int, drafts: int = 1, byte_v: bool = False) -> str:
    """The partial kernel the library's automatic choice (planner.hpp) runs: the matrix cores at a
    multiple of 8 query heads per kv head, or for a slot's drafts x heads filling 4 columns (8 at
    head_dim 512 with one-byte V)."""
    min_cols = 8 if (head_dim == 512 and byte_v) else 4
    if head_dim >= 128 and (G % 8 == 0 or drafts * G >= min_cols):
        return "attn_partial_mfma_kernel"
    return "attn_partial_kernel"


def gqa_sweep(only: str = "") -> int:
    import numpy as np
    import torch
    from decode_attention_kv_02_amd import binding
    binding.load_library()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    names = [x for x in only.split(",") if x]
    unknown = set(names) - {sh[0] for sh in GQA_SHAPES}
    if unknown:
        print(f"unknown shapes {sorted(unknown)}; choose from {[sh[0] for sh in GQA_SHAPES]}", file=sys.stderr)
        return 2
    for name, seq, nq, nkv, d, fmt in GQA_SHAPES:
        if names and name not in names:
            continue
        n = sum(seq) * nkv * d
        q = torch.randn(len(seq) * nq * d, generator=gen, device=dev).half()
        k = torch.randn(n, generator=gen, device=dev).half()
        out = torch.empty((len(seq), nq, d), dtype=torch.float32, device=dev)
        seq_a = np.asarray(seq, dtype=np.int32)
        if fmt == "codebook":
            vc = torch.randint(0, 256, (n,), generator=gen, device=dev, dtype=torch.uint8)
            vn = torch.rand(n // min(d, 256), generator=gen, device=dev) * 4 + 14
            cb = torch.randn(256, generator=gen, device=dev)
            nb = cb_kv_bytes(seq, 0, nkv, d)

            def call(st, path):
                binding.attn_decode_cb(q, k, vc, vn, cb, 8, seq_a, 0, out, len(seq), nq, nkv, d, d ** -0.5,
                                       stream=st, path=path)
        else:
            if fmt == "fp16":
                v, vs = torch.randn(n, generator=gen, device=dev).half(), None
            else:
                v = torch.randint(-127, 128, (n,), generator=gen, device=dev, dtype=torch.int8)
                vs = (torch.rand(n // 32, generator=gen, device=dev) * 0.03).half()
            nb = kv_bytes(seq, 0, nkv, d, fmt == "int8")

            def call(st, path):
                binding.attn_decode_ex(q, k, v, vs, seq_a, 0, out, len(seq), nq, nkv, d, d ** -0.5, stream=st,
                                       path=path)
        res = {"shape": name, "kv_bytes": nb}
        for path, key in ((1, "lanes"), (2, "matrix")):
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                for _ in range(3):
                    call(side, path)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                for _ in range(20):
                    call(side, path)
            torch.cuda.synchronize()
            samples = []
            for _ in range(5):
                t0 = time.perf_counter()
                for _ in range(10):
                    graph.replay()
                torch.cuda.synchronize()
                samples.append((time.perf_counter() - t0) * 1e6 / 200)
            us = statistics.median(samples)
            res[key + "_us"] = round(us, 2)
            res[key + "_hbm_frac"] = round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            del graph
        res["automatic"] = ("matrix" if partial_kernel_name(nq // nkv, d, byte_v=fmt != "fp16") ==
                            "attn_partial_mfma_kernel" else "lanes")
        print(json.dumps(res), flush=True)
        del q, k, out
        torch.cuda.empty_cache()
    return 0


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path would shard "
              "by slot, KV head or sequence chunk across GPUs, but no multi-GPU run exists)", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.torch_reductions:
        return torch_reductions()
    if args.gqa_sweep:
        return gqa_sweep(args.only)

    import numpy as np
    import torch

    from decode_attention_kv_02_amd import binding
    from decode_attention_kv_02_amd.workloads import (APPEND_WORKLOADS, CACHE_WORKLOADS, CODEBOOK_WORKLOADS,
                                                      SERVE_STEP_WORKLOADS, serve_step_inputs,
                                                      WORKLOADS, append_new_rows, cache_workload_inputs,
                                                      codebook_workload_inputs, workload_inputs)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    by_name = {w.name: w for w in WORKLOADS}
    cb_by_name = {w.name: w for w in CODEBOOK_WORKLOADS}
    cache_by_name = {w.name: w for w in CACHE_WORKLOADS}
    if args.workload not in by_name and args.workload not in cb_by_name and args.workload not in cache_by_name:
        print(f"unknown workload {args.workload}; choose from "
              f"{sorted(by_name) + sorted(cb_by_name) + sorted(cache_by_name)}", file=sys.stderr)
        return 2

    def upload(inp):
        return (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                None if inp.v_scales is None else inp.v_scales.to(dev))

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # materialise the underlying hipEvent_t
        return e

    def call(inp, tens, out, W, ev0=None, ev1=None, st=None, chunk=None):
        q, k, v, vs = tens
        binding.attn_decode_ex(q, k, v, vs, inp.seq_lens, W, out, inp.n_slots, inp.n_q_heads,
                               inp.n_kv_heads, inp.head_dim, inp.scale, stream=st or stream,
                               chunk=args.chunk if chunk is None else chunk, merge_mode=args.merge_mode,
                               ev_partial_begin=ev0.cuda_event if ev0 is not None else None,
                               ev_partial_end=ev1.cuda_event if ev1 is not None else None)

    if args.workload in by_name:
        cfg = by_name[args.workload]
        window = cfg.windows[0] if args.window < 0 else args.window
        print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
        inp = workload_inputs(cfg)
        tens = upload(inp)
        out = torch.empty((inp.n_slots, inp.n_q_heads, inp.head_dim), dtype=torch.float32, device=dev)
        nbytes = kv_bytes(inp.seq_lens, window, inp.n_kv_heads, inp.head_dim, inp.v_int8)
        v_format = "int8 codes, fp16 scale per 32 dims" if inp.v_int8 else "fp16"

        def step(ev0=None, ev1=None):
            call(inp, tens, out, window, ev0, ev1)
    elif args.workload in cache_by_name:
        cfg = cache_by_name[args.workload]
        window = cfg.window
        print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
        inp = cache_workload_inputs(cfg)
        tens = upload(inp)
        out = torch.empty((inp.n_queries, inp.n_q_heads, inp.head_dim), dtype=torch.float32, device=dev)
        # rates on the unique bytes (each cache row once, as HBM serves it); draft queries of one
        # slot share their rows, so bytes counted per query would exceed what is read
        per_query_bytes, nbytes = cache_kv_bytes(cfg)
        v_format = "int8 codes, fp16 scale per 32 dims" if inp.v_scales is not None else "fp16"
        c_sid = np.asarray(inp.slot_ids, dtype=np.int32)
        c_pos = np.asarray(inp.positions, dtype=np.int32)

        def step(ev0=None, ev1=None):
            binding.attn_decode_cache(*tens, c_sid, c_pos, inp.n_queries, inp.n_cache_slots, inp.capacity,
                                      inp.ring, window, out, inp.n_q_heads, inp.n_kv_heads, inp.head_dim,
                                      inp.scale, stream=stream, chunk=args.chunk,
                                      ev_partial_begin=ev0.cuda_event if ev0 is not None else None,
                                      ev_partial_end=ev1.cuda_event if ev1 is not None else None)
    else:
        cfg = cb_by_name[args.workload]
        window = cfg.window
        print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
        inp = codebook_workload_inputs(cfg)
        cb_t = tuple(t.to(dev) for t in (inp.q, inp.k, inp.v_codes, inp.v_norms, inp.codebook, inp.signs))
        out = torch.empty((inp.n_slots, inp.n_q_heads, inp.head_dim), dtype=torch.float32, device=dev)
        nbytes = cb_kv_bytes(inp.seq_lens, window, inp.n_kv_heads, inp.head_dim)
        v_format = f"{inp.codebook_bits}-bit codebook indices, fp32 norm per {min(inp.head_dim, 256)} dims"
        cb_seq = np.asarray(inp.seq_lens, dtype=np.int32)

        def step(ev0=None, ev1=None):
            q, k, vc, vn, cb, sg = cb_t
            binding.attn_decode_cb(q, k, vc, vn, cb, inp.codebook_bits, cb_seq, window, out, inp.n_slots,
                                   inp.n_q_heads, inp.n_kv_heads, inp.head_dim, inp.scale, stream=stream,
                                   chunk=args.chunk,
                                   ev_partial_begin=ev0.cuda_event if ev0 is not None else None,
                                   ev_partial_end=ev1.cuda_event if ev1 is not None else None)
            binding.attn_fwht_undo(out, sg, out, stream=stream)

    # context, not a ceiling: a plain 1 GiB device copy on this GPU, read plus written bytes per
    # second (a copy pays for its writes, so a read-only stream can exceed it); measured here, before
    # the warm-up steps, so the timed steps do not start on clocks still settling from idle
    copy_bufs = []
    copy_gbs, copy_s = measured_copy_gbs(dev, keep=copy_bufs)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def graph_us_per_call(fn, n_calls=20, n_replays=10):
        """GPU time per call with the host out of the loop: n_calls calls captured into one
        graph on a side stream (each call only enqueues kernels; the workspace was sized by
        the warm-up calls), replayed n_replays times back to back."""
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(n_calls):
                fn(side)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_replays):
            graph.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (n_replays * n_calls)
        del graph
        return us

    # Event pairs around the partial kernel on every `event_every`-th step only:
    # each event between kernels idles the GPU for several microseconds, so
    # recording them on every step would slow the steps being timed.
    sampled = set(range(0, args.steps, max(1, args.event_every)))
    evs = {i: (TimingEvent(stream), TimingEvent(stream)) for i in sampled}
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i in evs:
            step(*evs[i])
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    del copy_bufs[:]
    torch.cuda.empty_cache()
    partial_ms = [e0.elapsed_time(e1) for e0, e1 in evs.values()]
    partial_avg_s = statistics.fmean(partial_ms) * 1e-3
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / partial_avg_s / 1e9
    assert torch.isfinite(out).all().item(), "non-finite output"

    if args.workload in cache_by_name:
        shape = {"n_queries": inp.n_queries, "slot_ids": list(inp.slot_ids), "positions": list(inp.positions),
                 "n_cache_slots": inp.n_cache_slots, "capacity": inp.capacity, "ring": inp.ring,
                 "kv_bytes_per_query": per_query_bytes}
        drafts = max(inp.slot_ids.count(s_) for s_ in set(inp.slot_ids))
    else:
        shape = {"n_slots": inp.n_slots, "seq_lens": list(inp.seq_lens)}
        drafts = 1
    kernel = partial_kernel_name(inp.n_q_heads // inp.n_kv_heads, inp.head_dim, drafts, byte_v=v_format != "fp16")
    traffic = read_traffic(cfg.name, window, kernel)
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            **shape,
            "n_q_heads": inp.n_q_heads,
            "n_kv_heads": inp.n_kv_heads,
            "head_dim": inp.head_dim,
            "window": window,
            "k_format": "fp16",
            "v_format": v_format,
            "kv_bytes_per_call": nbytes,
            "us_per_call": round(ms_per_step * 1e3, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "chunk_override": args.chunk,
            "merge_mode": args.merge_mode,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(partial_avg_s * 1e6, 2),
            "launches_timed": len(partial_ms),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    result["device_copy_gbs"] = round(copy_gbs, 1)
    result["device_copy_seconds"] = round(copy_s, 3)

    # ---- every preset: cold (flushed) and warm
    if not args.quick:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        # the same flushed event pairs with nothing between them: what the pair itself adds
        empty = [(new_event(), new_event()) for _ in range(50)]
        torch.cuda.synchronize()
        for e0, e1 in empty:
            flush.sum()
            e0.record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        empty_pair_us = statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in empty)
        # and with timing-only events (TimingEvent: no system-scope fence when recorded)
        empty_t = [(TimingEvent(stream), TimingEvent(stream)) for _ in range(50)]
        torch.cuda.synchronize()
        for e0, e1 in empty_t:
            flush.sum()
            e0.record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        empty_pair_t_us = statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in empty_t)
        del empty_t
        per = []
        for wi, w in enumerate(WORKLOADS):
            if w.name != cfg.name or args.workload not in by_name:
                print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
                pin = workload_inputs(w)
                ptens = upload(pin)
            else:
                pin, ptens = inp, tens
            orc = {}
            if not args.no_cpu_baseline:
                # the three smallest presets also on one core; the larger ones on all cores only
                orc = {W: oracle_per_config(pin, W, wi <= 2) for W in w.windows}
                print(f"[bench] {w.name}: oracle {orc}", file=sys.stderr, flush=True)
            if pin is not inp:
                del pin.k, pin.v
            pout = torch.empty((pin.n_slots, pin.n_q_heads, pin.head_dim), dtype=torch.float32, device=dev)
            for W in w.windows:
                nb = kv_bytes(pin.seq_lens, W, pin.n_kv_heads, pin.head_dim, pin.v_int8)
                for _ in range(3):
                    call(pin, ptens, pout, W)

                def per_call_us(fn, n):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    for _ in range(n):
                        fn()
                    torch.cuda.synchronize()
                    return (time.perf_counter() - t0) * 1e6 / n

                def one_call():
                    call(pin, ptens, pout, W)

                def flush_only():
                    flush.sum()  # reads 1 GiB: evicts the inputs, leaves no dirty lines

                def flush_then_call():
                    flush.sum()
                    call(pin, ptens, pout, W)

                warm = statistics.median(per_call_us(one_call, args.reps) for _ in range(3))
                cold_samples = [per_call_us(flush_then_call, args.reps) - per_call_us(flush_only, args.reps)
                                for _ in range(5)]
                cold = statistics.median(cold_samples)
                pk = []
                for _ in range(5):
                    c0, c1 = TimingEvent(stream), TimingEvent(stream)
                    call(pin, ptens, pout, W, c0, c1)
                    torch.cuda.synchronize()
                    pk.append(c0.elapsed_time(c1) * 1e3)
                g_us = graph_us_per_call(lambda st: call(pin, ptens, pout, W, st=st))
                # the same call with the per-call chunk floor (chunk = CHUNK_PER_CALL; small calls
                # keep their chunks), context beside the per-slot figures
                call(pin, ptens, pout, W, chunk=binding.CHUNK_PER_CALL)
                g_pc = graph_us_per_call(lambda st: call(pin, ptens, pout, W, st=st, chunk=binding.CHUNK_PER_CALL))
                # 50 reps of: a 1 GiB flush read, then one whole call (plan upload, partial and
                # combine kernels) between two events on the call's stream
                pairs = [(new_event(), new_event()) for _ in range(50)]
                torch.cuda.synchronize()
                for e0, e1 in pairs:
                    flush.sum()
                    e0.record(stream)
                    call(pin, ptens, pout, W)
                    e1.record(stream)
                torch.cuda.synchronize()
                ev = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)
                ev_med, ev_p10, ev_p90 = statistics.median(ev), ev[len(ev) // 10], ev[(9 * len(ev)) // 10]
                # the same protocol between timing-only events
                pairs_t = [(TimingEvent(stream), TimingEvent(stream)) for _ in range(50)]
                torch.cuda.synchronize()
                for e0, e1 in pairs_t:
                    flush.sum()
                    e0.record(stream)
                    call(pin, ptens, pout, W)
                    e1.record(stream)
                torch.cuda.synchronize()
                evt = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs_t)
                del pairs_t
                evt_med = statistics.median(evt)
                per.append({
                    "workload": w.name, "window": W, "kv_bytes": nb,
                    "cold_event_us": {"median": round(ev_med, 2), "p10": round(ev_p10, 2),
                                      "p90": round(ev_p90, 2), "reps": len(ev),
                                      "empty_pair_median": round(empty_pair_us, 2)},
                    "cold_event_hbm_frac": round(nb / (ev_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "cold_timing_event_us": {"median": round(evt_med, 2), "p10": round(evt[len(evt) // 10], 2),
                                             "p90": round(evt[(9 * len(evt)) // 10], 2), "reps": len(evt),
                                             "empty_pair_median": round(empty_pair_t_us, 2)},
                    "cold_timing_event_hbm_frac": round(nb / (evt_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    **orc.get(W, {}),
                    "warm_us_per_call": round(warm, 2),
                    "warm_gbs": round(nb / (warm * 1e-6) / 1e9, 1),
                    "warm_hbm_frac": round(nb / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "cold_us_per_call": round(cold, 2),
                    "cold_gbs": round(nb / (cold * 1e-6) / 1e9, 1),
                    "cold_hbm_frac": round(nb / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "cold_us_samples": [round(x, 2) for x in cold_samples],
                    "partial_kernel_us_median": round(statistics.median(pk), 2),
                    "graph_us_per_call": round(g_us, 2),
                    "graph_gbs": round(nb / (g_us * 1e-6) / 1e9, 1),
                    "graph_hbm_frac": round(nb / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "graph_us_per_call_chunk_per_call": round(g_pc, 2),
                    "graph_hbm_frac_chunk_per_call": round(nb / (g_pc * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                })
                print(f"[bench] {w.name} W={W}: warm {warm:.2f} us ({per[-1]['warm_gbs']} GB/s), "
                      f"cold {cold:.2f} us ({per[-1]['cold_gbs']} GB/s), graph {g_us:.2f} us, "
                      f"flushed events median {ev_med:.2f} (p10 {ev_p10:.2f}, p90 {ev_p90:.2f}) us, "
                      f"timing-only events {evt_med:.2f} us",
                      file=sys.stderr, flush=True)
            if w.name != cfg.name or args.workload not in by_name:
                del ptens
                torch.cuda.empty_cache()

        # codebook-V presets (attn_decode_cb + attn_fwht_undo in place on the output)
        for bw in CODEBOOK_WORKLOADS:
            print(f"[bench] generating {bw.name}", file=sys.stderr, flush=True)
            bi = codebook_workload_inputs(bw)
            bq, bk, bvc, bvn, bcb = (t.to(dev) for t in (bi.q, bi.k, bi.v_codes, bi.v_norms, bi.codebook))
            bsg = bi.signs.to(dev)
            del bi.k, bi.v_codes, bi.v_norms
            bout = torch.empty((bi.n_slots, bi.n_q_heads, bi.head_dim), dtype=torch.float32, device=dev)
            b_seq = np.asarray(bi.seq_lens, dtype=np.int32)

            def cb_call(e0=None, e1=None, st=None, chunk=0):
                binding.attn_decode_cb(bq, bk, bvc, bvn, bcb, bi.codebook_bits, b_seq, bw.window, bout,
                                       bi.n_slots, bi.n_q_heads, bi.n_kv_heads, bi.head_dim, bi.scale,
                                       stream=st or stream, chunk=chunk,
                                       ev_partial_begin=e0.cuda_event if e0 is not None else None,
                                       ev_partial_end=e1.cuda_event if e1 is not None else None)
                binding.attn_fwht_undo(bout, bsg, bout, stream=st or stream)

            def per_call_us(fn, n):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(n):
                    fn()
                torch.cuda.synchronize()
                return (time.perf_counter() - t0) * 1e6 / n

            def flush_then_cb_call():
                flush.sum()
                cb_call()

            for _ in range(3):
                cb_call()
            nb = cb_kv_bytes(bi.seq_lens, bw.window, bi.n_kv_heads, bi.head_dim)
            warm = statistics.median(per_call_us(cb_call, args.reps) for _ in range(3))
            cold = statistics.median(per_call_us(flush_then_cb_call, args.reps) -
                                     per_call_us(lambda: flush.sum(), args.reps) for _ in range(5))
            pk = []
            for _ in range(5):
                c0, c1 = TimingEvent(stream), TimingEvent(stream)
                cb_call(c0, c1)
                torch.cuda.synchronize()
                pk.append(c0.elapsed_time(c1) * 1e3)
            assert torch.isfinite(bout).all().item(), "non-finite output"
            g_us = graph_us_per_call(lambda st: cb_call(st=st))
            per.append({
                "workload": bw.name, "window": bw.window, "kv_bytes": nb,
                "v_format": f"{bi.codebook_bits}-bit codebook indices, fp32 norm per {min(bi.head_dim, 256)} dims",
                "step": "attn_decode_cb + attn_fwht_undo",
                "warm_us_per_call": round(warm, 2),
                "warm_gbs": round(nb / (warm * 1e-6) / 1e9, 1),
                "warm_hbm_frac": round(nb / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "cold_us_per_call": round(cold, 2),
                "cold_gbs": round(nb / (cold * 1e-6) / 1e9, 1),
                "cold_hbm_frac": round(nb / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "partial_kernel_us_median": round(statistics.median(pk), 2),
                "partial_kernel_gbs": round(nb / (statistics.median(pk) * 1e-6) / 1e9, 1),
                "graph_us_per_call": round(g_us, 2),
                "graph_gbs": round(nb / (g_us * 1e-6) / 1e9, 1),
            })
            # the same step with the per-call chunk floor (chunk = CHUNK_PER_CALL)
            for _ in range(3):
                cb_call(chunk=binding.CHUNK_PER_CALL)
            pk_pc = []
            for _ in range(5):
                c0, c1 = TimingEvent(stream), TimingEvent(stream)
                cb_call(c0, c1, chunk=binding.CHUNK_PER_CALL)
                torch.cuda.synchronize()
                pk_pc.append(c0.elapsed_time(c1) * 1e3)
            g_pc = graph_us_per_call(lambda st: cb_call(st=st, chunk=binding.CHUNK_PER_CALL))
            per[-1].update({"partial_kernel_us_median_chunk_per_call": round(statistics.median(pk_pc), 2),
                            "graph_us_per_call_chunk_per_call": round(g_pc, 2)})
            print(f"[bench] {bw.name}: warm {warm:.2f} us ({per[-1]['warm_gbs']} GB/s), cold {cold:.2f} us, "
                  f"partial {per[-1]['partial_kernel_gbs']} GB/s", file=sys.stderr, flush=True)
            del bq, bk, bvc, bvn, bcb, bsg, bout
            torch.cuda.empty_cache()

        # fixed-capacity cache presets (attn_decode_cache)
        for cw in CACHE_WORKLOADS:
            print(f"[bench] generating {cw.name}", file=sys.stderr, flush=True)
            ci = cache_workload_inputs(cw)
            ct = upload(ci)
            del ci.k, ci.v
            cout = torch.empty((ci.n_queries, ci.n_q_heads, ci.head_dim), dtype=torch.float32, device=dev)

            c_sid = np.asarray(ci.slot_ids, dtype=np.int32)
            c_pos = np.asarray(ci.positions, dtype=np.int32)

            def cache_call(e0=None, e1=None, st=None, chunk=0):
                binding.attn_decode_cache(*ct, c_sid, c_pos, ci.n_queries, ci.n_cache_slots,
                                          ci.capacity, ci.ring, cw.window, cout, ci.n_q_heads,
                                          ci.n_kv_heads, ci.head_dim, ci.scale, stream=st or stream,
                                          chunk=chunk,
                                          ev_partial_begin=e0.cuda_event if e0 is not None else None,
                                          ev_partial_end=e1.cuda_event if e1 is not None else None)

            def per_call_us(fn, n):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(n):
                    fn()
                torch.cuda.synchronize()
                return (time.perf_counter() - t0) * 1e6 / n

            def flush_then_cache_call():
                flush.sum()
                cache_call()

            for _ in range(3):
                cache_call()
            read_b, uniq_b = cache_kv_bytes(cw)
            warm = statistics.median(per_call_us(cache_call, args.reps) for _ in range(3))
            cold = statistics.median(per_call_us(flush_then_cache_call, args.reps) -
                                     per_call_us(lambda: flush.sum(), args.reps) for _ in range(5))
            g_us = graph_us_per_call(lambda st: cache_call(st=st))
            # rates and fractions on the unique bytes (each cache row once, as HBM serves it);
            # kv_bytes_per_query counts every query's own rows, as if nothing were shared
            per.append({
                "workload": cw.name, "window": cw.window, "kv_bytes": uniq_b, "kv_bytes_per_query": read_b,
                "warm_us_per_call": round(warm, 2),
                "warm_gbs": round(uniq_b / (warm * 1e-6) / 1e9, 1),
                "warm_hbm_frac": round(uniq_b / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "cold_us_per_call": round(cold, 2),
                "cold_gbs": round(uniq_b / (cold * 1e-6) / 1e9, 1),
                "cold_hbm_frac": round(uniq_b / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "graph_us_per_call": round(g_us, 2),
                "graph_gbs": round(uniq_b / (g_us * 1e-6) / 1e9, 1),
                "graph_hbm_frac": round(uniq_b / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            })
            if ci.n_queries > 48:
                # the same batch with the per-call chunk floor (chunk = CHUNK_PER_CALL): longer
                # chunks for a large batch of short slots, rounding then depending on the batch
                for _ in range(3):
                    cache_call(chunk=binding.CHUNK_PER_CALL)
                g_pc = graph_us_per_call(lambda st: cache_call(st=st, chunk=binding.CHUNK_PER_CALL))
                per[-1].update({"graph_us_per_call_chunk_per_call": round(g_pc, 2),
                                "graph_hbm_frac_chunk_per_call": round(uniq_b / (g_pc * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
            print(f"[bench] {cw.name}: warm {warm:.2f} us ({per[-1]['warm_gbs']} GB/s), cold {cold:.2f} us",
                  file=sys.stderr, flush=True)
            del ct
            torch.cuda.empty_cache()
        # serving steps on a codebook-V cache: attn_kv_append_cb + attn_decode_cache_cb + attn_fwht_undo
        for sw in SERVE_STEP_WORKLOADS:
            print(f"[bench] generating {sw.name}", file=sys.stderr, flush=True)
            ci, kn_h, vn_h = serve_step_inputs(sw)
            sq, sk, svc, svn, scb, ssg = (t.to(dev) for t in (ci.q, ci.k, ci.v_codes, ci.v_norms, ci.codebook,
                                                              ci.signs))
            skn, svn_new = kn_h.to(dev), vn_h.to(dev)
            del ci.k, ci.v_codes
            sout = torch.empty((ci.n_queries, ci.n_q_heads, ci.head_dim), dtype=torch.float32, device=dev)
            s_sid = np.asarray(ci.slot_ids, dtype=np.int32)
            s_pos = np.asarray(ci.positions, dtype=np.int32)

            def serve_call(st=None):
                st = st or stream
                binding.attn_kv_append_cb(skn, svn_new, sk, svc, svn, ssg, scb, sw.bits, s_sid, s_pos, ci.n_queries,
                                          ci.n_cache_slots, ci.capacity, ci.ring, ci.n_kv_heads, ci.head_dim,
                                          stream=st)
                binding.attn_decode_cache_cb(sq, sk, svc, svn, scb, sw.bits, s_sid, s_pos, ci.n_queries,
                                             ci.n_cache_slots, ci.capacity, ci.ring, 0, sout, ci.n_q_heads,
                                             ci.n_kv_heads, ci.head_dim, ci.scale, stream=st)
                binding.attn_fwht_undo(sout, ssg, sout, stream=st)

            def per_call_us(fn, n):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(n):
                    fn()
                torch.cuda.synchronize()
                return (time.perf_counter() - t0) * 1e6 / n

            for _ in range(3):
                serve_call()
            d, B = ci.head_dim, min(ci.head_dim, 256)
            att = sum(cache_attended(p, ci.capacity, ci.ring, 0) for p in ci.positions)
            nb = att * ci.n_kv_heads * (2 * d + d + 4 * (d // B))   # K fp16 + codes + norms read
            warm = statistics.median(per_call_us(serve_call, args.reps) for _ in range(3))
            g_us = graph_us_per_call(lambda st: serve_call(st=st))
            assert torch.isfinite(sout).all().item(), "non-finite output"
            per.append({
                "workload": sw.name, "window": 0, "kv_bytes": nb,
                "step": "attn_kv_append_cb + attn_decode_cache_cb + attn_fwht_undo",
                "warm_us_per_call": round(warm, 2),
                "warm_gbs": round(nb / (warm * 1e-6) / 1e9, 1),
                "warm_hbm_frac": round(nb / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "graph_us_per_call": round(g_us, 2),
                "graph_gbs": round(nb / (g_us * 1e-6) / 1e9, 1),
            })
            print(f"[bench] {sw.name}: warm {warm:.2f} us, graph {g_us:.2f} us ({per[-1]['graph_gbs']} GB/s)",
                  file=sys.stderr, flush=True)
            del sq, sk, svc, svn, scb, ssg, skn, svn_new, sout
            torch.cuda.empty_cache()
        # KV append presets (attn_kv_append): bytes = fp32 K and V read + fp16 K and V (+ scales) written
        for aw in APPEND_WORKLOADS:
            d = aw.head_dim
            n_el = aw.n_rows * aw.n_kv_heads * d
            cache_el = aw.n_cache_slots * aw.n_kv_heads * aw.capacity * d
            kc = torch.zeros(cache_el, dtype=torch.float16, device=dev)
            vc = torch.zeros(cache_el, dtype=torch.int8 if aw.v_int8 else torch.float16, device=dev)
            sc = torch.zeros(cache_el // 32, dtype=torch.float16, device=dev) if aw.v_int8 else None
            kn, vn = (t.to(dev) for t in append_new_rows(aw))
            a_sid = np.asarray(aw.slot_ids, dtype=np.int32)
            a_pos = np.asarray(aw.positions, dtype=np.int32)

            def append_call(st=None):
                binding.attn_kv_append(kn, vn, kc, vc, sc, a_sid, a_pos, aw.n_rows,
                                       aw.n_cache_slots, aw.capacity, aw.ring, aw.n_kv_heads, d,
                                       stream=st or stream)

            def per_call_us(fn, n):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(n):
                    fn()
                torch.cuda.synchronize()
                return (time.perf_counter() - t0) * 1e6 / n

            for _ in range(3):
                append_call()
            nb = n_el * 8 + n_el * (2 + (1 + 2 / 32 if aw.v_int8 else 2))
            warm = statistics.median(per_call_us(append_call, args.reps) for _ in range(3))
            g_us = graph_us_per_call(lambda st: append_call(st=st))
            per.append({
                "workload": aw.name, "window": 0, "bytes": int(nb),
                "warm_us_per_call": round(warm, 2),
                "warm_gbs": round(nb / (warm * 1e-6) / 1e9, 1),
                "warm_hbm_frac": round(nb / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "graph_us_per_call": round(g_us, 2),
                "graph_gbs": round(nb / (g_us * 1e-6) / 1e9, 1),
                "graph_hbm_frac": round(nb / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            })
            print(f"[bench] {aw.name}: warm {warm:.2f} us ({per[-1]['warm_gbs']} GB/s), graph {g_us:.2f} us "
                  f"({per[-1]['graph_gbs']} GB/s)", file=sys.stderr, flush=True)
            del kc, vc, sc, kn, vn
            torch.cuda.empty_cache()
        result["per_config"] = per

    # ---- CPU fp64 oracle on a bounded sample of the headline workload
    if not args.quick and not args.no_cpu_baseline and args.workload in by_name:
        from oracle import oracle_attn_decode
        threads = len(os.sched_getaffinity(0))
        n_sample_slots = inp.n_slots
        rows = list(range(n_sample_slots * inp.n_q_heads))
        print(f"[bench] cpu oracle on {len(rows)} rows with {threads} threads", file=sys.stderr, flush=True)
        qn, kn, vn = inp.q.numpy(), inp.k.numpy(), inp.v.numpy()
        sn = None if inp.v_scales is None else inp.v_scales.numpy()
        t0 = time.perf_counter()
        oracle_attn_decode(qn, kn, vn, sn, inp.seq_lens, window, inp.n_q_heads, inp.n_kv_heads,
                           inp.head_dim, inp.scale, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        sb = kv_bytes(inp.seq_lens[:n_sample_slots], window, inp.n_kv_heads, inp.head_dim, inp.v_int8)
        result["cpu_baseline"] = {
            "value": round(sb / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"all {n_sample_slots} slots of {cfg.name} "
                      f"({len(rows)} query rows, {sb} KV bytes), one pass, {dt:.2f} s wall",
        }

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
