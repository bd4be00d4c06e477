"""Seeded synthetic decode-attention inputs, shared by the tests and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the CPU oracle and the HIP path consume exactly
the tensors made here.

Recipe (one per workload):
  * ``torch.Generator('cpu').manual_seed(seed_base + t)`` with t = 1 for q,
    2 for K, 3 for V; the workload presets use ``seed_base = 1000 * index``.
  * Values are float32 N(0, 1) rounded to float16 (round-to-nearest-even).
  * K and V are drawn slot by slot, each slot as one ``[n_kv, L_s, D]`` block,
    and packed back to back (ragged, no padding): slot s starts at element
    ``sum_{t<s} n_kv * L_t * D``.
  * Block-int8 V: the float32 N(0, 1) draw is quantised per block of 32
    consecutive dims: ``scale = fp16(max|v| / 127)``,
    ``code = clamp(round_half_even(v / scale), -127, 127)``; an all-zero block
    gets scale 0 and codes 0.  Scales are laid out ``[slot][n_kv][L_s][D/32]``.
  * q is ``[n_slots, n_q, D]`` and the softmax scale is ``1/sqrt(D)`` in float32.

The presets are gemma-style decode shapes (16 query heads over 8 KV heads at
head_dim 256, contexts from 1K to 131K, several decode slots) as the pages
describe them (hf2q gemma4 batched_body.rs; tessl nn.rs decode tuning tables).
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Optional, Sequence, Tuple

import torch

QUANT_BLOCK = 32


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    index: int
    name: str
    description: str
    seq_lens: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    v_int8: bool
    windows: Tuple[int, ...] = (0,)

    @property
    def n_slots(self) -> int:
        return len(self.seq_lens)

    @property
    def seed_base(self) -> int:
        return 1000 * self.index


WORKLOADS = (
    WorkloadConfig(0, "single_d64_L256",
                   "1 slot, 1 q / 1 kv head, head_dim 64, KV length 256, fp16 K/V",
                   (256,), 1, 1, 64, False),
    WorkloadConfig(1, "gqa_d256_L4096",
                   "1 slot, 16 q / 8 kv heads, head_dim 256, KV length 4096, fp16 K/V",
                   (4096,), 16, 8, 256, False),
    WorkloadConfig(2, "ragged_4slot_d256",
                   "4 slots, KV lengths 1024/8192/32768/2000, 16 q / 8 kv, head_dim 256, fp16 K/V",
                   (1024, 8192, 32768, 2000), 16, 8, 256, False),
    WorkloadConfig(3, "hybrid_int8v_8x32768",
                   "8 slots x 32768, 16 q / 8 kv, head_dim 256, fp16 K, int8 V (blocks of 32, fp16 scales)",
                   (32768,) * 8, 16, 8, 256, True),
    WorkloadConfig(4, "long_131072_window1024",
                   "1 slot x 131072, 16 q / 8 kv, head_dim 256, fp16 K/V; full and last-1024 window",
                   (131072,), 16, 8, 256, False, (0, 1024)),
)


@dataclasses.dataclass
class DecodeInputs:
    """Host (CPU) tensors of one decode-attention call."""
    q: torch.Tensor                    # float16 [n_slots, n_q, D]
    k: torch.Tensor                    # float16 packed [sum_s n_kv*L_s*D]
    v: torch.Tensor                    # float16 or int8, same layout as k
    v_scales: Optional[torch.Tensor]   # float16 [sum_s n_kv*L_s*D/32] or None
    seq_lens: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float

    @property
    def n_slots(self) -> int:
        return len(self.seq_lens)

    @property
    def v_int8(self) -> bool:
        return self.v_scales is not None


def quantize_int8_blocks(v32: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Symmetric int8 per block of 32 along the last dim (input generation only)."""
    d = v32.shape[-1]
    if d % QUANT_BLOCK:
        raise ValueError("head_dim must be a multiple of 32 for block-int8 V")
    blocks = v32.reshape(*v32.shape[:-1], d // QUANT_BLOCK, QUANT_BLOCK)
    amax = blocks.abs().amax(dim=-1)
    scale16 = (amax / 127.0).to(torch.float16)
    scale32 = scale16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(scale32 == 0, torch.ones_like(scale32), scale32)
    codes = torch.round(blocks / safe).clamp_(-127, 127)
    codes = torch.where(scale32 == 0, torch.zeros_like(codes), codes)
    return codes.to(torch.int8).reshape(v32.shape), scale16


def make_inputs(seq_lens: Sequence[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                v_int8: bool, seed_base: int, scale: Optional[float] = None) -> DecodeInputs:
    seq_lens = tuple(int(x) for x in seq_lens)
    n_slots = len(seq_lens)
    total_rows = sum(seq_lens) * n_kv_heads
    gq = torch.Generator("cpu").manual_seed(seed_base + 1)
    gk = torch.Generator("cpu").manual_seed(seed_base + 2)
    gv = torch.Generator("cpu").manual_seed(seed_base + 3)

    q = torch.randn((n_slots, n_q_heads, head_dim), generator=gq, dtype=torch.float32).to(torch.float16)
    k = torch.empty(total_rows * head_dim, dtype=torch.float16)
    if v_int8:
        v = torch.empty(total_rows * head_dim, dtype=torch.int8)
        vs = torch.empty(total_rows * head_dim // QUANT_BLOCK, dtype=torch.float16)
    else:
        v = torch.empty(total_rows * head_dim, dtype=torch.float16)
        vs = None
    off = 0
    for L in seq_lens:
        n = n_kv_heads * L * head_dim
        if n:
            kb = torch.randn((n_kv_heads, L, head_dim), generator=gk, dtype=torch.float32)
            k[off:off + n] = kb.reshape(-1).to(torch.float16)
            del kb
            vb = torch.randn((n_kv_heads, L, head_dim), generator=gv, dtype=torch.float32)
            if v_int8:
                codes, sc = quantize_int8_blocks(vb)
                v[off:off + n] = codes.reshape(-1)
                vs[off // QUANT_BLOCK:(off + n) // QUANT_BLOCK] = sc.reshape(-1)
            else:
                v[off:off + n] = vb.reshape(-1).to(torch.float16)
            del vb
        off += n
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))
    return DecodeInputs(q, k, v, vs, seq_lens, n_q_heads, n_kv_heads, head_dim, scale)


def workload_inputs(cfg: WorkloadConfig) -> DecodeInputs:
    return make_inputs(cfg.seq_lens, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                       cfg.v_int8, cfg.seed_base)


@dataclasses.dataclass
class CacheInputs:
    """Host tensors of one fixed-capacity-cache call (every cache row is filled)."""
    q: torch.Tensor                    # float16 [n_queries, n_q, D]
    k: torch.Tensor                    # float16 [n_cache_slots * n_kv * capacity * D]
    v: torch.Tensor                    # float16 or int8, same layout as k
    v_scales: Optional[torch.Tensor]   # float16 [n_cache_slots * n_kv * capacity * D/32] or None
    slot_ids: Tuple[int, ...]
    positions: Tuple[int, ...]
    n_cache_slots: int
    capacity: int
    ring: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float

    @property
    def n_queries(self) -> int:
        return len(self.slot_ids)


def make_cache_inputs(n_cache_slots: int, capacity: int, ring: int, slot_ids: Sequence[int],
                      positions: Sequence[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                      v_int8: bool, seed_base: int, scale: Optional[float] = None) -> CacheInputs:
    """A [slot][kv][capacity][D] cache with every row drawn (same recipe as make_inputs)."""
    slot_ids = tuple(int(x) for x in slot_ids)
    positions = tuple(int(x) for x in positions)
    base = make_inputs((capacity,) * n_cache_slots, n_q_heads, n_kv_heads, head_dim, v_int8, seed_base, scale)
    gq = torch.Generator("cpu").manual_seed(seed_base + 4)
    q = torch.randn((len(slot_ids), n_q_heads, head_dim), generator=gq, dtype=torch.float32).to(torch.float16)
    return CacheInputs(q, base.k, base.v, base.v_scales, slot_ids, positions, n_cache_slots, capacity,
                       int(ring), n_q_heads, n_kv_heads, head_dim, base.scale)


@dataclasses.dataclass(frozen=True)
class CacheWorkloadConfig:
    """A fixed-capacity-cache call: query rows (slot id, position) over a [slot][kv][capacity][D] cache."""
    index: int
    name: str
    description: str
    n_cache_slots: int
    capacity: int
    ring: int
    slot_ids: Tuple[int, ...]
    positions: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    v_int8: bool
    window: int = 0

    @property
    def seed_base(self) -> int:
        return 1000 * self.index


CACHE_WORKLOADS = (
    CacheWorkloadConfig(10, "ring1024_8slot_d256",
                        "sliding-window layer: 8 slots, a 1024-row ring each, tokens deep into long contexts",
                        8, 1024, 1, tuple(range(8)), (131071, 90000, 50001, 77777, 2047, 300000, 1024, 65536),
                        16, 8, 256, False),
    CacheWorkloadConfig(11, "verify4x4_linear32768_d256",
                        "speculative verify: 4 slots x 4 consecutive draft positions over a 32768-row linear cache",
                        4, 32768, 0, tuple(s for s in range(4) for _ in range(4)),
                        tuple(32764 + t for _ in range(4) for t in range(4)), 16, 8, 256, False),
    # the hybrid regime's bytes (1.64 GB) as a serving batch of 128 sequences on a sliding-window layer:
    # one query per slot, each attending its ring's 2048 rows (one launch, the large query table)
    CacheWorkloadConfig(12, "batch128_ring2048_d256_int8",
                        "serving batch: 128 slots, a 2048-row ring each (int8 V), tokens deep into long contexts",
                        128, 2048, 1, tuple(range(128)), tuple(4096 + 997 * s for s in range(128)),
                        16, 8, 256, True),
)


def cache_workload_inputs(cfg: CacheWorkloadConfig) -> CacheInputs:
    return make_cache_inputs(cfg.n_cache_slots, cfg.capacity, cfg.ring, cfg.slot_ids, cfg.positions,
                             cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.v_int8, cfg.seed_base)


@dataclasses.dataclass(frozen=True)
class AppendWorkloadConfig:
    """A KV append: n_rows new tokens (fp32 K and V) written into a fixed-capacity cache."""
    index: int
    name: str
    description: str
    n_cache_slots: int
    capacity: int
    ring: int
    slot_ids: Tuple[int, ...]
    positions: Tuple[int, ...]
    n_kv_heads: int
    head_dim: int
    v_int8: bool

    @property
    def n_rows(self) -> int:
        return len(self.slot_ids)


APPEND_WORKLOADS = (
    AppendWorkloadConfig(20, "append_decode_8slot_d256_int8",
                         "one decode step: a new token for each of 8 slots (8 kv heads, head_dim 256, int8 V)",
                         8, 32768, 0, tuple(range(8)), (32767,) * 8, 8, 256, True),
    AppendWorkloadConfig(21, "append_4096tok_d256_int8",
                         "4096 consecutive tokens into one slot (8 kv heads, head_dim 256, int8 V)",
                         1, 32768, 0, (0,) * 4096, tuple(range(4096)), 8, 256, True),
)


def append_new_rows(cfg: AppendWorkloadConfig) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 N(0, 1) K and V rows [n_rows, n_kv, D] (seeds seed_base + 5 and + 6)."""
    gk = torch.Generator("cpu").manual_seed(1000 * cfg.index + 5)
    gv = torch.Generator("cpu").manual_seed(1000 * cfg.index + 6)
    shape = (cfg.n_rows, cfg.n_kv_heads, cfg.head_dim)
    return (torch.randn(shape, generator=gk, dtype=torch.float32),
            torch.randn(shape, generator=gv, dtype=torch.float32))


# ----------------------------------------------------------------------------
# Codebook V (the pages' hybrid format): V is stored rotated by a sign-flipped,
# normalised Walsh-Hadamard transform, as one byte per coordinate indexing a
# codebook, with one fp32 norm per block of min(D, 256) rotated coordinates
# (mlx-native flash_attn_vec_hybrid.metal: header layouts, the codebook
# dequant, the per-block norms at D = 512; hf2q gemma4 batched_body.rs: the
# FWHT-undo of the attention output).  Everything below is input generation.

CB_BLOCK = 256


# The codebooks the pages' hybrid V uses: mlx-native 0.21.1 flash_attn_vec_hybrid.metal prints
# three fixed tables of N(0, 1) levels, CODEBOOK_HB_5BIT, _6BIT and _8BIT, which its codebook
# dequant (dequant_hb_single, dequant_hb_float4) indexes with the low 5 or 6 bits of a byte, or
# the whole byte at 8 bits.  Transcribed here level by level, as float32 literals, in table order.
PAGE_CODEBOOKS = {
    5: (
        -3.2606790, -2.6910589, -2.3176743, -2.0286608, -1.7871646, -1.5761599, -1.3862739, -1.2117410,
        -1.0487242, -0.8945114, -0.7470884, -0.6048936, -0.4666676, -0.3313550, -0.1980377, -0.0658849,
        0.0658849, 0.1980377, 0.3313550, 0.4666676, 0.6048936, 0.7470884, 0.8945114, 1.0487242,
        1.2117410, 1.3862739, 1.5761599, 1.7871646, 2.0286608, 2.3176743, 2.6910589, 3.2606790,
    ),
    6: (
        -3.6996161, -3.1907215, -2.8640626, -2.6161277, -2.4129324, -2.2388464, -2.0853192, -1.9471373,
        -1.8208742, -1.7041502, -1.5952401, -1.4928497, -1.3959804, -1.3038428, -1.2157998, -1.1313277,
        -1.0499889, -0.9714118, -0.8952766, -0.8213046, -0.7492492, -0.6788902, -0.6100285, -0.5424819,
        -0.4760822, -0.4106724, -0.3461048, -0.2822386, -0.2189392, -0.1560761, -0.0935225, -0.0311537,
        0.0311537, 0.0935225, 0.1560761, 0.2189392, 0.2822386, 0.3461048, 0.4106724, 0.4760822,
        0.5424819, 0.6100285, 0.6788902, 0.7492492, 0.8213046, 0.8952766, 0.9714118, 1.0499889,
        1.1313277, 1.2157998, 1.3038428, 1.3959804, 1.4928497, 1.5952401, 1.7041502, 1.8208742,
        1.9471373, 2.0853192, 2.2388464, 2.4129324, 2.6161277, 2.8640626, 3.1907215, 3.6996161,
    ),
    8: (
        -5.0652659, -4.6836997, -4.4467193, -4.2715508, -4.1311907, -4.0132856, -3.9111092, -3.8205780,
        -3.7390194, -3.6645851, -3.5959415, -3.5320936, -3.4722785, -3.4158977, -3.3624729, -3.3116156,
        -3.2630056, -3.2163758, -3.1715011, -3.1281899, -3.0862780, -3.0456229, -3.0061011, -2.9676040,
        -2.9300362, -2.8933131, -2.8573596, -2.8221086, -2.7874999, -2.7534795, -2.7199985, -2.6870129,
        -2.6544825, -2.6223710, -2.5906452, -2.5592748, -2.5282321, -2.4974918, -2.4670306, -2.4368270,
        -2.4068614, -2.3771157, -2.3475732, -2.3182184, -2.2890372, -2.2600165, -2.2311440, -2.2024086,
        -2.1737998, -2.1453081, -2.1169245, -2.0886408, -2.0604493, -2.0323430, -2.0043154, -1.9763603,
        -1.9484722, -1.9206458, -1.8928763, -1.8651592, -1.8374904, -1.8098662, -1.7822828, -1.7547372,
        -1.7272261, -1.6997469, -1.6722970, -1.6448739, -1.6174755, -1.5900996, -1.5627445, -1.5354084,
        -1.5080897, -1.4807869, -1.4534986, -1.4262237, -1.3989610, -1.3717093, -1.3444678, -1.3172356,
        -1.2900118, -1.2627956, -1.2355865, -1.2083838, -1.1811868, -1.1539951, -1.1268081, -1.0996255,
        -1.0724469, -1.0452718, -1.0180999, -0.9909310, -0.9637647, -0.9366008, -0.9094390, -0.8822793,
        -0.8551212, -0.8279648, -0.8008098, -0.7736561, -0.7465035, -0.7193520, -0.6922014, -0.6650517,
        -0.6379027, -0.6107544, -0.5836067, -0.5564596, -0.5293129, -0.5021667, -0.4750208, -0.4478753,
        -0.4207301, -0.3935852, -0.3664405, -0.3392960, -0.3121517, -0.2850076, -0.2578636, -0.2307198,
        -0.2035761, -0.1764324, -0.1492888, -0.1221453, -0.0950019, -0.0678584, -0.0407151, -0.0135717,
        0.0135717, 0.0407151, 0.0678584, 0.0950019, 0.1221453, 0.1492888, 0.1764324, 0.2035761,
        0.2307198, 0.2578636, 0.2850076, 0.3121517, 0.3392960, 0.3664405, 0.3935852, 0.4207301,
        0.4478753, 0.4750208, 0.5021667, 0.5293129, 0.5564596, 0.5836067, 0.6107544, 0.6379027,
        0.6650517, 0.6922014, 0.7193520, 0.7465035, 0.7736561, 0.8008098, 0.8279648, 0.8551212,
        0.8822793, 0.9094390, 0.9366008, 0.9637647, 0.9909310, 1.0180999, 1.0452718, 1.0724469,
        1.0996255, 1.1268081, 1.1539951, 1.1811868, 1.2083838, 1.2355865, 1.2627956, 1.2900118,
        1.3172356, 1.3444678, 1.3717093, 1.3989610, 1.4262237, 1.4534986, 1.4807869, 1.5080897,
        1.5354084, 1.5627445, 1.5900996, 1.6174755, 1.6448739, 1.6722970, 1.6997469, 1.7272261,
        1.7547372, 1.7822828, 1.8098662, 1.8374904, 1.8651592, 1.8928763, 1.9206458, 1.9484722,
        1.9763603, 2.0043154, 2.0323430, 2.0604493, 2.0886408, 2.1169245, 2.1453081, 2.1737998,
        2.2024086, 2.2311440, 2.2600165, 2.2890372, 2.3182184, 2.3475732, 2.3771157, 2.4068614,
        2.4368270, 2.4670306, 2.4974918, 2.5282321, 2.5592748, 2.5906452, 2.6223710, 2.6544825,
        2.6870129, 2.7199985, 2.7534795, 2.7874999, 2.8221086, 2.8573596, 2.8933131, 2.9300362,
        2.9676040, 3.0061011, 3.0456229, 3.0862780, 3.1281899, 3.1715011, 3.2163758, 3.2630056,
        3.3116156, 3.3624729, 3.4158977, 3.4722785, 3.5320936, 3.5959415, 3.6645851, 3.7390194,
        3.8205780, 3.9111092, 4.0132856, 4.1311907, 4.2715508, 4.4467193, 4.6836997, 5.0652659,
    ),
}


def codebook_levels(bits: int) -> torch.Tensor:
    """The V codebook (float32, ascending) that the presets and tests use for ``bits``: the
    pages' printed table at 5, 6 and 8 bits (PAGE_CODEBOOKS); at other widths, which the pages
    do not use, a Lloyd iteration computed here (lloyd_max_gaussian)."""
    if int(bits) in PAGE_CODEBOOKS:
        return torch.tensor(PAGE_CODEBOOKS[int(bits)], dtype=torch.float32)
    return lloyd_max_gaussian(bits)


@functools.lru_cache(maxsize=None)
def _lloyd_levels(bits: int, iters: int) -> Tuple[float, ...]:
    import numpy as np
    from scipy.stats import norm
    n = 1 << bits
    c = norm.ppf((np.arange(n) + 0.5) / n)
    for _ in range(iters):
        b = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
        mass = norm.cdf(b[1:]) - norm.cdf(b[:-1])
        c = (norm.pdf(b[:-1]) - norm.pdf(b[1:])) / mass
    return tuple(float(x) for x in c)


def lloyd_max_gaussian(bits: int, iters: int = 2000) -> torch.Tensor:
    """Lloyd-Max levels for N(0, 1), computed here, with 2**bits levels (float32, ascending),
    an alternative to the pages' printed tables and the levels of the widths they do not print.

    Lloyd's iteration from the quantile midpoints: cell boundaries at the
    midpoints of neighbouring levels, each level moved to the conditional mean
    of N(0, 1) on its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  It
    converges slowly for many levels: after 2000 steps the levels are within
    2e-4 of the fixed point at 8 bits and within 1e-6 at 5 bits.
    """
    return torch.tensor(_lloyd_levels(int(bits), int(iters)), dtype=torch.float32)


def fwht_rows(x: torch.Tensor) -> torch.Tensor:
    """Unnormalised Walsh-Hadamard transform along the last dim (a power of two), float64."""
    y = x.to(torch.float64).clone()
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a, b = y[..., 0, :], y[..., 1, :]
        y = torch.stack((a + b, a - b), dim=-2).reshape(*y.shape[:-3], d)
        h *= 2
    return y


def make_signs(head_dim: int, seed: int) -> torch.Tensor:
    """A seeded +-1 vector (as fp32) of length head_dim."""
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randint(0, 2, (head_dim,), generator=g) * 2 - 1).to(torch.float32)


def codebook_quantize(v: torch.Tensor, signs: torch.Tensor, codebook: torch.Tensor):
    """Rotate rows of v ([..., D] fp32) by fwht(signs * v) / sqrt(D), then encode them
    (codebook_encode_rotated).  Returns (uint8 indices [..., D], fp32 norms [..., D / B])."""
    d = v.shape[-1]
    rot = (fwht_rows(v.to(torch.float64) * signs.to(torch.float64)) / math.sqrt(d)).to(torch.float32)
    return codebook_encode_rotated(rot, codebook)


def codebook_encode_rotated(rot: torch.Tensor, codebook: torch.Tensor):
    """Per block of B = min(D, 256) coordinates of already rotated rows: norm = ||block||
    (fp32), index = nearest level to x * sqrt(B) / norm."""
    d = rot.shape[-1]
    B = min(d, CB_BLOCK)
    blocks = rot.reshape(*rot.shape[:-1], d // B, B)
    norms = blocks.to(torch.float64).pow(2).sum(-1).sqrt().to(torch.float32)
    safe = torch.where(norms == 0, torch.ones_like(norms), norms)
    u = blocks * (math.sqrt(B) / safe).unsqueeze(-1)
    idx = torch.bucketize(u.contiguous(), (codebook[1:] + codebook[:-1]) / 2)
    return idx.to(torch.uint8).reshape(rot.shape), norms


@dataclasses.dataclass
class CodebookInputs:
    """Host tensors of a packed-slot call with codebook V (the pages' hybrid KV regime)."""
    q: torch.Tensor            # float16 [n_slots, n_q, D]
    k: torch.Tensor            # float16 packed [sum_s n_kv*L_s*D]
    v_codes: torch.Tensor      # uint8 packed like k (indices into the codebook)
    v_norms: torch.Tensor      # float32 [sum_s n_kv*L_s*D/B], B = min(D, 256)
    codebook: torch.Tensor     # float32 [2**bits]
    codebook_bits: int
    signs: torch.Tensor        # float32 +-1 [D]: the rotation's sign flips
    seq_lens: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float
    v_plain: Optional[torch.Tensor] = None   # float32 packed like k: V before rotation (on request)

    @property
    def n_slots(self) -> int:
        return len(self.seq_lens)


def make_codebook_inputs(seq_lens: Sequence[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                         bits: int, seed_base: int, keep_plain: bool = False,
                         direct: bool = False) -> CodebookInputs:
    """K and q as make_inputs; V drawn N(0, 1) (seed_base + 3), rotated and codebook-quantised.
    keep_plain also returns V itself (float32), for checks of the whole encode / attend / undo chain.
    direct draws the rotated coordinates themselves: an orthogonal rotation of i.i.d. N(0, 1)
    coordinates is again i.i.d. N(0, 1), so codes and norms have the same distribution, without
    the transform's cost at full cache sizes (and with no plain V to keep)."""
    if direct and keep_plain:
        raise ValueError("direct draws no plain V")
    base = make_inputs(seq_lens, n_q_heads, n_kv_heads, head_dim, False, seed_base)
    cb = codebook_levels(bits)
    signs = make_signs(head_dim, seed_base + 7)
    gv = torch.Generator("cpu").manual_seed(seed_base + 3)
    B = min(head_dim, CB_BLOCK)
    total = sum(seq_lens) * n_kv_heads
    codes = torch.empty(total * head_dim, dtype=torch.uint8)
    norms = torch.empty(total * head_dim // B, dtype=torch.float32)
    plain = torch.empty(total * head_dim, dtype=torch.float32) if keep_plain else None
    off = 0
    for L in seq_lens:
        n = n_kv_heads * L
        for r0 in range(0, n, 1 << 16):          # bounded temporaries at full cache sizes
            r1 = min(n, r0 + (1 << 16))
            vb = torch.randn((r1 - r0, head_dim), generator=gv, dtype=torch.float32)
            c, nr = codebook_encode_rotated(vb, cb) if direct else codebook_quantize(vb, signs, cb)
            a = off + r0
            codes[a * head_dim:(a + r1 - r0) * head_dim] = c.reshape(-1)
            norms[a * head_dim // B:(a + r1 - r0) * head_dim // B] = nr.reshape(-1)
            if plain is not None:
                plain[a * head_dim:(a + r1 - r0) * head_dim] = vb.reshape(-1)
        off += n
    return CodebookInputs(base.q, base.k, codes, norms, cb, bits, signs, tuple(int(x) for x in seq_lens),
                          n_q_heads, n_kv_heads, head_dim, base.scale, plain)


@dataclasses.dataclass(frozen=True)
class CodebookWorkloadConfig:
    """A packed-slot workload with codebook V (byte indices, Lloyd-Max levels, block norms)."""
    name: str
    index: int
    seq_lens: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    bits: int
    window: int = 0

    @property
    def seed_base(self) -> int:
        return 1000 * self.index


CODEBOOK_WORKLOADS = (
    # the hybrid workload's shape with the pages' own V format (8-bit levels, D 256 sliding layers)
    CodebookWorkloadConfig("hybrid_codebook8_8x32768", 30, (32768,) * 8, 16, 8, 256, 8),
    # a global layer: head_dim 512 with 2 KV heads (gemma4's global layers), two norms per row
    CodebookWorkloadConfig("global_d512_codebook8_8x32768", 31, (32768,) * 8, 16, 2, 512, 8),
)


def codebook_workload_inputs(cfg: CodebookWorkloadConfig) -> CodebookInputs:
    return make_codebook_inputs(cfg.seq_lens, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.bits,
                                cfg.seed_base, direct=True)


@dataclasses.dataclass
class CacheCodebookInputs:
    """Host tensors of a fixed-capacity-cache call with codebook V."""
    q: torch.Tensor            # float16 [n_queries, n_q, D]
    k: torch.Tensor            # float16 [n_cache_slots * n_kv * capacity * D]
    v_codes: torch.Tensor      # uint8, laid out like k
    v_norms: torch.Tensor      # float32 [n_cache_slots * n_kv * capacity * D / B], B = min(D, 256)
    codebook: torch.Tensor     # float32 [2**bits]
    codebook_bits: int
    signs: torch.Tensor        # float32 +-1 [D]
    slot_ids: Tuple[int, ...]
    positions: Tuple[int, ...]
    n_cache_slots: int
    capacity: int
    ring: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    scale: float

    @property
    def n_queries(self) -> int:
        return len(self.slot_ids)


def make_cache_codebook_inputs(n_cache_slots: int, capacity: int, ring: int, slot_ids: Sequence[int],
                               positions: Sequence[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
                               bits: int, seed_base: int) -> CacheCodebookInputs:
    """A [slot][kv][capacity][D] cache with codebook V: the packed recipe of make_codebook_inputs
    with every slot holding `capacity` rows (the same layout), rotated coordinates drawn directly;
    q per query row as make_cache_inputs draws it."""
    ci = make_codebook_inputs((capacity,) * n_cache_slots, n_q_heads, n_kv_heads, head_dim, bits, seed_base,
                              direct=True)
    gq = torch.Generator("cpu").manual_seed(seed_base + 4)
    q = torch.randn((len(slot_ids), n_q_heads, head_dim), generator=gq, dtype=torch.float32).to(torch.float16)
    return CacheCodebookInputs(q, ci.k, ci.v_codes, ci.v_norms, ci.codebook, bits, ci.signs,
                               tuple(int(x) for x in slot_ids), tuple(int(x) for x in positions), n_cache_slots,
                               capacity, int(ring), n_q_heads, n_kv_heads, head_dim, ci.scale)


@dataclasses.dataclass(frozen=True)
class ServeStepWorkloadConfig:
    """One decode step of the hybrid regime on a fixed-capacity codebook-V cache: append each
    query's new token (K fp16, V codebook-encoded), attend from it, undo the rotation."""
    index: int
    name: str
    description: str
    n_cache_slots: int
    capacity: int
    ring: int
    slot_ids: Tuple[int, ...]
    positions: Tuple[int, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    bits: int

    @property
    def seed_base(self) -> int:
        return 1000 * self.index


SERVE_STEP_WORKLOADS = (
    ServeStepWorkloadConfig(40, "serve_step_codebook8_8x32768_d256",
                            "8 slots, each appending its token 32768 and attending 0..32767 (linear cache)",
                            8, 32768, 0, tuple(range(8)), (32767,) * 8, 16, 8, 256, 8),
    ServeStepWorkloadConfig(41, "serve_step_codebook8_ring1024_d256",
                            "8 slots on 1024-row rings, tokens deep into long contexts",
                            8, 1024, 1, tuple(range(8)), (131071, 90000, 50001, 77777, 2047, 300000, 1024, 65536),
                            16, 8, 256, 8),
)


def serve_step_inputs(cfg: ServeStepWorkloadConfig):
    """The cache (make_cache_codebook_inputs) and the step's new fp32 K and V rows [n_queries, n_kv, D]
    (seeds seed_base + 5 and + 6)."""
    ci = make_cache_codebook_inputs(cfg.n_cache_slots, cfg.capacity, cfg.ring, cfg.slot_ids, cfg.positions,
                                    cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.bits, cfg.seed_base)
    gk = torch.Generator("cpu").manual_seed(cfg.seed_base + 5)
    gv = torch.Generator("cpu").manual_seed(cfg.seed_base + 6)
    shape = (len(cfg.slot_ids), cfg.n_kv_heads, cfg.head_dim)
    return ci, torch.randn(shape, generator=gk, dtype=torch.float32), torch.randn(shape, generator=gv,
                                                                                    dtype=torch.float32)
