// attn_decode_kernels.hpp -- gfx950 (CDNA4, wave64) kernels of split-KV decode attention.
//
// Two kernels, the FlashDecoding pair the pages describe (tessl nn.rs,
// flash_attn_decode: a partial pass over KV chunks and a reduce pass; mlx-native
// flash_attn_vec_hybrid.metal: per-split partial O plus (S, M) and a
// log-sum-exp merge):
//
//  * attn_partial_kernel: one workgroup (4 waves) per (slot, kv head, chunk of
//    positions, block of GB query heads).  Every query head of the block
//    shares the K and V rows the workgroup streams, so each byte of the chunk
//    is read from HBM once for all of them (the GQA grouping of mlx-native's
//    flash_attn_vec_hybrid_batched_gqa_impl; tessl's DecodeHeadBlock::Group).
//    A row is read by R = head_dim/16 lanes with 16-byte non-temporal loads (a wave loads
//    64/R consecutive rows per instruction, fully coalesced); the QK dot uses
//    v_dot2_f32_f16 on the fp16 pairs and an all-reduce over the R lanes made
//    of DPP row ops (quad_perm, row_half_mirror, row_mirror) plus one swizzle
//    at R = 32.  Each lane group keeps its own fp32 online softmax (running
//    max M and sum S in the log2 domain) and accumulates its 16 output dims;
//    at the end the lane groups are merged with cross-lane shuffles and the
//    4 waves through LDS.  A slot with one chunk writes out = O / S directly
//    (S == 0, an empty slot, writes zeros); otherwise O and (M, S) go to the
//    workspace.
//  * the log-sum-exp merge of a split slot's chunks, per (slot, query head,
//    64-dim slice): M* = max_c M_c, S* = sum_c S_c 2^(M_c - M*),
//    out = sum_c O_c 2^(M_c - M*) / S*.  Either in attn_combine_kernel, a
//    second launch, or (single-launch merge) in extra workgroups at the end of
//    the partial kernel's own grid, which read the chunks' partials as
//    self-validating flagged pairs (tail_merge).
//
// The logits are kept in the log2 domain (scale * log2 e folded into the
// scale), so every exponential is one v_exp_f32; exp(x - m) = 2^((x - m) log2 e).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "planner.hpp"  // kMaxSlotsPerLaunch, shared with the host planner

namespace attn_decode_impl {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// One query row of a launch (a decode slot, or one query of a cache call).
struct SlotDesc {
    int64_t kv_row0;    // row of (slot, kv head 0, position-row 0) in the K / V arrays
    int64_t part_row0;  // first plain partial row of the query, -1 when it has none
    int32_t L;          // one past the last attended position
    int32_t lo;         // first attended position
    int32_t chunk;      // positions per chunk
    int32_t n_chunks;   // chunks of the query
    int32_t item_begin; // first partial workgroup of the query in this launch
    int32_t comb_begin; // first merge row of the query in this launch (combine kernel, or the
                        // merge workgroups at the end of a single-launch grid)
    int32_t flag_row0;  // first flagged partial row of the query when its chunks are merged in
                        // the partial kernel's launch (single-launch merge), else -1
    int32_t slot_idx;   // index of the query row in the call (q / out rows)
    int32_t kv_stride;  // rows between consecutive kv heads
    int32_t ring_cap;   // ring capacity, INT32_MAX when rows do not wrap
    int32_t ring_base;  // position held by row 0 of the current ring lap (multiple of ring_cap)
    int16_t group_n;    // on a group leader: queries in the group (leader first), else 0
    int16_t lead_off;   // table entries back to the group leader (0 on the leader)
};
static_assert(sizeof(SlotDesc) == 64, "query descriptor layout");

// Formats of the V cache.
enum VFormat : int {
    kVF16 = 0,   // fp16 values
    kVI8 = 1,    // int8 codes, one fp16 scale per 32 dims
    kVCB = 2,    // byte indices into a codebook, one fp32 norm per block of min(D, 256) dims
};

// The kernel arguments.  A workgroup cannot start its loads before it has found
// its query: it reads the table size and searches the keys, each read a scalar
// load that waits for the previous one, and the scalar cache is empty when a
// kernel starts.  So those reads sit together at the front (the first 64-byte
// line holds the sizes and the first 12 keys; a search over up to 12 entries
// misses once), and every query descriptor fills exactly one line.
// NS is the table's capacity: kSmallTableSlots (3.4 KB of arguments) for launches
// of up to 48 query rows, kMaxSlotsPerLaunch (18.5 KB) for larger ones, so a batch
// of up to 256 rows is one launch while a small call copies only the small table.
template <int NS>
struct alignas(64) LaunchArgsT {
    int32_t n_slots;        // slots in this launch (table entries, longest chunks first)
    int32_t n_items;        // partial-kernel workgroups of this launch
    int32_t n_sub;          // G / GB
    int32_t G;              // query heads per kv head
    int32_t key[NS];        // per entry, non-decreasing: its first work item (partial
                            // kernels) or its first combine row (combine kernel)
    int32_t tkey[NS];       // partial kernels, per entry, non-decreasing: its first row
                            // among the merge workgroups at the end of the grid
    const uint16_t *q;      // fp16 [n_slots_total][n_q][D]
    const uint16_t *k;      // fp16 packed cache
    const void *v;          // fp16, int8 or codebook-index cache
    const void *vs;         // int8: fp16 block scales; codebook: fp32 block norms; fp16: null
    const float *codebook;  // codebook levels [cb_mask + 1], codebook V only
    float *out;             // fp32 [n_slots_total][n_q][D]
    float *ws_o;            // partial O rows [part_rows][D]
    float *ws_ml;           // partial (M, S) [part_rows][2]
    uint64_t *flags;        // flagged partial rows of single-launch merges, zero between calls
    int32_t cb_mask;        // codebook V: 2^bits - 1 (the index bits that are used)
    int32_t n_q;
    float scale_log2;       // scale * log2(e)
    float cb_scale;         // codebook V: 1 / sqrt(min(D, 256))
    alignas(64) SlotDesc slot[NS];
};
static_assert(offsetof(LaunchArgsT<kSmallTableSlots>, key) == 16 &&
              offsetof(LaunchArgsT<kSmallTableSlots>, slot) % 64 == 0 &&
              offsetof(LaunchArgsT<kMaxSlotsPerLaunch>, slot) % 64 == 0, "argument layout");

// ---------------------------------------------------------------- helpers

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of R lanes (R a power of two, 2..32); every lane gets the sum.
template <int R>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (R >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (R >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (R >= 8) x += dpp<0x141>(x);   // row_half_mirror: the other quad of the 8
    if constexpr (R >= 16) x += dpp<0x140>(x);  // row_mirror: the other 8 of the 16-lane row
    if constexpr (R >= 32)                      // swizzle, bit mode: lane ^ 16 within 32
        x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
    return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, shfl_xor_f32(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += shfl_xor_f32(x, off);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load: each KV byte is used once, so it is marked non-temporal.
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }

// Largest i in [0, n) with key(i) <= x, given key(0) <= x and key non-decreasing.
template <typename F>
__device__ __forceinline__ int upper_index(int n, int x, F key) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (key(mid) <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD
// b mod 8) and each XCD has its own L2.  The n_sub head blocks of one chunk
// read the same K and V rows, so they get workgroup ids b, b + 8, b + 16, ...:
// the same XCD, dispatched close together, so the reads after the first are
// served by that XCD's L2.  Maps a workgroup id to its work item; a
// permutation of [0, n_items) (the tail that does not fill 8 * n_sub ids is
// left in place).
__device__ __forceinline__ int xcd_item(int b, int n_items, int n_sub) {
    if (n_sub == 1) return b;
    const int z = 8 * n_sub;
    if (b >= (n_items / z) * z) return b;
    const int grp = b / z;
    const int rem = b - grp * z;
    return (grp * 8 + (rem & 7)) * n_sub + (rem >> 3);
}

// ---------------------------------------------------------------- chunk merge

// Dims of one output row merged by one wave: lane l owns dim slice * 64 + l.
constexpr int kCombineDims = 64;
static_assert(kCombineDims == kMergeSliceDims, "one merge slice per flagged block");
static_assert(kWaves == kMergeSlicesPerGroup, "a merge workgroup of the partial kernel: one slice per wave");
// Chunks whose partial values a merging wave loads before it uses them.
constexpr int kMergeBatch = 32;
// The combine kernel's workgroup: one wave.
constexpr int kCombineThreads = 64;

// x of lane `lane` (the same for every lane), through the LDS crossbar (no LDS
// allocation, no SGPR).
__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(lane << 2, __builtin_bit_cast(int, x)));
}

// Log-sum-exp merge of the sd.n_chunks partials of query head h (of the query
// whose descriptor is sd) for the 64 output dims of `slice`, by one wave:
//   M* = max_c M_c;
//   per block of 64 chunks, lane l takes chunk c0 + l: w = 2^(M_c - M*), and its
//   share of S* = fmaf(w, S_c, share); then every lane adds w_c O_c[its dim]
//   for the block's chunks in chunk order (w_c read from lane c - c0);
//   S* = the wave sum of the shares; out = acc / S* (S* == 0 gives zeros).
// Each partial row of the slice is one whole-wave load of 256 consecutive
// bytes.  The first kMergeBatch rows are loaded together with the statistics,
// so a merge of up to 32 chunks takes one memory round trip, and there is no
// LDS and no barrier.  tail_merge runs the same arithmetic in the same order.
template <int D, class Args>
__device__ __forceinline__ void merge_wave(const Args &args, const SlotDesc &sd, int h, int slice) {
    const int lane = threadIdx.x & 63;
    const int nc = sd.n_chunks;
    const int64_t base = sd.part_row0 + (int64_t)h * nc;
    const float *src = args.ws_o + base * D + slice * kCombineDims + lane;    // chunk c at src + c * D
    const float2 *ml = reinterpret_cast<const float2 *>(args.ws_ml) + base;   // chunk c's (M, S)

    // the first batch of partial values (indices past the last chunk re-read it; unused)
    float o[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) o[u] = src[(int64_t)min(u, nc - 1) * D];
    const float2 st0 = lane < nc ? ml[lane] : make_float2(-INFINITY, 0.f);

    float mloc = st0.x;
    for (int c = lane + 64; c < nc; c += 64) mloc = fmaxf(mloc, ml[c].x);
    const float mx = wave_max(mloc);
    const float ms = (mx == -INFINITY) ? 0.f : mx;

    float acc = 0.f, share = 0.f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        const float2 st = c0 == 0 ? st0 : (c < nc ? ml[c] : make_float2(-INFINITY, 0.f));
        const float w = c < nc ? fast_exp2(st.x - ms) : 0.f;
        share = fmaf(w, st.y, share);
        for (int b0 = 0; b0 < 64 && c0 + b0 < nc; b0 += kMergeBatch) {
            if (c0 + b0 > 0) {
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u) o[u] = src[(int64_t)min(c0 + b0 + u, nc - 1) * D];
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u)
                if (c0 + b0 + u < nc) acc = fmaf(lane_value(w, b0 + u), o[u], acc);
        }
    }
    const float lsum = wave_sum(share);
    args.out[((int64_t)sd.slot_idx * args.n_q + h) * D + slice * kCombineDims + lane] =
        (lsum == 0.f) ? 0.f : acc / lsum;
}

// Single-launch merge.  The workgroups past the n_items partial workgroups of a
// launch merge, in the same launch, the split queries' heads, each wave one
// 64-dim slice of one query head (a workgroup takes up to four slices of a
// head), as soon as every chunk of it has been written.
//
// Publication needs no wait.  A fused query's partial workgroup writes each
// value as one 8-byte pair {value bits, 1} with an agent-scope store (on
// gfx942/gfx950 such stores go through to the memory side of the per-XCD L2
// caches); per 64-dim slice of a partial row, a block of kFlagPairsPerSlice
// pairs holds the 64 value pairs, then the pairs of M and S.  An aligned 8-byte
// access is single-copy atomic, so a pair whose flag reads 1 holds the value
// that came with that flag: each pair validates itself, whatever order the
// stores arrive in (the protocol of RCCL's "LL" transfers).  The workgroup ends
// without waiting for any of it.
//
// Lane 0 of the merging wave first polls a single pair, the M of the last chunk
// (the last of the query's chunks to be dispatched), with a sleep between
// polls, so that the merge workgroups, which may be resident long before their
// chunks finish, load almost nothing while they wait.  Then the wave reads
// every pair it needs (lane c the statistics of chunk c; one whole-wave load of
// 512 consecutive bytes per chunk's values), reloads those whose flag is not
// yet 1, and after using a pair writes zeros back over it.  Each pair is
// written by exactly one partial workgroup and read and cleared by exactly one
// merging wave of the same call, so every call leaves the region all zero, as
// the next call requires.  (Two designs with an arrival counter per
// (query, kv head) measured far slower: each chunk waiting for its stores to
// complete before counting itself, and each chunk counting itself without
// waiting, the pairs still carrying the data.)
//
// Workgroups are dispatched in increasing id order on each XCD, and every merge
// workgroup has a larger id than every partial workgroup, so each partial
// workgroup is resident or finished before any merge workgroup on its XCD can
// hold a slot: every awaited pair arrives.  The polls are still bounded
// (kTailMaxPolls per lane, about a second); a merge that gives up writes NaN,
// so a failure shows instead of hanging the GPU.
constexpr int kTailMaxPolls = 1 << 20;

__device__ __forceinline__ void store_pair(uint64_t *p, float v) {
    __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | (uint64_t(1) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_pair(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void clear_pair(uint64_t *p) {
    __hip_atomic_store(p, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float pair_value(uint64_t x) { return __builtin_bit_cast(float, (uint32_t)x); }
__device__ __forceinline__ bool pair_ready(uint64_t x) { return (uint32_t)(x >> 32) == 1u; }

// The merge of one (query head, 64-dim slice) per wave from flagged pairs: the
// arithmetic of merge_wave, in the same order, so both merges give the same
// bits.  At most 64 chunks (lane c holds chunk c's statistics); the values are
// read kTailBatch chunks at a time.
constexpr int kTailBatch = 16;
template <int D, class Args>
__device__ __forceinline__ void tail_merge(const Args &args) {
    constexpr int SLICES = D / kCombineDims;
    constexpr int TG = (SLICES + kWaves - 1) / kWaves;                  // merge workgroups per query head
    constexpr int64_t CS = (int64_t)SLICES * kFlagPairsPerSlice;        // pairs from a chunk's block to the next's
    static_assert(kSingleLaunchMaxChunks <= 64, "one chunk's statistics per lane");
    static_assert(kTailBatch <= kMergeBatch && 64 % kTailBatch == 0, "batches of whole chunks");
    const int jt = (int)blockIdx.x - args.n_items;
    const int row = jt / TG;
    const int slice = (jt - row * TG) * kWaves + (int)(threadIdx.x >> 6);
    if (slice >= SLICES) return;   // a wave with no slice of this head
    const int si = upper_index(args.n_slots, row, [&](int i) { return args.tkey[i]; });
    const SlotDesc sd = args.slot[si];
    const int h = row - sd.comb_begin;
    const int nc = sd.n_chunks;
    const int lane = threadIdx.x & 63;
    uint64_t *const blk =
        args.flags + (((int64_t)sd.flag_row0 + (int64_t)h * nc) * SLICES + slice) * kFlagPairsPerSlice;
    int polls = 0;
    bool bad = false;
    if (lane == 0) {
        const uint64_t *p = blk + (int64_t)(nc - 1) * CS + kMergeSliceDims;   // the last chunk's M
        while (!pair_ready(load_pair(p)) && polls < kTailMaxPolls) {
            __builtin_amdgcn_s_sleep(16);
            ++polls;
        }
        polls = 0;
    }

    // statistics: lane c holds chunk c's (M, S)
    float mc = -INFINITY, sc = 0.f;
    if (lane < nc) {
        uint64_t *p = blk + (int64_t)lane * CS + kMergeSliceDims;
        uint64_t x = load_pair(p), y = load_pair(p + 1);
        while (!(pair_ready(x) && pair_ready(y)) && polls < kTailMaxPolls) {
            __builtin_amdgcn_s_sleep(2);
            if (!pair_ready(x)) x = load_pair(p);
            if (!pair_ready(y)) y = load_pair(p + 1);
            ++polls;
        }
        bad |= !(pair_ready(x) && pair_ready(y));
        mc = pair_value(x);
        sc = pair_value(y);
        clear_pair(p);
        clear_pair(p + 1);
    }
    const float mx = wave_max(mc);
    const float ms = (mx == -INFINITY) ? 0.f : mx;
    const float w = lane < nc ? fast_exp2(mc - ms) : 0.f;
    const float share = fmaf(w, sc, 0.f);

    float acc = 0.f;
    uint64_t *const col = blk + lane;   // this lane's value pair of chunk c: col + c * CS
    for (int b0 = 0; b0 < nc; b0 += kTailBatch) {
        uint64_t x[kTailBatch];
#pragma unroll
        for (int u = 0; u < kTailBatch; ++u) x[u] = load_pair(col + (int64_t)min(b0 + u, nc - 1) * CS);
        for (;;) {
            bool all = true;
#pragma unroll
            for (int u = 0; u < kTailBatch; ++u) all &= (b0 + u >= nc) || pair_ready(x[u]);
            if (all || polls >= kTailMaxPolls) break;
            __builtin_amdgcn_s_sleep(2);
            ++polls;
#pragma unroll
            for (int u = 0; u < kTailBatch; ++u)
                if (b0 + u < nc && !pair_ready(x[u])) x[u] = load_pair(col + (int64_t)(b0 + u) * CS);
        }
#pragma unroll
        for (int u = 0; u < kTailBatch; ++u) {
            if (b0 + u < nc) {
                bad |= !pair_ready(x[u]);
                acc = fmaf(lane_value(w, b0 + u), pair_value(x[u]), acc);
                clear_pair(col + (int64_t)(b0 + u) * CS);
            }
        }
    }
    const float lsum = wave_sum(share);
    float r = (lsum == 0.f) ? 0.f : acc / lsum;
    if (__builtin_amdgcn_ballot_w64(bad) != 0) r = NAN;
    args.out[((int64_t)sd.slot_idx * args.n_q + h) * D + slice * kCombineDims + lane] = r;
}

// ---------------------------------------------------------------- partial kernel

// U: rows per lane group in flight per register buffer.  fp16 V at
// head_dim >= 256 takes half of it, which keeps 4-row variants at two waves
// per SIMD (the full U needs more than 256 VGPRs).  Measured on graph-replayed
// calls: a speculative verify with 4 drafts at 2 heads 357 -> 335 us, 4 heads
// per kv head at 256 187 -> 177 us, the ragged 4-slot call 63.4 -> 61.9 us; the
// byte formats lose with it.  U depends on head_dim and the V format only, so
// a query computed in a group of drafts and alone takes the same steps.
template <int D, int VF>
struct Geometry {
    static constexpr int R = D / 16;                        // lanes per KV row (16 dims each)
    static constexpr int P = 64 / R;                        // rows per wave load
    static constexpr int U0 = (D == 512) ? 4 : (16 / P);
    static constexpr int U = (VF == kVF16 && D >= 256) ? U0 / 2 : U0;   // loads per wave iteration
    static constexpr int RW = P * U;                        // rows per wave iteration
    static constexpr int HALF = D / 2;
};

// Registers of one wave iteration: U K rows (two 16-byte halves per lane) and
// U V rows (fp16: two halves; int8: one 16-byte code load and one fp16 scale;
// codebook: one 16-byte index load and one fp32 norm).
template <int U>
struct Frag {
    uint4 ka[U], kb[U];
    uint4 va[U], vb[U];
    uint16_t vsc[U];
    float vn[U];
};

// One workgroup per (query group, kv head, chunk, block of GB heads).  A group
// is QB queries of one slot that share the attended start and the chunk size
// (draft tokens of a speculative-verify step): its NR = QB * GB rows are
// (query, head) pairs that all read the same K and V rows once.  Each row
// masks the positions at or past its own end, and a chunk past a query's own
// last chunk is computed fully masked and not written, so every query gets
// exactly the arithmetic it would get alone (the row-to-lane assignment does
// not depend on QB).
//
// V formats (VF): fp16; int8 codes times the fp16 scale of their 32-dim block;
// codebook indices, where an element is level[index & mask] * norm / sqrt(B)
// with one norm per block of B = min(D, 256) dims (the pages' hybrid V).  For
// the byte formats each lane reads 16 consecutive dims of a row, which lie in
// one scale block, so the block's scale (or norm) is folded into the row's
// softmax weight.  The codebook is expanded once per workgroup into a
// 256-entry LDS table already masked and multiplied by 1/sqrt(B), so an
// element costs one byte extract and one LDS read.
//
// SINGLE: one register buffer, each iteration's loads issued right before it is
// consumed, for launches whose every chunk is at most one iteration per wave
// (attn_partial_single_kernel); the rows, their order and the arithmetic are
// those of the buffered form.
template <int D, int QB, int GB, int VF, bool SINGLE, class Args>
__device__ __forceinline__ void partial_lanes(const Args &args) {
    using Geo = Geometry<D, VF>;
    constexpr int R = Geo::R, P = Geo::P, U = Geo::U, RW = Geo::RW, HALF = Geo::HALF;
    constexpr int NR = QB * GB;   // rows: (query of the group, head of the block)
    constexpr bool BYTES = VF != kVF16;                 // one byte per V element
    constexpr int CB_B = D < 256 ? D : 256;             // codebook norm block
    static_assert(kThreads == 256, "one thread per codebook table entry");

    if ((int)blockIdx.x >= args.n_items) {   // a merge workgroup of a single-launch call
        tail_merge<D>(args);
        return;
    }
    const int item = xcd_item(blockIdx.x, args.n_items, args.n_sub);
    int si = upper_index(args.n_slots, item, [&](int i) { return args.key[i]; });
    si -= args.slot[si].lead_off;
    const SlotDesc sd = args.slot[si];   // group leader: the longest query of the group
    const int local = item - sd.item_begin;
    const int sub = local % args.n_sub;
    const int t = local / args.n_sub;
    const int c = t % sd.n_chunks;
    const int kvh = t / sd.n_chunks;
    const int cbeg = sd.lo + c * sd.chunk;
    const int cend = min(cbeg + sd.chunk, sd.L);
    const int h0 = kvh * args.G + sub * GB;            // first query head of the block (in the slot)
    const int64_t rowbase = sd.kv_row0 + (int64_t)kvh * sd.kv_stride;
    const int n_mem = QB == 1 ? 1 : (int)sd.group_n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int rg = lane / R;   // lane group = row within a wave load
    const int sl = lane % R;   // lane within the group

    // per row: query row in q / out, and the end of the positions it attends in this chunk
    int64_t qrow[NR];
    int rend[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int mt = r / GB;
        if (mt < n_mem) {
            const SlotDesc &mb = args.slot[si + mt];
            qrow[r] = mb.slot_idx * (int64_t)args.n_q + h0 + (r % GB);
            rend[r] = min(cend, mb.L);
        } else {
            qrow[r] = -1;
            rend[r] = cbeg;   // an absent member: every position masked
        }
    }

    // q fragment of each row: dims [sl*8, sl*8+8) and [HALF + sl*8, HALF + sl*8 + 8)
    half2_t qv[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (qrow[r] >= 0) {
            const uint16_t *qp = args.q + qrow[r] * D;
            a = *(const uint4 *)(qp + sl * 8);
            b = *(const uint4 *)(qp + HALF + sl * 8);
        }
        qv[r][0] = as_h2(a.x); qv[r][1] = as_h2(a.y); qv[r][2] = as_h2(a.z); qv[r][3] = as_h2(a.w);
        qv[r][4] = as_h2(b.x); qv[r][5] = as_h2(b.y); qv[r][6] = as_h2(b.z); qv[r][7] = as_h2(b.w);
    }

    float m[NR], l[NR], o[NR][16];
#pragma unroll
    for (int g = 0; g < NR; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
    }

    const float sl2 = args.scale_log2;
    const uint16_t *kbase = args.k + rowbase * D;
    __shared__ float s_cb[VF == kVCB ? 256 : 1];   // codebook V: level[i & mask] / sqrt(B)

    // Rows [wb, wb + RW) of one wave iteration: lane group rg reads row wb + u*P + rg.
    // Rows past the chunk end are clamped to its last row (in bounds) and masked.
    auto load = [&](int wb, Frag<U> &f) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = wb + u * P + rg;
            // position -> row: clamp past the chunk end (masked below), then wrap the ring
            int rc = (row < cend ? row : cend - 1) - sd.ring_base;
            if (rc >= sd.ring_cap) rc -= sd.ring_cap;
            const uint16_t *kp = kbase + (int64_t)rc * D;
            f.ka[u] = load_stream16(kp + sl * 8);
            f.kb[u] = load_stream16(kp + HALF + sl * 8);
            if constexpr (VF == kVI8) {
                const int8_t *vp = (const int8_t *)args.v + (rowbase + rc) * D;
                f.va[u] = load_stream16(vp + sl * 16);
                f.vsc[u] = ((const uint16_t *)args.vs)[(rowbase + rc) * (D / 32) + (sl >> 1)];
            } else if constexpr (VF == kVCB) {
                const uint8_t *vp = (const uint8_t *)args.v + (rowbase + rc) * D;
                f.va[u] = load_stream16(vp + sl * 16);
                f.vn[u] = ((const float *)args.vs)[(rowbase + rc) * (D / CB_B) + (sl * 16) / CB_B];
            } else {
                const uint16_t *vp = (const uint16_t *)args.v + (rowbase + rc) * D;
                f.va[u] = load_stream16(vp + sl * 8);
                f.vb[u] = load_stream16(vp + HALF + sl * 8);
            }
        }
    };

    auto consume = [&](int wb, const Frag<U> &f) {
        // ---- logits (log2 domain)
        float s[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int g = 0; g < NR; ++g) {
                float acc = 0.f;
                acc = __builtin_amdgcn_fdot2(as_h2(f.ka[u].x), qv[g][0], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.ka[u].y), qv[g][1], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.ka[u].z), qv[g][2], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.ka[u].w), qv[g][3], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.kb[u].x), qv[g][4], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.kb[u].y), qv[g][5], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.kb[u].z), qv[g][6], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(f.kb[u].w), qv[g][7], acc, false);
                acc = group_sum<R>(acc);
                s[u][g] = (wb + u * P + rg) < rend[g] ? acc * sl2 : -INFINITY;
            }
        }

        // ---- online softmax: new running max, rescale, weights of the U rows
        float p[U][NR];
#pragma unroll
        for (int g = 0; g < NR; ++g) {
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
            const float ms = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = fast_exp2(m[g] - ms);
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u][g] = fast_exp2(s[u][g] - ms);
                psum += p[u][g];
            }
            l[g] = l[g] * alpha + psum;
            m[g] = mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) o[g][i] *= alpha;
        }

        // ---- V accumulation: each row is converted to fp32 once and used by the NR rows
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[16];
            if constexpr (VF == kVCB) {
                const uint32_t wd[4] = {f.va[u].x, f.va[u].y, f.va[u].z, f.va[u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) vf[4 * j + b] = s_cb[(wd[j] >> (8 * b)) & 0xFF];
                }
            } else if constexpr (VF == kVI8) {
                const uint32_t wd[4] = {f.va[u].x, f.va[u].y, f.va[u].z, f.va[u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vf[4 * j + 0] = (float)(int8_t)(wd[j]);
                    vf[4 * j + 1] = (float)(int8_t)(wd[j] >> 8);
                    vf[4 * j + 2] = (float)(int8_t)(wd[j] >> 16);
                    vf[4 * j + 3] = (float)(int8_t)(wd[j] >> 24);
                }
            } else {
                const uint32_t wd[8] = {f.va[u].x, f.va[u].y, f.va[u].z, f.va[u].w,
                                        f.vb[u].x, f.vb[u].y, f.vb[u].z, f.vb[u].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    vf[2 * j + 0] = h2f((uint16_t)(wd[j] & 0xFFFF));
                    vf[2 * j + 1] = h2f((uint16_t)(wd[j] >> 16));
                }
            }
#pragma unroll
            for (int g = 0; g < NR; ++g) {
                float wgt = p[u][g];
                if constexpr (VF == kVI8) wgt *= h2f(f.vsc[u]);
                if constexpr (VF == kVCB) wgt *= f.vn[u];
#pragma unroll
                for (int i = 0; i < 16; ++i) o[g][i] = fmaf(wgt, vf[i], o[g][i]);
            }
        }
    };

    constexpr int STEP = kWaves * RW;
    // Register buffers of loads in flight: three where the third keeps the
    // variant's occupancy (one or two rows up to head_dim 256, one row at 512),
    // else two; one in the SINGLE form.  The rows of each iteration and the
    // order they are consumed in do not change, so neither do the results.
    constexpr int NBUF = SINGLE ? 1 : (NR == 1 || (NR == 2 && D <= 256)) ? 3 : 2;
    int wb = cbeg + w * RW;
    if constexpr (NBUF == 1) {
        Frag<U> f0;
        if constexpr (VF == kVCB) {
            s_cb[tid] = args.codebook[tid & args.cb_mask] * args.cb_scale;
            __syncthreads();
        }
        while (wb < cend) {
            load(wb, f0);
            consume(wb, f0);
            wb += STEP;
        }
    } else if constexpr (NBUF == 3) {
        Frag<U> f0, f1, f2;
        if (wb < cend) load(wb, f0);
        if (wb + STEP < cend) load(wb + STEP, f1);
        if constexpr (VF == kVCB) {
            s_cb[tid] = args.codebook[tid & args.cb_mask] * args.cb_scale;
            __syncthreads();
        }
        while (wb < cend) {
            if (wb + 2 * STEP < cend) load(wb + 2 * STEP, f2);
            consume(wb, f0);
            wb += STEP;
            if (wb >= cend) break;
            if (wb + 2 * STEP < cend) load(wb + 2 * STEP, f0);
            consume(wb, f1);
            wb += STEP;
            if (wb >= cend) break;
            if (wb + 2 * STEP < cend) load(wb + 2 * STEP, f1);
            consume(wb, f2);
            wb += STEP;
        }
    } else {
        Frag<U> fa, fb;
        if (wb < cend) load(wb, fa);
        if constexpr (VF == kVCB) {
            s_cb[tid] = args.codebook[tid & args.cb_mask] * args.cb_scale;
            __syncthreads();
        }
        while (wb < cend) {
            int wn = wb + STEP;
            if (wn < cend) load(wn, fb);
            consume(wb, fa);
            wb = wn;
            if (wb >= cend) break;
            wn = wb + STEP;
            if (wn < cend) load(wn, fa);
            consume(wb, fb);
            wb = wn;
        }
    }

    // ---- merge the P lane groups of the wave (lanes lane ^ off share the dims)
#pragma unroll
    for (int off = R; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < NR; ++g) {
            const float m2 = shfl_xor_f32(m[g], off);
            const float l2 = shfl_xor_f32(l[g], off);
            const float mx = fmaxf(m[g], m2);
            const float ms = (mx == -INFINITY) ? 0.f : mx;
            const float a1 = fast_exp2(m[g] - ms);
            const float a2 = fast_exp2(m2 - ms);
            l[g] = l[g] * a1 + l2 * a2;
            m[g] = mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float o2 = shfl_xor_f32(o[g][i], off);
                o[g][i] = o[g][i] * a1 + o2 * a2;
            }
        }
    }

    // ---- merge the waves through LDS
    __shared__ float s_o[kWaves][NR][D];
    __shared__ float s_ml[kWaves][NR][2];
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < NR; ++g) {
            if constexpr (BYTES) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s_o[w][g][sl * 16 + i] = o[g][i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    s_o[w][g][sl * 8 + i] = o[g][i];
                    s_o[w][g][HALF + sl * 8 + i] = o[g][8 + i];
                }
            }
            if (sl == 0) {
                s_ml[w][g][0] = m[g];
                s_ml[w][g][1] = l[g];
            }
        }
    }
    __syncthreads();

    // A query merged in this launch (flag_row0 >= 0: not in a query group, several chunks)
    // writes its partials as flagged pairs and is done (tail_merge).
    const bool publish = sd.flag_row0 >= 0;
    for (int idx = tid; idx < NR * D; idx += kThreads) {
        const int g = idx / D;
        const int d = idx - g * D;
        const int mt = g / GB;
        if (mt >= n_mem) continue;
        const SlotDesc &mb = args.slot[si + mt];
        if (c >= mb.n_chunks) continue;   // past this query's last chunk: nothing to write
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) mx = fmaxf(mx, s_ml[ww][g][0]);
        const float ms = (mx == -INFINITY) ? 0.f : mx;
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float a = fast_exp2(s_ml[ww][g][0] - ms);
            acc += s_o[ww][g][d] * a;
            lsum += s_ml[ww][g][1] * a;
        }
        if (mb.n_chunks == 1) {
            args.out[qrow[g] * D + d] = (lsum == 0.f) ? 0.f : acc / lsum;
        } else if (publish) {
            constexpr int SL = D / kMergeSliceDims;
            const int64_t r = (int64_t)mb.flag_row0 + (int64_t)(h0 + g % GB) * mb.n_chunks + c;
            uint64_t *blk = args.flags + (r * SL + d / kMergeSliceDims) * kFlagPairsPerSlice;
            store_pair(blk + (d % kMergeSliceDims), acc);
            if (d % kMergeSliceDims == 0) {
                store_pair(blk + kMergeSliceDims, mx);
                store_pair(blk + kMergeSliceDims + 1, lsum);
            }
        } else {
            const int64_t prow = mb.part_row0 + (int64_t)(h0 + g % GB) * mb.n_chunks + c;
            args.ws_o[prow * D + d] = acc;
            if (d == 0) {
                args.ws_ml[prow * 2 + 0] = mx;
                args.ws_ml[prow * 2 + 1] = lsum;
            }
        }
    }
}

template <int D, int QB, int GB, int VF, int NS>
__global__ __launch_bounds__(kThreads) void attn_partial_kernel(const LaunchArgsT<NS> args) {
    partial_lanes<D, QB, GB, VF, false>(args);
}

// The lane kernel for launches of many chunks of at most one iteration per wave
// (one-byte V at head_dim 256: up to 64 positions, the chunks of slots of up to
// 2048 positions).  There the buffered form's extra buffers are never filled,
// and without them the registers allow four waves per SIMD instead of two, so
// twice the workgroups per CU overlap their fixed start and merge costs.  Same
// results bit for bit.
template <int D, int GB, int VF, int NS>
__global__ __launch_bounds__(kThreads, 4) void attn_partial_single_kernel(const LaunchArgsT<NS> args) {
    partial_lanes<D, 1, GB, VF, true>(args);
}

// ---------------------------------------------------------------- combine kernel

// One wave per (query, query head, 64-dim slice) of a query with several
// chunks, after the partial kernel has finished.
template <int D, int NS>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const LaunchArgsT<NS> args) {
    constexpr int SLICES = D / kCombineDims;
    const int row = blockIdx.x / SLICES;
    const int slice = blockIdx.x - row * SLICES;
    const int si = upper_index(args.n_slots, row, [&](int i) { return args.key[i]; });
    const SlotDesc sd = args.slot[si];
    merge_wave<D>(args, sd, row - sd.comb_begin, slice);
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t value) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

}  // namespace attn_decode_impl
