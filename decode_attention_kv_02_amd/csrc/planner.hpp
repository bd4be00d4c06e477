// planner.hpp -- host-side split-KV planner of the decode-attention library.
//
// Pure C++ (no HIP): validates shapes and turns per-slot KV lengths into the
// flat work list the partial kernel runs over.  The pages split the KV range
// of each query row over workgroups and merge the pieces by log-sum-exp
// (mlx-native flash_attn_vec_hybrid.metal, the NWG split-K of
// flash_attn_vec_hybrid_impl; tessl nn.rs, flash_attn_decode and the
// DecodeChunk table); mlx-native's GQA-grouped batched kernel lets every slot
// run its own split (FlashAttnHybridSlotBucket).  Here the split of a slot is a
// function of that slot's attended length alone, so batching slots never
// changes any slot's result, and every workgroup of a launch does one chunk of
// at most `chunk` positions (a flat list instead of a padded grid).
//
// Every query row is first described by a span: its attended positions
// [lo, L), where its (slot, kv head 0) rows start, the row stride between kv
// heads, and the ring wrap.  Packed ragged slots and fixed-capacity linear or
// ring caches differ only in how the spans are made (mlx-native batched
// kernels: per-slot offset slot * n_kv * capacity * D, kv_seq_len =
// min(pos + 1, capacity) on the ring, physical row = position mod capacity).
#pragma once

#include <algorithm>
#include <climits>
#include <cstdint>
#include <string>
#include <vector>

namespace attn_decode_impl {

constexpr int kMaxSlotsPerLaunch = 256;  // query table passed by value in the kernel arguments
constexpr int kSmallTableSlots = 48;     // launches of up to this many query rows take the small table
constexpr int kMaxChunks = 4096;         // per slot; bounds the combine kernel's LDS weights
constexpr int kChunkQuantum = 64;        // chunk sizes are multiples of this (one workgroup iteration at D=256)
constexpr int kChunkMin = 64;
constexpr int kChunkMax = 2048;
constexpr int64_t kMaxItemsPerLaunch = int64_t(1) << 24;  // 2^24 workgroups x 256 threads < 2^32
constexpr int kQuantBlock = 32;          // int8 V: dims per fp16 scale
constexpr int GROUP_ROWS = 4;            // (query, head) rows one workgroup may carry

// Positions and rows one query row attends.
struct QuerySpan {
    int32_t L = 0;             // one past the last attended position
    int32_t lo = 0;            // first attended position
    int64_t kv_row0 = 0;       // row of (slot, kv head 0) holding position-row 0
    int32_t kv_stride = 0;     // rows between consecutive kv heads of the slot
    int32_t ring_cap = INT32_MAX;  // ring capacity (INT32_MAX: rows never wrap)
    int32_t ring_base = 0;     // multiple of ring_cap <= lo: row of position p is p - ring_base (mod ring_cap)
};

struct SlotPlan {
    int32_t L = 0;          // one past the last attended position
    int32_t lo = 0;         // first attended position
    int32_t n = 0;          // attended positions (L - lo)
    int32_t kv_stride = 0;
    int32_t ring_cap = INT32_MAX;
    int32_t ring_base = 0;
    int32_t chunk = 0;      // positions per chunk
    int32_t n_chunks = 1;   // >= 1 (an empty slot has one empty chunk)
    int64_t kv_row0 = 0;    // row of (slot, kv head 0, position-row 0)
    int64_t part_row0 = -1; // first partial row when n_chunks > 1, else -1
    bool fused = false;     // merged by the partial kernel's own launch (single-launch merge)
    int32_t flag_row0 = -1; // fused: first of its partial rows in the flagged region, else -1
    int32_t group_n = 1;    // on a group leader: queries of its group; 0 on a follower
    int32_t leader = -1;    // on a follower: the leader's index
    std::vector<int32_t> members;   // on a leader: followers in table order
    bool mfma = false;      // computed by the matrix-core partial kernel
};


// How one partial kernel splits the work: query heads per workgroup (GB, dividing G),
// G / GB workgroups per (query group, kv head, chunk), queries per workgroup (QB).
struct KernelShape {
    int GB = 1;
    int n_sub = 1;   // workgroups per chunk: head blocks, G / GB
    int QB = 1;      // lane kernel: its template parameter (QB * GB <= 4); matrix cores: the largest group
};

struct LaunchGroup {
    std::vector<int32_t> slots;        // slot indices, in work-list order
    int64_t items = 0;                 // partial-kernel workgroups
    bool single = false;               // lane kernel in its single-buffer form (see single_pass_positions)
    int64_t combine_rows = 0;          // query heads merged by the combine kernel
    int64_t tail_rows = 0;             // query heads merged by merge workgroups at the end of the
                                       // partial kernel's grid (head_dim / 64 workgroups each)
    bool mfma = false;                 // which partial kernel computes this launch
};

struct CallPlan {
    bool mfma = false;   // every query on the matrix-core kernel (8k heads per kv head, head_dim >= 128)
    int G = 1;           // query heads per KV head
    KernelShape lanes;   // the lane kernel's shape: GB 1, 2 or 4
    KernelShape matrix;  // the matrix-core kernel's: GB 8 or 16, or GB = G for draft groups
    std::vector<SlotPlan> slots;
    std::vector<LaunchGroup> groups;
    int64_t part_rows = 0;         // plain partial rows (each head_dim floats + 2 stats)
    int64_t flag_rows = 0;         // partial rows of fused queries, as flagged pairs
    int fuse_limit = 1;            // largest chunk count merged in the partial kernel's launch
    int64_t workspace_bytes = 0;   // flagged region (256-byte aligned) + plain partial rows
    int64_t total_items = 0;
};

// With the single-launch merge, lane-kernel queries split into at most this many
// chunks (a merging wave keeps one chunk's statistics per lane) that are not
// part of a query group are merged by workgroups at the end of the partial
// kernel's own grid; the others still go to the combine kernel.
constexpr int kSingleLaunchMaxChunks = 64;

// kMergeAuto currently selects the combine kernel.
enum MergeMode { kMergeAuto = 0, kMergeCombineKernel = 1, kMergeInKernel = 2 };

// A fused query's partial rows are written as 8-byte pairs {value bits, 1}: per
// 64-dim slice of a row, a block of 80 pairs (640 bytes, five 128-byte lines)
// holding the 64 value pairs, the pair of M, the pair of S and 14 unused pairs,
// so every slice's values start on a 128-byte line.  The pairs sit at the front
// of the workspace in a 256-byte aligned region that is all zero between calls
// (each call clears the pairs it wrote).
constexpr int kMergeSliceDims = 64;
constexpr int kFlagPairsPerSlice = 80;
inline int64_t flag_region_bytes(int64_t flag_rows, int32_t head_dim) {
    return (flag_rows * (head_dim / kMergeSliceDims) * kFlagPairsPerSlice * 8 + 255) / 256 * 256;
}
// A merge workgroup at the end of a single-launch grid merges up to this many
// slices of one query head, one per wave.
constexpr int kMergeSlicesPerGroup = 4;
inline int64_t merge_groups(int32_t head_dim) {
    return (head_dim / kMergeSliceDims + kMergeSlicesPerGroup - 1) / kMergeSlicesPerGroup;
}

inline bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunks per (slot, kv head) the planner aims for, by attended length.  Short
// slots are split finely so that a lone slot still fills the GPU; long slots
// get long chunks, because every workgroup pays a fixed cost (first-load
// latency, the lane/wave merge, a partial row per head) and the combine reads
// one partial row per chunk.  Measured on MI355X with forced chunk sizes
// (warm, back-to-back calls): a 1024-position window runs fastest at 64
// positions per chunk, 1 x 131072 at 2048, 8 x 32768 int8-V at 2048 (1024 is
// 2% slower there but twice as fast for a lone 32768 slot, so 32768 gets
// 1024).  1 x 4096 at D = 256 takes 128 (graph-replayed, alternating on one
// box: 11.97 -> 11.46 us against 64, 8 x 4096 51.7 -> 49.6 us; another box
// measured the single slot 3% slower).  The pages weigh the same two costs
// when they pick a chunk (tessl nn.rs, the DecodeChunk table): more chunks give
// more workgroups, but leave more partial rows for the merge to read.
inline int64_t target_chunks(int64_t n) {
    if (n <= 65536) return 32;
    return 16;
}

// Above 4096 positions a chunk also carries at least 256 KiB of fp16 K and V
// per kv head (65536 / head_dim positions): slots that long usually come in
// batches, where fine chunks leave each workgroup too little work for its
// fixed cost.  Measured with forced chunks (lane kernel, graph-replayed):
// 8 x 8192 at head_dim 128 with 4 heads per kv head 83.5 us at 128 positions,
// 54.9 at 512; at head_dim 64 68.9 -> 36.0 us (1024); 8 x 8192 int8 V at 256
// 82.2 -> 73.4 us (256), while a lone 8192 slot moves by 0.3-2 us.  Lone
// slots of 4096 or less (1 x 4096: 11.5 us at 128 positions, 14.4 at 256)
// keep a finer split, down to 64 KiB of K and V per chunk and kv head
// (64 positions at head_dim 256, 128 at 128, 256 at 64).  Below that floor
// batches lose to the workgroups' fixed cost: at head_dim 128, 16 x 2048 took
// 38.3 us in 64-position chunks and 29.6 in 128-position ones, 8 x 4096 37.6
// and 29.8; at head_dim 64 16 x 2048 took 22.0 us and 18.0 in 256-position
// chunks.  A lone 2048 slot moves by +0.1 / +0.3 us there, a lone 4096 slot
// gains 0.6-0.9 us.
constexpr int64_t kLongSlot = 4096;
// floors of fp16 K + V bytes per chunk and kv head (chunk * 2 * head_dim * 2)
constexpr int64_t kMinLongChunkKVBytes = 262144;   // slots of more than kLongSlot positions
constexpr int64_t kMinShortChunkKVBytes = 65536;   // the others

inline int64_t min_chunk_long(int32_t head_dim) { return kMinLongChunkKVBytes / (4 * (int64_t)head_dim); }
inline int64_t min_chunk_short(int32_t head_dim) {
    const int64_t c = kMinShortChunkKVBytes / (4 * (int64_t)head_dim);
    return (c + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
}

// A slot whose fp16 K and V rows of one kv head fit in this many bytes is not
// split: one workgroup streams it in about the time of the first-load latency,
// and splitting it would add the combine launch (measured: 1 x 256 at
// head_dim 64 takes the same partial-kernel time in one chunk as in four).
constexpr int64_t kSingleChunkBytes = 128 * 1024;

// Positions per chunk for a slot attending n positions (n >= 1).  Depends on
// the slot's own length and head_dim only, so a slot is split the same way in
// every batch.
// The matrix-core kernel runs 4 waves of 16-key tiles per workgroup, at most 2
// workgroups per CU: it takes longer chunks, n / 32 within [512, 2048]
// (measured with forced chunks at 8 and 16 heads per kv head: 512 beats 128
// and 256 on 8 x 8192 at head_dim 128 by 10-20%, 1024 beats 512 on 4 x 32768
// fp16 at 256 and 512, and 512 beats 1024 on 4 x 16384, where 1024 leaves too
// few workgroups).
constexpr int64_t kMfmaChunkMin = 512;
constexpr int64_t kMfmaChunkTarget = 32;

inline int64_t chunk_for(int64_t n, int32_t head_dim, int32_t forced, bool mfma = false) {
    int64_t c;
    if (forced > 0) {
        c = forced;
    } else if (n * 4 * head_dim <= kSingleChunkBytes) {
        c = ceil_div(n, kChunkQuantum) * kChunkQuantum;
    } else if (mfma) {
        c = ceil_div(ceil_div(n, kMfmaChunkTarget), kChunkQuantum) * kChunkQuantum;
        if (c < kMfmaChunkMin) c = kMfmaChunkMin;
        if (c > kChunkMax) c = kChunkMax;
    } else {
        c = ceil_div(n, target_chunks(n));
        c = ceil_div(c, kChunkQuantum) * kChunkQuantum;
        if (c < kChunkMin) c = kChunkMin;
        if (n > kLongSlot && c < min_chunk_long(head_dim)) c = min_chunk_long(head_dim);
        if (n <= kLongSlot && c < min_chunk_short(head_dim)) c = min_chunk_short(head_dim);
        if (c > kChunkMax) c = kChunkMax;
    }
    const int64_t floor_c = ceil_div(n, kMaxChunks);
    if (c < floor_c) c = forced > 0 ? floor_c : ceil_div(floor_c, kChunkQuantum) * kChunkQuantum;
    return c;
}

// The chunk option's per-call mode (ATTN_DECODE_CHUNK_PER_CALL): every query's chunk is at least a
// floor the planner takes from the whole call, so that a large batch runs about as many workgroups
// of long chunks as its kernel keeps resident over one or two generations, instead of many short
// ones: 1024 on the lane kernel (two or three 4-wave workgroups per CU), 256 on the matrix cores
// at head_dim 512 (one 8-wave workgroup per CU), 512 on the matrix cores below.  The floor depends
// on the batch, so in this mode a slot's result can differ in rounding between a batched call and
// a call of that slot alone; the default mode keeps them bitwise equal.  Measured (graph-replayed):
// 128 ring slots of 2048 rows, int8 V, D = 256, 340 -> 244 us; 8 x 32768 at D = 512, codebook V,
// 16 q / 2 kv heads, forced chunks 1024 -> 2048: 145.0 -> 136.8 us, 16 x 32768 283.7 -> 264.6.
constexpr int32_t kChunkPerCall = -1;
inline int64_t per_call_items(bool mfma, int32_t head_dim) { return !mfma ? 1024 : head_dim == 512 ? 256 : 512; }
inline int64_t per_call_floor(int64_t positions_x_heads, int64_t items) {
    int64_t c = ceil_div(ceil_div(positions_x_heads, items), kChunkQuantum) * kChunkQuantum;
    return c < kChunkMin ? kChunkMin : c > kChunkMax ? kChunkMax : c;
}

// Shape checks shared by every entry point.  Returns "" when valid.
inline std::string check_common(int32_t n_q, int32_t n_kv, int32_t head_dim, bool v_int8,
                                int32_t window, int32_t chunk, int32_t merge_mode) {
    if (merge_mode != kMergeAuto && merge_mode != kMergeCombineKernel && merge_mode != kMergeInKernel)
        return "unknown merge_mode";
    if (n_q <= 0 || n_kv <= 0) return "n_q_heads and n_kv_heads must be positive";
    if (n_q % n_kv != 0) return "n_q_heads must be a multiple of n_kv_heads";
    if (!supported_head_dim(head_dim)) return "head_dim must be 64, 128, 256 or 512";
    if (v_int8 && head_dim % kQuantBlock != 0) return "int8 V needs head_dim % 32 == 0";
    if (window < 0) return "window must be >= 0";
    if (chunk < 0 && chunk != kChunkPerCall) return "chunk override must be >= 0, or -1 for the per-call floor";
    return "";
}

inline std::string check_shapes(const int32_t *seq_lens, int32_t n_slots, int32_t window,
                                int32_t n_q, int32_t n_kv, int32_t head_dim, bool v_int8,
                                int32_t chunk, int32_t merge_mode = 0) {
    if (n_slots < 0) return "n_slots must be >= 0";
    std::string err = check_common(n_q, n_kv, head_dim, v_int8, window, chunk, merge_mode);
    if (!err.empty()) return err;
    if (n_slots > 0 && seq_lens == nullptr) return "seq_lens is NULL";
    for (int32_t s = 0; s < n_slots; ++s)
        if (seq_lens[s] < 0) return "seq_lens[" + std::to_string(s) + "] is negative";
    return "";
}

// Spans of packed ragged slots: slot s's rows follow those of slots t < s.
inline void spans_packed(const int32_t *seq_lens, int32_t n_slots, int32_t window, int32_t n_kv,
                         std::vector<QuerySpan> &spans) {
    spans.assign(n_slots, QuerySpan());
    int64_t rows = 0;   // running sum of L_t (positions)
    for (int32_t s = 0; s < n_slots; ++s) {
        QuerySpan &q = spans[s];
        q.L = seq_lens[s];
        q.lo = (window > 0 && q.L > window) ? q.L - window : 0;
        q.kv_row0 = rows * n_kv;
        q.kv_stride = q.L;
        rows += q.L;
    }
}

// Checks of the fixed-capacity cache entry point.  Returns "" when valid.
inline std::string check_cache(const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
                               int32_t n_cache_slots, int32_t capacity, int32_t ring) {
    if (n_queries < 0) return "n_queries must be >= 0";
    if (ring != 0 && ring != 1) return "ring must be 0 or 1";
    if (capacity <= 0) return "capacity must be positive";
    if (n_queries > 0 && (slot_ids == nullptr || positions == nullptr)) return "slot_ids / positions is NULL";
    for (int32_t i = 0; i < n_queries; ++i) {
        if (slot_ids[i] < 0 || slot_ids[i] >= n_cache_slots)
            return "slot_ids[" + std::to_string(i) + "] is outside [0, n_cache_slots)";
        if (positions[i] < 0) return "positions[" + std::to_string(i) + "] is negative";
        if (positions[i] == INT32_MAX) return "positions[" + std::to_string(i) + "] is too large";
        if (!ring && positions[i] >= capacity)
            return "positions[" + std::to_string(i) + "] is not below the capacity of a linear cache";
    }
    return "";
}

// Spans of a [slot][kv head][capacity][D] cache: query i attends positions up to
// positions[i] of cache slot slot_ids[i]; linear storage keeps position p in row
// p, ring storage in row p mod capacity (only the last `capacity` positions).
inline void spans_cache(const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
                        int32_t capacity, int32_t ring, int32_t window, int32_t n_kv,
                        std::vector<QuerySpan> &spans) {
    spans.assign(n_queries, QuerySpan());
    for (int32_t i = 0; i < n_queries; ++i) {
        QuerySpan &q = spans[i];
        q.L = positions[i] + 1;
        int32_t lo = 0;
        if (ring && q.L > capacity) lo = q.L - capacity;
        if (window > 0 && q.L - window > lo) lo = q.L - window;
        q.lo = lo;
        q.kv_row0 = (int64_t)slot_ids[i] * n_kv * capacity;
        q.kv_stride = capacity;
        if (ring) {
            q.ring_cap = capacity;
            q.ring_base = lo / capacity * capacity;
        }
    }
}

inline int heads_per_workgroup(int G) {
    if (G % 4 == 0) return 4;
    if (G % 2 == 0) return 2;
    return 1;
}

// A lane-kernel call with fewer workgroups than this (fewer than the GPU's 256
// compute units) takes half the heads per workgroup, down to one: twice the
// workgroups, the sibling reading the same K and V rows from its XCD's L2.
// Measured (graph-replayed / flushed events): the 1024-position window of one
// 131072 slot, 128 -> 256 workgroups, 8.2 -> 7.2 us / 13.5 -> 12.3 us; calls
// that already fill the chip lose (the ragged 4-slot call 60 -> 81 us, 1 x 4096
// 11.9 -> 12.5 us).  Each (query, head) row takes the same steps whatever the
// number of heads per workgroup, so the results do not change.
constexpr int64_t kSplitHeadsBelowItems = 256;

// Positions one iteration of the lane kernel's four waves covers with one-byte V at head_dim 256
// (each wave 16 rows); 0 where the single-buffer form is not built.  A lane-kernel launch whose
// every chunk fits in one such iteration, with at least kSingleMinItems workgroups, runs the
// single-buffer form (attn_partial_single_kernel): its workgroups never fill a second buffer, and
// without the buffers the registers allow four waves per SIMD instead of two.  The arithmetic is
// the same, so the choice never changes a result.  Measured (graph-replayed, 16 q / 8 kv heads,
// int8 V): 48 x 2048 150.0 -> 134.8 us, 128 x 1024 209.5 -> 189.9, 16 x 2048 55.4 -> 50.6,
// 8 x 1024 19.1 -> 17.0; a lone 2048 slot (256 workgroups) 9.3 -> 10.7 us, so small grids keep
// the buffered form.
inline int single_pass_positions(int32_t head_dim, bool byte_v) { return head_dim == 256 && byte_v ? 64 : 0; }
constexpr int64_t kSingleMinItems = 1024;

// Which partial kernel computes a query.  The matrix-core kernel
// (attn_partial_mfma_kernel) puts up to 16 (query, head) columns in one
// workgroup.  It applies to a whole call at a multiple of 8 query heads per kv
// head and head_dim >= 128, where it measured faster than the lane kernel on
// every shape (graph-replayed, fp16 / int8 / codebook V, head_dim 128..512:
// 1.46x at 8 heads and 512, up to 2.7x at 16 heads and 128).  With fewer heads
// per kv head, the draft queries of one slot (a speculative-verify step), or
// one query alone, go to the matrix cores as one workgroup when they fill at
// least mfma_group_min_cols columns (drafts x heads: 4, e.g. 2 drafts at 2
// heads per kv head or one query with 4; 8 at head_dim 512 with one-byte V),
// so each K and V byte is read once for all of them; the lane kernel holds at
// most 4 rows.  Which kernel a query gets depends only on the queries of its
// own slot, so a batched call equals per-slot calls bitwise.
// kPathLanes forces the lane kernel everywhere, kPathMatrix the matrix cores
// (where they apply to the whole call).
enum KernelPath { kPathAuto = 0, kPathLanes = 1, kPathMatrix = 2 };

inline bool mfma_applies(int G, int head_dim) { return G % 8 == 0 && head_dim >= 128; }
inline bool mfma_preferred(int G, int head_dim) { return mfma_applies(G, head_dim); }
constexpr int kMfmaColumns = 16;      // (query, head) columns of one matrix-core workgroup
// Query groups (a slot's drafts x heads, or one query's heads) at least this many columns wide
// go to the matrix cores.  Four wherever that kernel takes the fp16 products; measured against the
// lanes (graph-replayed): one query with 4 heads per kv head at head_dim 128, 8 x 8192, 53.4 ->
// 46.3 us, codebook V at 256 146.1 -> 136.7 us, fp16 at 256 and 512 within 1%; 3 drafts x 2 heads
// over 4 x 32768 329.0 -> 171.4 us (the lanes' groups hold at most 4 rows, so 6 rows took two
// reads of the cache).  Eight at head_dim 512 with one-byte V: one query with 4 heads per kv head
// (8 x 32768, 16 q / 4 kv heads) runs as fast on the lanes (int8 278.9 us against 284.2 on the
// matrix cores, codebook 283.3 against 279.2; with one wave per SIMD there the matrix cores took
// 164 us against the lanes' 143 on int8 at 8 heads).
inline int mfma_group_min_cols(int head_dim, bool byte_v) { return head_dim == 512 && byte_v ? 8 : 4; }
// Waves of a matrix-core workgroup that share each 16-key tile by dims: at head_dim 512, two (an
// 8-wave workgroup): each wave loads K for 256 of the dims and V for 256 of the output dims, so
// that its accumulators and V buffers halve and two waves run per SIMD instead of one; the two
// halves of each QK product are summed through LDS.
constexpr int mfma_dim_splits(int head_dim) { return head_dim == 512 ? 2 : 1; }

// Builds the plan from the query spans; returns "" on success or an error message.
inline std::string make_plan(const std::vector<QuerySpan> &spans, int32_t n_q, int32_t n_kv,
                             int32_t head_dim, int32_t chunk, int32_t merge_mode, CallPlan &plan,
                             int32_t path = kPathAuto, bool byte_v = false, int32_t lanes_gb = 0,
                             int32_t group_gb = 0) {
    plan = CallPlan();
    const int32_t n_slots = (int32_t)spans.size();
    plan.G = n_q / n_kv;
    if (path != kPathAuto && path != kPathLanes && path != kPathMatrix) return "unknown kernel path";
    if (path == kPathMatrix && !mfma_applies(plan.G, head_dim))
        return "the matrix-core path needs a multiple of 8 query heads per kv head and head_dim >= 128";
    plan.mfma = path == kPathMatrix || (path == kPathAuto && mfma_preferred(plan.G, head_dim));
    const int G = plan.G;
    plan.lanes.GB = lanes_gb > 0 ? lanes_gb : heads_per_workgroup(G);
    plan.lanes.n_sub = G / plan.lanes.GB;
    // query groups are bounded by the automatic heads per workgroup, so splitting the heads of a
    // small call (below) changes no group
    const int lane_qb_max = GROUP_ROWS / (group_gb > 0 ? group_gb : plan.lanes.GB);
    int mfma_qb_max = 1;
    if (plan.mfma) {
        plan.matrix.GB = G % 16 == 0 ? 16 : 8;
        plan.matrix.n_sub = G / plan.matrix.GB;
        mfma_qb_max = kMfmaColumns / plan.matrix.GB;
    } else if (path == kPathAuto && head_dim >= 128 && G <= kMfmaColumns / 2) {
        plan.matrix.GB = G;             // draft groups: every head of the kv head, for each draft
        plan.matrix.n_sub = 1;
        mfma_qb_max = kMfmaColumns / G;
    }
    // the matrix-core kernel always merges in the combine kernel
    plan.fuse_limit = merge_mode == kMergeInKernel ? kSingleLaunchMaxChunks : 1;
    plan.slots.resize(n_slots);
    for (int32_t s = 0; s < n_slots; ++s) {
        SlotPlan &sp = plan.slots[s];
        const QuerySpan &qs = spans[s];
        sp.L = qs.L;
        sp.lo = qs.lo;
        sp.n = sp.L - sp.lo;
        sp.kv_row0 = qs.kv_row0;
        sp.kv_stride = qs.kv_stride;
        sp.ring_cap = qs.ring_cap;
        sp.ring_base = qs.ring_base;
        sp.mfma = plan.mfma;
    }
    int64_t call_units = 0;   // the per-call mode: attended positions x kv heads of the call
    if (chunk == kChunkPerCall)
        for (int32_t s = 0; s < n_slots; ++s) call_units += (int64_t)plan.slots[s].n * n_kv;
    auto set_chunks = [&](SlotPlan &sp) {
        if (sp.n == 0) {
            sp.chunk = 0;
            sp.n_chunks = 1;
        } else {
            int64_t c = chunk_for(sp.n, head_dim, chunk > 0 ? chunk : 0, sp.mfma);
            if (chunk == kChunkPerCall) {
                const int64_t floor_c = per_call_floor(call_units, per_call_items(sp.mfma, head_dim));
                if (c < floor_c) c = floor_c;
            }
            sp.chunk = (int32_t)(c > sp.n ? sp.n : c);
            sp.n_chunks = (int32_t)ceil_div(sp.n, sp.chunk);
        }
    };

    // Query groups: queries of one slot with the same attended start and chunk
    // size (draft tokens of a speculative-verify step) share one workgroup, so
    // their K and V rows are read once: on the lane kernel up to 4 / GB of
    // them, on the matrix cores up to 16 / GB.
    // Candidates are the non-empty queries with the same rows and start,
    // longest first (a group's leader is its longest query).
    std::vector<int32_t> idx;
    for (int32_t s = 0; s < n_slots; ++s)
        if (plan.slots[s].n > 0) idx.push_back(s);
    auto same_rows = [&](int32_t a, int32_t b) {
        const SlotPlan &x = plan.slots[a], &y = plan.slots[b];
        return x.kv_row0 == y.kv_row0 && x.kv_stride == y.kv_stride && x.ring_cap == y.ring_cap &&
               x.ring_base == y.ring_base && x.lo == y.lo;
    };
    std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
        const SlotPlan &x = plan.slots[a], &y = plan.slots[b];
        if (x.kv_row0 != y.kv_row0) return x.kv_row0 < y.kv_row0;
        if (x.kv_stride != y.kv_stride) return x.kv_stride < y.kv_stride;
        if (x.ring_cap != y.ring_cap) return x.ring_cap < y.ring_cap;
        if (x.ring_base != y.ring_base) return x.ring_base < y.ring_base;
        if (x.lo != y.lo) return x.lo < y.lo;
        if (x.L != y.L) return x.L > y.L;
        return a < b;
    });
    auto make_group = [&](const std::vector<int32_t> &q, size_t i, size_t j) {
        SlotPlan &lead = plan.slots[q[i]];
        lead.group_n = (int32_t)(j - i);
        for (size_t k = i + 1; k < j; ++k) {
            lead.members.push_back(q[k]);
            plan.slots[q[k]].group_n = 0;
            plan.slots[q[k]].leader = q[i];
        }
    };
    // within a run of candidates, consecutive queries of one chunk size form groups of up to qb_max
    auto group_run = [&](const std::vector<int32_t> &q, int qb_max, int min_size, int &qb_used,
                         std::vector<int32_t> *rest) {
        for (size_t i = 0; i < q.size();) {
            size_t j = i + 1;
            while (j < q.size() && (int)(j - i) < qb_max && plan.slots[q[j]].chunk == plan.slots[q[i]].chunk) ++j;
            if ((int)(j - i) >= min_size && j - i > 1) {
                make_group(q, i, j);
                qb_used = std::max(qb_used, (int)(j - i));
            } else if (rest) {
                for (size_t k = i; k < j; ++k) rest->push_back(q[k]);
            }
            i = j;
        }
    };
    std::vector<int32_t> lane_q;   // queries left to the lane kernel, in candidate order
    const int min_cols = mfma_group_min_cols(head_dim, byte_v);
    for (size_t i = 0; i < idx.size();) {
        size_t j = i + 1;
        while (j < idx.size() && same_rows(idx[i], idx[j])) ++j;
        std::vector<int32_t> run(idx.begin() + i, idx.begin() + j);
        if (plan.mfma) {
            for (int32_t q : run) set_chunks(plan.slots[q]);
            if (mfma_qb_max > 1) group_run(run, mfma_qb_max, 2, plan.matrix.QB, nullptr);
        } else if (mfma_qb_max > 1 && (int64_t)run.size() * G >= min_cols) {
            // query groups for the matrix cores: chunks by their rule; what does not fill
            // min_cols columns goes back to the lane kernel (a query that fills them alone stays)
            for (int32_t q : run) {
                plan.slots[q].mfma = true;
                set_chunks(plan.slots[q]);
            }
            std::vector<int32_t> back;
            const int min_q = (min_cols + G - 1) / G;
            group_run(run, mfma_qb_max, min_q, plan.matrix.QB, min_q > 1 ? &back : nullptr);
            for (int32_t q : back) {
                plan.slots[q].mfma = false;
                lane_q.push_back(q);
            }
        } else {
            lane_q.insert(lane_q.end(), run.begin(), run.end());
        }
        i = j;
    }
    for (int32_t s = 0; s < n_slots; ++s)
        if (plan.slots[s].n == 0) set_chunks(plan.slots[s]);
    for (int32_t q : lane_q) set_chunks(plan.slots[q]);
    if (lane_qb_max > 1) {
        // lane groups need equal chunks too: runs of same rows, split where the chunk changes
        for (size_t i = 0; i < lane_q.size();) {
            size_t j = i + 1;
            while (j < lane_q.size() && same_rows(lane_q[i], lane_q[j])) ++j;
            std::vector<int32_t> run(lane_q.begin() + i, lane_q.begin() + j);
            std::stable_sort(run.begin(), run.end(), [&](int32_t a, int32_t b) {
                return plan.slots[a].chunk < plan.slots[b].chunk;
            });
            int qb = 1;
            group_run(run, lane_qb_max, 2, qb, nullptr);
            if (qb > 1) plan.lanes.QB = lane_qb_max;
            i = j;
        }
    }

    // partial rows: plain rows for the combine kernel, flagged pairs for the single-launch merge
    int64_t part = 0, flagged = 0;
    for (int32_t s = 0; s < n_slots; ++s) {
        SlotPlan &sp = plan.slots[s];
        if (sp.n_chunks <= 1) continue;
        const bool grouped = sp.leader >= 0 || sp.group_n > 1;
        sp.fused = !sp.mfma && !grouped && sp.n_chunks <= plan.fuse_limit;
        if (sp.fused) {
            if (flagged + (int64_t)n_q * sp.n_chunks > INT32_MAX) return "too many split slots";
            sp.flag_row0 = (int32_t)flagged;
            flagged += (int64_t)n_q * sp.n_chunks;
        } else {
            sp.part_row0 = part;
            part += (int64_t)n_q * sp.n_chunks;
        }
    }
    plan.part_rows = part;
    plan.flag_rows = flagged;
    plan.workspace_bytes = flag_region_bytes(flagged, head_dim) +
                           part * (int64_t)(head_dim + 2) * (int64_t)sizeof(float);

    // Work-list order: longest chunks first (ties by slot index), so the
    // longest workgroups start first and short ones fill the tail.  The order
    // decides only which workgroup runs when, never a slot's arithmetic.
    // Matrix-core queries come first (their launches run longer chunks).
    std::vector<int32_t> order;
    for (int32_t s = 0; s < n_slots; ++s)
        if (plan.slots[s].group_n > 0) order.push_back(s);   // leaders and ungrouped queries
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        if (plan.slots[a].mfma != plan.slots[b].mfma) return plan.slots[a].mfma;
        return plan.slots[a].chunk > plan.slots[b].chunk;
    });

    // launch groups: one kernel each, at most kMaxSlotsPerLaunch table entries and
    // kMaxItemsPerLaunch workgroups; a query group's entries (leader, then followers)
    // stay in one launch
    LaunchGroup g;
    for (int32_t s : order) {
        const SlotPlan &sp = plan.slots[s];
        const int n_sub = sp.mfma ? plan.matrix.n_sub : plan.lanes.n_sub;
        // a fused query's merge workgroups count against the launch's workgroups
        const int64_t items = (int64_t)n_kv * n_sub * sp.n_chunks + (sp.fused ? (int64_t)n_q * merge_groups(head_dim) : 0);
        if (items > kMaxItemsPerLaunch) return "too many workgroups for one slot (n_kv_heads too large)";
        const int entries = sp.group_n;
        const bool full = (int)g.slots.size() + entries > kMaxSlotsPerLaunch || g.items + g.tail_rows * merge_groups(head_dim) + items > kMaxItemsPerLaunch ||
                          (!g.slots.empty() && g.mfma != sp.mfma);
        if (full) {
            plan.groups.push_back(g);
            g = LaunchGroup();
        }
        g.mfma = sp.mfma;
        g.slots.push_back(s);
        for (int32_t f : sp.members) g.slots.push_back(f);
        g.items += (int64_t)n_kv * n_sub * sp.n_chunks;
        if (sp.n_chunks > 1) (sp.fused ? g.tail_rows : g.combine_rows) += n_q;
        for (int32_t f : sp.members)
            if (plan.slots[f].n_chunks > 1) g.combine_rows += n_q;   // group members are never fused
    }
    if (!g.slots.empty()) plan.groups.push_back(g);
    for (const LaunchGroup &lg : plan.groups) plan.total_items += lg.items;
    const int one_pass = single_pass_positions(head_dim, byte_v);
    for (LaunchGroup &lg : plan.groups) {
        if (lg.mfma || one_pass == 0 || plan.lanes.QB != 1 || plan.lanes.GB > 2 || lg.items < kSingleMinItems)
            continue;
        bool fits = true;
        for (int32_t s : lg.slots) fits = fits && plan.slots[s].chunk <= one_pass;
        lg.single = fits;
    }
    // a small lane-kernel call without query groups: fewer heads per workgroup, more workgroups
    bool lanes_only = plan.lanes.QB == 1;
    for (const SlotPlan &sp : plan.slots) lanes_only = lanes_only && !sp.mfma;
    if (lanes_only && plan.lanes.GB > 1 && plan.total_items < kSplitHeadsBelowItems)
        return make_plan(spans, n_q, n_kv, head_dim, chunk, merge_mode, plan, path, byte_v, plan.lanes.GB / 2,
                         group_gb > 0 ? group_gb : plan.lanes.GB);
    return "";
}

}  // namespace attn_decode_impl
