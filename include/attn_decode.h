/*
 * attn_decode.h -- C ABI of the MI355X (gfx950) split-KV decode-attention library.
 *
 * One call computes, for every decode slot s and query head h,
 *
 *     out[s,h,:] = sum_j softmax_j(scale * q[s,h,:] . K[s,kvh,j,:]) * V[s,kvh,j,:]
 *
 * with kvh = h / (n_q_heads / n_kv_heads) (consecutive query heads share a KV
 * head), and j over the attended range [lo_s, L_s): lo_s = L_s - window when
 * window > 0 and L_s > window, else 0.  This is the operation of the pages'
 * decode flash-attention kernels: mlx-native 0.21.1 flash_attn_vec_hybrid.metal
 * (flash_attn_vec_hybrid_impl and its batched and GQA-grouped forms: GQA map,
 * sliding-window start, QK dot then scale, online softmax, split-K partials
 * merged by log-sum-exp, S == 0 writing zeros) and tessl 0.2.0 nn.rs
 * (flash_attn_decode: FlashDecoding split over the KV sequence, window 0 =
 * global attention, host-side validation before any dispatch).
 *
 * The K cache is fp16.  The V cache is fp16, or ("hybrid" regime) symmetric
 * int8 codes in blocks of 32 consecutive dims along head_dim with one fp16
 * scale per block: V = code * scale, exact in fp32.  Int8 values must lie
 * within fp16's range (|code * scale| <= 65504): the matrix-core kernel
 * carries them as exact pairs of fp16 values.
 *
 * Memory layout (all device memory unless stated otherwise, caller-owned):
 *   q        fp16  [n_slots][n_q_heads][head_dim], 16-byte aligned
 *   k_cache  fp16  packed ragged slots: slot s is a [n_kv_heads][L_s][head_dim]
 *                  block starting at element sum_{t<s} n_kv_heads*L_t*head_dim;
 *                  16-byte aligned
 *   v_cache  fp16 (v_scales == NULL) or int8 codes, same layout as k_cache;
 *                  16-byte aligned
 *   v_scales fp16  [slot][n_kv_heads][L_s][head_dim/32], packed like k_cache;
 *                  NULL selects fp16 V; 2-byte aligned
 *   seq_lens HOST  int32 [n_slots], each L_s >= 0
 *   out      fp32  [n_slots][n_q_heads][head_dim], 16-byte aligned; must not
 *                  overlap q, k_cache, v_cache or v_scales
 *
 * Execution: every entry point that takes a stream is asynchronous on it
 * (a hipStream_t passed as void*; NULL = the null stream of the current
 * device).  A call enqueues one partial kernel per launch group of up to 256
 * slots (normally one group) and, when some slot is split into several KV
 * chunks, one log-sum-exp combine kernel per such group.  The slot table goes
 * to the kernels by value: 3.4 KB of arguments per launch for groups of up to
 * 48 slots, 18.5 KB for larger ones.  It never
 * synchronises the host and never reads device memory from the host.  Inputs
 * must stay alive and unmodified until the work completes.
 *
 * Workspace: the library keeps one growable buffer per (device, stream): a
 * region of flagged partials used by the single-launch merge mode (zeroed by
 * a fill kernel when the buffer is allocated; every call clears the flags it
 * sets) followed by the per-chunk partials of the combine kernel, which are
 * never zeroed (every partial a merge reads was written by the same call).  A call that
 * needs more than the stream's buffer holds calls hipMalloc for a larger one
 * (so it should not be the call that is captured into a HIP graph: size the
 * workspace with one eager call of the largest shape first); a call that fits
 * only enqueues kernels.  The buffer a workspace outgrows is not freed: it
 * stays allocated until attn_decode_release, so a graph captured on it, work
 * still queued on it, or another host thread calling on the same stream keep
 * a valid buffer.  Calls on different streams use different buffers; calls on
 * the same stream are ordered by it.  attn_decode_release frees every buffer,
 * current and outgrown, after synchronising each device that owns one: a
 * graph captured before it must not be replayed after it.
 *
 * Determinism: the KV split of a slot depends only on that slot's own
 * attended length, head_dim, the V format and the chunk override, so a
 * batched call returns bitwise the same rows as one call per slot, and
 * repeated calls are bitwise identical.
 *
 * Errors: every int-returning entry point returns ATTN_DECODE_OK (0) or a
 * negative code; attn_decode_last_error() then describes the failure (per
 * host thread).  Argument errors are detected before anything is enqueued,
 * so a failed call leaves the stream untouched.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_DECODE_OK 0
#define ATTN_DECODE_EINVAL (-1) /* invalid argument: shape, pointer, alignment, overlap */
#define ATTN_DECODE_ENOMEM (-2) /* workspace allocation failed */
#define ATTN_DECODE_EHIP (-3)   /* a HIP runtime call or kernel launch failed */

/* Largest number of query rows (slots, or cache queries) one kernel launch
 * covers; more are split into several launch groups inside one call. */
#define ATTN_DECODE_MAX_SLOTS_PER_LAUNCH 256
/* Upper bound of KV chunks per slot; the planner widens chunks to stay below. */
#define ATTN_DECODE_MAX_CHUNKS 4096
/* attn_decode_options.chunk value selecting the per-call chunk floor (below). */
#define ATTN_DECODE_CHUNK_PER_CALL (-1)

/*
 * attn_decode -- decode attention for n_slots slots in one call.
 *
 * head_dim must be 64, 128, 256 or 512; n_q_heads a positive multiple of
 * n_kv_heads; window >= 0 (0 = full attention, window >= L_s also means full);
 * scale finite (e.g. 1/sqrt(head_dim)).  A slot with L_s = 0 gets zeros.
 * n_slots = 0 is a no-op that returns 0.  Pointers may be NULL only for
 * arrays with no elements (k_cache/v_cache when every L_s is 0).
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const void *v_scales, const int32_t *seq_lens, int32_t window,
                float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim, float scale, void *stream);

/* Options of attn_decode_ex.  Zero-initialise and set what is needed. */
typedef struct attn_decode_options {
    /* KV positions per chunk: 0 = the planner's choice, which depends on each
     * slot's own length only, so a slot gives bitwise the same result batched
     * or alone; a positive value forces that chunk size for every slot (still
     * widened to keep at most ATTN_DECODE_MAX_CHUNKS chunks per slot), used by
     * tuning sweeps and by the chunking-invariance tests (cf. tessl nn.rs,
     * flash_attn_decode_with_chunk); ATTN_DECODE_CHUNK_PER_CALL = the
     * planner's choice raised to a floor taken from the whole call (its
     * attended positions times n_kv_heads over the workgroups the partial
     * kernel keeps busy: 1024 on the lane kernel, 256 on the matrix cores at
     * head_dim 512, 512 below; a multiple of 64 in [64, 2048]), for throughput
     * on large batches: results then depend on the batch in fp32 rounding
     * (they stay deterministic for a given call).  Other negative values are
     * EINVAL. */
    int32_t chunk;
    /* How a slot split over several chunks is merged: 0 = automatic (today
     * the combine kernel, the faster of the two on MI355X), 1 = the separate
     * combine kernel, 2 = single launch: the lane kernel's queries with at
     * most 64 chunks that are not part of a query group are merged by extra
     * workgroups at the end of the partial kernel's own grid (one launch per
     * call where every split query qualifies), the others by the combine
     * kernel.  Both merges run the same arithmetic in the same order, so the
     * modes give bitwise the same results. */
    int32_t merge_mode;
    /* hipEvent_t handles (as void*) recorded on the stream immediately before
     * the first partial-kernel launch and immediately after the last one, or
     * NULL.  They bracket the partial (KV-streaming) kernels, including the
     * merges of a single-launch call, and exclude the combine kernel. */
    void *ev_partial_begin;
    void *ev_partial_end;
    /* Which partial kernel computes the call: 0 = automatic (the matrix-core
     * kernel wherever it applies, the lane kernel otherwise), 1 = the lane
     * kernel, 2 = the matrix-core kernel (EINVAL unless the query heads per
     * kv head are a multiple of 8 and head_dim >= 128).  The two kernels
     * split a slot into different chunks and differ only in fp32 rounding.
     * The matrix-core kernel always merges split slots in the combine kernel
     * (merge_mode 2 then behaves like 1). */
    int32_t path;
} attn_decode_options;

/* attn_decode with options; opts == NULL behaves exactly like attn_decode. */
int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                   const void *v_scales, const int32_t *seq_lens, int32_t window,
                   float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, float scale, void *stream,
                   const attn_decode_options *opts);

/* Bytes of device scratch attn_decode_noalloc has for a call's partials. */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * attn_decode_noalloc -- attn_decode_ex for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no hipMalloc, hipFree or other allocating
 * routine.  The per-chunk partials go to a fixed device array of
 * ATTN_DECODE_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held
 * until the process ends) instead of a per-stream workspace; a call whose
 * partials need more (attn_decode_plan's workspace_bytes) returns
 * ATTN_DECODE_EINVAL before any GPU work.  Split slots are always merged by
 * the combine kernel (opts->merge_mode 2 is rejected), so the results equal
 * attn_decode_ex's bitwise.  Nothing in the array has to start at zero: every
 * partial a merge reads was written by the same call.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several host threads without ordering) race and
 * must not be issued.  Arguments, layout, asynchrony and errors are as for
 * attn_decode_ex; opts may be NULL.
 */
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                        const void *v_scales, const int32_t *seq_lens, int32_t window,
                        float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, float scale, void *stream,
                        const attn_decode_options *opts);

/*
 * attn_decode_cache -- decode attention over a fixed-capacity KV cache.
 *
 * The cache holds n_cache_slots slots of `capacity` rows per KV head (the
 * layout of mlx-native flash_attn_vec_hybrid.metal's batched kernels, slot
 * offset slot * n_kv * capacity * D):
 *   k_cache  fp16  [n_cache_slots][n_kv_heads][capacity][head_dim]
 *   v_cache  fp16 or int8 codes, same layout; v_scales fp16
 *            [n_cache_slots][n_kv_heads][capacity][head_dim/32] or NULL
 *   q        fp16  [n_queries][n_q_heads][head_dim]; out fp32, same shape
 *   slot_ids HOST  int32 [n_queries]: the cache slot query row i reads
 *   positions HOST int32 [n_queries]: absolute position of query i's token;
 *            it attends positions <= positions[i] (its own K/V row must
 *            already be in the cache)
 * ring = 0: linear storage, position p in row p; positions[i] < capacity.
 * ring = 1: ring storage, position p in row p mod capacity, so only the last
 *           `capacity` positions exist (the pages' sliding-window ring:
 *           kv_seq_len = min(pos + 1, capacity), rows remapped from
 *           ring_start).
 * window > 0 further keeps only the last `window` positions; 0 keeps every
 * stored one.  Several queries may read the same slot, e.g. consecutive
 * positions of draft tokens in a speculative-decoding verify step: each is
 * causal on its own position.  Rows the query does not attend are never read.
 * Alignment, asynchrony, workspace, determinism (per query row) and errors
 * are as for attn_decode; opts may be NULL.
 */
int attn_decode_cache(const void *q, const void *k_cache, const void *v_cache,
                      const void *v_scales, const int32_t *slot_ids, const int32_t *positions,
                      int32_t n_queries, int32_t n_cache_slots, int32_t capacity, int32_t ring,
                      int32_t window, float *out, int32_t n_q_heads, int32_t n_kv_heads,
                      int32_t head_dim, float scale, void *stream,
                      const attn_decode_options *opts);

/*
 * attn_decode_cb -- attn_decode with codebook V (the pages' own hybrid KV
 * regime: mlx-native flash_attn_vec_hybrid.metal, the TQ-HB V layout and its
 * byte-index dequant with 5-, 6- or 8-bit Lloyd-Max codebooks; hf2q gemma4
 * batched_body.rs, the KV encode and the FWHT sign-undo).
 *
 * V is stored in a rotated basis, v_rot = H (s * v) / sqrt(head_dim) (H the
 * Walsh-Hadamard matrix, s a vector of +-1), as one byte per element: the
 * element is
 *     codebook[code & (2^codebook_bits - 1)] * norm[block] / sqrt(B)
 * with B = min(head_dim, 256) and one fp32 norm per block of B consecutive
 * dims (one per row up to head_dim 256, two at 512).  The output is the
 * attention result in the same rotated basis; attn_fwht_undo takes it back.
 *   v_codes   uint8 indices, packed like k_cache; 16-byte aligned
 *   v_norms   fp32 [slot][n_kv_heads][L_s][head_dim / B], packed like
 *             k_cache; 4-byte aligned
 *   codebook  fp32 [2^codebook_bits] levels, device memory; 4-byte aligned
 *   codebook_bits  1..8 (the pages use 5, 6 and 8)
 * The matrix-core kernel carries levels and norm-scaled weights as pairs of
 * fp16 values: levels must stay below 8192 in magnitude and block norms
 * below 16376 (V of rms below about 1000 at 256 dims per block).  Below a
 * norm of about 4 the weights of the less likely keys lose relative
 * precision gradually (measured relative-L2 3e-4 at norm 0.01, under 1e-5
 * from norm 1.6 up).
 * Everything else (q, k_cache, seq_lens, window, out, head_dim, asynchrony,
 * workspace, determinism, errors) is as for attn_decode; opts may be NULL.
 * out must not overlap v_norms or the codebook either.
 */
int attn_decode_cb(const void *q, const void *k_cache, const void *v_codes, const float *v_norms,
                   const float *codebook, int32_t codebook_bits, const int32_t *seq_lens,
                   int32_t window, float *out, int32_t n_slots, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t head_dim, float scale, void *stream,
                   const attn_decode_options *opts);

/*
 * attn_decode_cache_cb -- attn_decode_cache with codebook V (the pages' hybrid
 * KV regime on their fixed-capacity serving cache: mlx-native
 * flash_attn_vec_hybrid.metal, the batched kernels' slot / ring addressing
 * and the TQ-HB V layout; hf2q gemma4 batched_body.rs, the batched flash
 * over slot_id / position tables).
 *   v_codes   uint8 [n_cache_slots][n_kv_heads][capacity][head_dim]; 16-byte aligned
 *   v_norms   fp32  [n_cache_slots][n_kv_heads][capacity][head_dim / B],
 *             B = min(head_dim, 256); 4-byte aligned
 *   codebook, codebook_bits: as for attn_decode_cb (element = level * norm / sqrt(B))
 * Everything else (q, k_cache, slot_ids, positions, ring, window, out, the
 * rotated-basis result, asynchrony, workspace, determinism, errors) is as for
 * attn_decode_cache and attn_decode_cb; opts may be NULL.
 */
int attn_decode_cache_cb(const void *q, const void *k_cache, const void *v_codes, const float *v_norms,
                         const float *codebook, int32_t codebook_bits, const int32_t *slot_ids,
                         const int32_t *positions, int32_t n_queries, int32_t n_cache_slots,
                         int32_t capacity, int32_t ring, int32_t window, float *out, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, float scale, void *stream,
                         const attn_decode_options *opts);

/*
 * attn_fwht_undo -- y = s * (H x) / sqrt(head_dim) per row: the output of
 * attn_decode_cb back in the original basis (hf2q gemma4 batched_body.rs, the
 * FWHT sign-undo after the attention; the inverse of the rotation of codebook
 * V, since H H = head_dim * I).
 *   x, y   fp32 [n_rows][head_dim], device, 16-byte aligned; y == x (in
 *          place) is allowed, any other overlap is rejected
 *   signs  fp32 [head_dim], device, 4-byte aligned: the diagonal s (normally
 *          +-1, the rotation's sign flips)
 * head_dim 64, 128, 256 or 512.  fp32 butterflies: the error is a few fp32
 * ulps of the row's norm.  n_rows = 0 is a no-op.  Asynchronous on `stream`;
 * no workspace.
 */
int attn_fwht_undo(const float *x, const float *signs, float *y, int64_t n_rows, int32_t head_dim,
                   void *stream);

/*
 * attn_kv_append -- write new tokens' K and V into a fixed-capacity cache (the
 * step before decode attention: hf2q gemma4 batched_body.rs, the attention
 * phase's KV encode, an F16 copy of K and the quantisation of V per slot and
 * position).
 *   k_new, v_new  fp32 [n_rows][n_kv_heads][head_dim], 16-byte aligned
 *   k_cache, v_cache, v_scales: the cache of attn_decode_cache (v_scales NULL
 *                 selects fp16 V); written in place
 *   slot_ids, positions HOST int32 [n_rows]: row i goes to cache slot
 *                 slot_ids[i] at position positions[i], i.e. row
 *                 positions[i] (ring = 0, positions[i] < capacity) or
 *                 positions[i] mod capacity (ring = 1)
 * K and fp16 V are rounded to fp16 (nearest even).  int8 V, per block of 32
 * dims: scale = fp16(max|v| / 127), code = clamp(rint(v / scale), -127, 127),
 * all in IEEE fp32 (codes 0 when the scale is 0); finite inputs with
 * |v| <= 127 * 65504.  Two rows may not land on the same cache row (EINVAL).
 * Only the rows named are written.  Asynchronous on `stream`; no workspace.
 */
int attn_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache,
                   void *v_scales, const int32_t *slot_ids, const int32_t *positions,
                   int32_t n_rows, int32_t n_cache_slots, int32_t capacity, int32_t ring,
                   int32_t n_kv_heads, int32_t head_dim, void *stream);

/*
 * attn_kv_append_cb -- attn_kv_append into a cache with codebook V (the
 * hybrid regime's KV encode: hf2q gemma4 batched_body.rs, the F16 copy of K
 * and the FWHT-V encode per slot and position into packed bytes and norms;
 * mlx-native flash_attn_vec_hybrid.metal, the TQ-HB layout with its D = 512
 * per-block norms, which the encode fills).
 *   k_new, v_new  fp32 [n_rows][n_kv_heads][head_dim], 16-byte aligned
 *   k_cache, v_codes, v_norms: the cache of attn_decode_cache_cb, written in
 *                 place (only the rows named)
 *   signs         fp32 [head_dim] (+-1), device, 4-byte aligned: the rotation's
 *                 sign flips (attn_fwht_undo takes results back with the same)
 *   codebook      fp32 [2^codebook_bits], device, 4-byte aligned; the levels
 *                 must increase (otherwise the codes are unspecified but stay
 *                 below 2^codebook_bits); codebook_bits 1..8
 *   slot_ids, positions, ring, capacity: as for attn_kv_append
 * K is rounded to fp16 (nearest even).  Each V row is rotated,
 * y = H (s * v) / sqrt(head_dim) (H the Walsh-Hadamard matrix), split into
 * blocks of B = min(head_dim, 256) coordinates with norm_b = ||y_block||, and
 * each coordinate stored as the index of the level nearest to
 * u = y * sqrt(B) / norm_b (the lower index on a tie; 0 in a block whose norm
 * is 0).  All in fp32: where u lies within fp32 rounding of the midpoint of
 * two levels either index can result.  Finite inputs.  Two rows may not land
 * on the same cache row (EINVAL).  Asynchronous on `stream`; no workspace.
 */
int attn_kv_append_cb(const float *k_new, const float *v_new, void *k_cache, void *v_codes, float *v_norms,
                      const float *signs, const float *codebook, int32_t codebook_bits,
                      const int32_t *slot_ids, const int32_t *positions, int32_t n_rows,
                      int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t n_kv_heads,
                      int32_t head_dim, void *stream);

/*
 * attn_decode_plan -- the host planner alone (no HIP call, usable without a
 * GPU).  For the given shapes it writes, per slot, the KV positions per chunk
 * and the number of chunks (arrays of n_slots, may be NULL), the workspace
 * bytes the call needs and the number of partial-kernel workgroups it
 * launches (may be NULL).  v_int8 != 0 selects the int8 V format (the
 * codebook format, also one byte per element, plans the same).
 * Returns 0 or ATTN_DECODE_EINVAL for shapes attn_decode would reject.
 */
int attn_decode_plan(const int32_t *seq_lens, int32_t n_slots, int32_t window,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int32_t v_int8, int32_t chunk, int32_t *chunk_keys,
                     int32_t *n_chunks, int64_t *workspace_bytes,
                     int64_t *n_partial_workgroups);

/*
 * attn_decode_cache_plan -- the host planner alone for the query rows of an
 * attn_decode_cache / attn_decode_cache_cb call (no HIP call, usable without a
 * GPU).  Arguments are those of the call (slot_ids and positions are host
 * arrays of n_queries) plus v_format: 0 fp16 V, 1 int8 V, 2 codebook V.  Per
 * query it writes the KV positions per chunk, the number of chunks, the partial
 * kernel that computes it (0 the lane kernel, 1 the matrix-core kernel) and the
 * leader of its query group (its own index when it leads a group or is alone):
 * arrays of n_queries, each may be NULL.  It also writes the workspace bytes
 * and the number of partial-kernel workgroups (may be NULL).  Returns 0 or
 * ATTN_DECODE_EINVAL for shapes attn_decode_cache would reject.
 */
int attn_decode_cache_plan(const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
                           int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t window,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t v_format,
                           int32_t chunk, int32_t *chunk_keys, int32_t *n_chunks, int32_t *kernel,
                           int32_t *group_leader, int64_t *workspace_bytes,
                           int64_t *n_partial_workgroups);

/* Message describing the last non-zero return on this host thread ("" if none). */
const char *attn_decode_last_error(void);

/* Free every workspace the library holds (the current buffer of each
 * (device, stream) and every buffer a workspace outgrew), after synchronising
 * each device that owns one.  HIP graphs captured before this call hold the
 * freed addresses and must not be replayed after it.  Later calls allocate
 * again.  Returns 0 or ATTN_DECODE_EHIP. */
int attn_decode_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
