/*
 * attn_decode_oracle.c -- CPU fp64 oracle for single-query (decode) attention
 * over a grouped-query KV cache with an F16 K cache and an F16, block-int8 or
 * codebook V cache, and of the steps around it (the KV append and codebook
 * encode before it, the undo of the codebook rotation after it).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP path is compared against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * constant or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes is the plain definition of the result that the pages'
 * split-KV decode kernels reach up to rounding order:
 *
 *   for each slot s, query head h, dim d:
 *     G    = n_q / n_kv,  kvh = floor(h / G)
 *          (mlx-native flash_attn_vec_hybrid.metal, flash_attn_vec_hybrid_impl,
 *           the GQA head mapping: consecutive query heads share a KV head)
 *     lo   = (W > 0 && L_s > W) ? L_s - W : 0,  hi = L_s
 *          (same kernel, the sliding-window start; tessl nn.rs,
 *           flash_attn_decode: window 0 selects the global rule)
 *     x_j  = scale * sum_d q[s,h,d] * K[s,kvh,j,d]          for j in [lo, hi)
 *          (same kernel, its QK block: the dot is formed first and the
 *           scale is applied to the finished dot)
 *     out  = sum_j exp(x_j - m) V[s,kvh,j,:] / sum_j exp(x_j - m),  m = max x_j
 *          (same kernel, its online-softmax block and the final 1/S normalisation;
 *           an empty range writes zeros because S == 0 gives inv_S = 0)
 *
 * The softmax is evaluated in two exact passes (max, then weights) rather than
 * online; the online form and the split over KV chunks only change rounding.
 *
 * V dequantisation (block-int8 regime): a V element is int8 code times the
 * fp16 scale of its block of 32 consecutive dims along head_dim.  The oracle
 * reads the stored codes and scales and never re-quantises.  The block size
 * and scale type are the library's int8 V format (the pages' own hybrid V is
 * the codebook format, handled by the codebook functions further below).
 *
 * Cache layout (packed ragged slots): slot s's K occupies n_kv * L_s * D
 * elements starting at element offset sum_{t<s} n_kv * L_t * D, laid out
 * [kv_head][pos][dim]; V codes are packed identically; V scales are laid out
 * [kv_head][pos][D/32] per slot, packed the same way.
 *
 * Cache layout (fixed capacity, per query row): query row i reads cache slot
 * slot_ids[i], whose K occupies rows [(slot * n_kv + kvh) * cap, ... + cap)
 * for kv head kvh.  The query's token sits at absolute position
 * positions[i], so it attends positions [lo, positions[i] + 1).  Linear
 * storage keeps position p in row p (p < cap).  Ring storage keeps position p
 * in row p mod cap, so only the last cap positions exist and
 * lo >= positions[i] + 1 - cap (mlx-native flash_attn_vec_hybrid.metal,
 * the batched kernels: kv_seq_len = min(pos + 1, capacity) for the ring,
 * ring_start and the logical-to-physical row remap).
 *
 * All arithmetic is IEEE double.  fp16 -> double is exact (decoded from the
 * bit pattern below).  Built without fast-math and without FP contraction.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE-754 binary16 -> double, exact.  1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 is the subnormal range (no implicit 1, scale
 * 2^-24), exponent 31 is inf / NaN. */
double oracle_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

typedef struct {
    const uint16_t *q;
    const uint16_t *k;
    const void *v;
    const uint16_t *v_scales; /* NULL => V is fp16 (unless codebook != NULL) */
    /* codebook V: byte indices into codebook, one fp32 norm per block of cb_block coordinates */
    const float *codebook;
    const float *v_norms;
    uint32_t cb_mask;
    int32_t cb_block;
    /* packed ragged slots */
    const int32_t *seq_lens;
    const int64_t *slot_first_pos; /* sum of L_t for t < s */
    /* fixed-capacity cache (used when slot_ids != NULL) */
    const int32_t *slot_ids;
    const int32_t *positions;
    int32_t capacity;
    int32_t ring;
    int32_t window;
    double *out;
    int32_t n_slots, n_q, n_kv, d; /* n_slots: query rows (slots or cache queries) */
    double scale;
    const int32_t *rows; /* NULL => every (s, h) row in order */
    int64_t n_rows;
    int n_threads;
    int thread_id;
    int status;
} oracle_job;

/* Attention of one fp16 query over the cache rows row_idx[0..n) (row indices
 * into the K / V-code arrays, in position order) by the plain definition. */
static int oracle_attend(const oracle_job *jb, const uint16_t *qrow, const int64_t *row_idx,
                         int64_t n, double *dst)
{
    const int32_t D = jb->d;
    int d;
    for (d = 0; d < D; ++d) dst[d] = 0.0;
    if (n <= 0) return 0; /* empty range: zeros */

    double *x = (double *)malloc(sizeof(double) * (size_t)n);
    double *qd = (double *)malloc(sizeof(double) * (size_t)D);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    if (!x || !qd || !acc) {
        free(x); free(qd); free(acc);
        return -1;
    }
    for (d = 0; d < D; ++d) { qd[d] = oracle_half_to_double(qrow[d]); acc[d] = 0.0; }

    /* pass 1: logits and their maximum */
    double m = -INFINITY;
    int64_t j;
    for (j = 0; j < n; ++j) {
        const uint16_t *krow = jb->k + row_idx[j] * D;
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += qd[d] * oracle_half_to_double(krow[d]);
        x[j] = jb->scale * dot;
        if (x[j] > m) m = x[j];
    }

    /* pass 2: weights, their sum, and the weighted sum of dequantised V */
    double Z = 0.0;
    for (j = 0; j < n; ++j) {
        const double w = exp(x[j] - m);
        Z += w;
        if (jb->codebook != NULL) {
            const uint8_t *vrow = (const uint8_t *)jb->v + row_idx[j] * D;
            const float *nrow = jb->v_norms + row_idx[j] * (D / jb->cb_block);
            const double inv_sqrt_b = 1.0 / sqrt((double)jb->cb_block);
            for (d = 0; d < D; ++d) {
                const double vdq = (double)jb->codebook[vrow[d] & jb->cb_mask] *
                                   (double)nrow[d / jb->cb_block] * inv_sqrt_b;
                acc[d] += w * vdq;
            }
        } else if (jb->v_scales == NULL) {
            const uint16_t *vrow = (const uint16_t *)jb->v + row_idx[j] * D;
            for (d = 0; d < D; ++d) acc[d] += w * oracle_half_to_double(vrow[d]);
        } else {
            const int8_t *vrow = (const int8_t *)jb->v + row_idx[j] * D;
            const uint16_t *srow = jb->v_scales + row_idx[j] * (D / 32);
            for (d = 0; d < D; ++d) {
                const double vdq = (double)vrow[d] * oracle_half_to_double(srow[d / 32]);
                acc[d] += w * vdq;
            }
        }
    }
    for (d = 0; d < D; ++d) dst[d] = acc[d] / Z;

    free(x); free(qd); free(acc);
    return 0;
}

/* One output row (query row s, query head h): list the attended cache rows, then attend. */
static int oracle_row(const oracle_job *jb, int64_t row, double *dst)
{
    const int32_t s = (int32_t)(row / jb->n_q);
    const int32_t h = (int32_t)(row % jb->n_q);
    const int32_t G = jb->n_q / jb->n_kv;
    const int32_t kvh = h / G;
    const int32_t W = jb->window;
    const uint16_t *qrow = jb->q + ((int64_t)s * jb->n_q + h) * jb->d;
    int64_t L, lo, base, p;

    if (jb->slot_ids == NULL) {
        /* packed ragged slots: position p of (s, kvh) is row n_kv * first[s] + kvh * L + p */
        L = jb->seq_lens[s];
        lo = (W > 0 && L > W) ? L - W : 0;
        base = (int64_t)jb->n_kv * jb->slot_first_pos[s] + (int64_t)kvh * L;
    } else {
        /* fixed-capacity cache: position p of (slot, kvh) is row (slot*n_kv + kvh)*cap + phys(p) */
        const int64_t cap = jb->capacity;
        L = (int64_t)jb->positions[s] + 1;
        lo = 0;
        if (jb->ring && L > cap) lo = L - cap;
        if (W > 0 && L - W > lo) lo = L - W;
        base = ((int64_t)jb->slot_ids[s] * jb->n_kv + kvh) * cap;
    }
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > lo ? L - lo : 1));
    if (!idx) return -1;
    for (p = lo; p < L; ++p) {
        int64_t phys = p;
        if (jb->slot_ids != NULL && jb->ring) phys = p % jb->capacity;
        idx[p - lo] = base + phys;
    }
    const int rc = oracle_attend(jb, qrow, idx, L - lo, dst);
    free(idx);
    return rc;
}

static void *oracle_worker(void *arg)
{
    oracle_job *jb = (oracle_job *)arg;
    int64_t i;
    for (i = jb->thread_id; i < jb->n_rows; i += jb->n_threads) {
        const int64_t row = jb->rows ? (int64_t)jb->rows[i] : i;
        if (oracle_row(jb, row, jb->out + i * jb->d) != 0) {
            jb->status = -2;
            break;
        }
    }
    return NULL;
}

static int oracle_run(oracle_job *proto, int32_t n_threads)
{
    int t;
    oracle_job *jobs = (oracle_job *)malloc(sizeof(oracle_job) * (size_t)n_threads);
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!jobs || !tids) {
        free(jobs); free(tids);
        return -2;
    }
    for (t = 0; t < n_threads; ++t) {
        jobs[t] = *proto;
        jobs[t].n_threads = n_threads;
        jobs[t].thread_id = t;
        jobs[t].status = 0;
    }
    int started = 0;
    for (t = 1; t < n_threads; ++t) {
        if (pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) != 0) break;
        started = t;
    }
    /* threads that failed to start: run their share here */
    for (t = started + 1; t < n_threads; ++t) oracle_worker(&jobs[t]);
    oracle_worker(&jobs[0]);
    for (t = 1; t <= started; ++t) pthread_join(tids[t], NULL);

    int status = 0;
    for (t = 0; t < n_threads; ++t)
        if (jobs[t].status != 0) status = jobs[t].status;
    free(jobs); free(tids);
    return status;
}

static int check_rows(const int32_t *rows, int64_t n_rows, int64_t n_all)
{
    int64_t i;
    if (rows == NULL) return 0;
    for (i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= n_all) return -1;
    return 0;
}

/*
 * oracle_attn_decode_f64 -- packed ragged slots
 *   q         fp16 bits [n_slots][n_q][D]
 *   k         fp16 bits, packed ragged [slot][n_kv][L_s][D]
 *   v         fp16 bits (v_scales == NULL) or int8 codes, same layout as k
 *   v_scales  fp16 bits [slot][n_kv][L_s][D/32], or NULL
 *   seq_lens  [n_slots], each >= 0
 *   window    0 = full attention, W > 0 = last W positions
 *   out       double [n_rows][D] where row i is rows[i] (= s * n_q + h),
 *             or [n_slots][n_q][D] when rows == NULL
 *   n_threads worker threads (>= 1)
 * Returns 0, -1 for invalid arguments, -2 for allocation failure.
 */
int oracle_attn_decode_f64(const uint16_t *q, const uint16_t *k, const void *v,
                           const uint16_t *v_scales, const int32_t *seq_lens,
                           int32_t window, double *out, int32_t n_slots,
                           int32_t n_q, int32_t n_kv, int32_t head_dim, float scale,
                           const int32_t *rows, int64_t n_rows, int32_t n_threads)
{
    int32_t s;
    if (n_slots < 0 || n_q <= 0 || n_kv <= 0 || head_dim <= 0 || window < 0) return -1;
    if (n_q % n_kv != 0) return -1;
    if (v_scales != NULL && head_dim % 32 != 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (rows == NULL) n_rows = (int64_t)n_slots * n_q;
    if (n_rows == 0) return 0;
    for (s = 0; s < n_slots; ++s)
        if (seq_lens[s] < 0) return -1;
    if (check_rows(rows, n_rows, (int64_t)n_slots * n_q) != 0) return -1;

    int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_slots + 1));
    if (!first) return -2;
    first[0] = 0;
    for (s = 0; s < n_slots; ++s) first[s + 1] = first[s] + seq_lens[s];

    oracle_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v; jb.v_scales = v_scales;
    jb.seq_lens = seq_lens; jb.slot_first_pos = first; jb.window = window;
    jb.out = out; jb.n_slots = n_slots; jb.n_q = n_q; jb.n_kv = n_kv;
    jb.d = head_dim; jb.scale = (double)scale; jb.rows = rows; jb.n_rows = n_rows;
    const int status = oracle_run(&jb, n_threads);
    free(first);
    return status;
}

/*
 * oracle_attn_decode_cache_f64 -- fixed-capacity (linear or ring) cache
 *   q          fp16 bits [n_queries][n_q][D]
 *   k          fp16 bits [n_cache_slots][n_kv][capacity][D]
 *   v          fp16 bits (v_scales == NULL) or int8 codes, same layout as k
 *   v_scales   fp16 bits [n_cache_slots][n_kv][capacity][D/32], or NULL
 *   slot_ids   [n_queries], each in [0, n_cache_slots)
 *   positions  [n_queries], each >= 0; < capacity when ring == 0
 *   ring       0 = linear storage (row p), 1 = ring storage (row p mod capacity)
 *   window     0 = every stored position, W > 0 = last W positions
 *   out, rows, n_rows, n_threads as for oracle_attn_decode_f64 (row i = query * n_q + h)
 */
int oracle_attn_decode_cache_f64(const uint16_t *q, const uint16_t *k, const void *v,
                                 const uint16_t *v_scales, const int32_t *slot_ids,
                                 const int32_t *positions, int32_t n_queries,
                                 int32_t n_cache_slots, int32_t capacity, int32_t ring,
                                 int32_t window, double *out, int32_t n_q, int32_t n_kv,
                                 int32_t head_dim, float scale, const int32_t *rows,
                                 int64_t n_rows, int32_t n_threads)
{
    int32_t i;
    if (n_queries < 0 || n_cache_slots < 0 || capacity <= 0 || n_q <= 0 || n_kv <= 0 ||
        head_dim <= 0 || window < 0 || (ring != 0 && ring != 1))
        return -1;
    if (n_q % n_kv != 0) return -1;
    if (v_scales != NULL && head_dim % 32 != 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (rows == NULL) n_rows = (int64_t)n_queries * n_q;
    if (n_rows == 0) return 0;
    for (i = 0; i < n_queries; ++i) {
        if (slot_ids[i] < 0 || slot_ids[i] >= n_cache_slots) return -1;
        if (positions[i] < 0 || (!ring && positions[i] >= capacity)) return -1;
    }
    if (check_rows(rows, n_rows, (int64_t)n_queries * n_q) != 0) return -1;

    oracle_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v; jb.v_scales = v_scales;
    jb.slot_ids = slot_ids; jb.positions = positions; jb.capacity = capacity; jb.ring = ring;
    jb.window = window; jb.out = out; jb.n_slots = n_queries; jb.n_q = n_q; jb.n_kv = n_kv;
    jb.d = head_dim; jb.scale = (double)scale; jb.rows = rows; jb.n_rows = n_rows;
    return oracle_run(&jb, n_threads);
}

/*
 * oracle_attn_decode_cb_f64 -- packed ragged slots with codebook V (the pages'
 * hybrid regime: F16 K, V stored rotated as byte indices into a codebook with
 * one fp32 norm per block of B = min(D, 256) coordinates; mlx-native
 * flash_attn_vec_hybrid.metal, dequant_hb_single and the D = 512 per-block
 * norms).  V[j][d] = codebook[code & (2^bits - 1)] * norm[j][d / B] / sqrt(B).
 * The result is in the rotated basis (see oracle_fwht_undo_f64).
 *   v_codes  uint8 packed like k; v_norms fp32 [rows][D / B]; codebook fp32 [2^bits]
 */
int oracle_attn_decode_cb_f64(const uint16_t *q, const uint16_t *k, const uint8_t *v_codes,
                              const float *v_norms, const float *codebook, int32_t codebook_bits,
                              const int32_t *seq_lens, int32_t window, double *out,
                              int32_t n_slots, int32_t n_q, int32_t n_kv, int32_t head_dim,
                              float scale, const int32_t *rows, int64_t n_rows, int32_t n_threads)
{
    int32_t s;
    if (n_slots < 0 || n_q <= 0 || n_kv <= 0 || head_dim <= 0 || window < 0) return -1;
    if (n_q % n_kv != 0) return -1;
    if (codebook_bits < 1 || codebook_bits > 8) return -1;
    const int32_t B = head_dim < 256 ? head_dim : 256;
    if (head_dim % B != 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (rows == NULL) n_rows = (int64_t)n_slots * n_q;
    if (n_rows == 0) return 0;
    for (s = 0; s < n_slots; ++s)
        if (seq_lens[s] < 0) return -1;
    if (check_rows(rows, n_rows, (int64_t)n_slots * n_q) != 0) return -1;

    int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_slots + 1));
    if (!first) return -2;
    first[0] = 0;
    for (s = 0; s < n_slots; ++s) first[s + 1] = first[s] + seq_lens[s];

    oracle_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v_codes; jb.v_scales = NULL;
    jb.codebook = codebook; jb.v_norms = v_norms;
    jb.cb_mask = (1u << codebook_bits) - 1u; jb.cb_block = B;
    jb.seq_lens = seq_lens; jb.slot_first_pos = first; jb.window = window;
    jb.out = out; jb.n_slots = n_slots; jb.n_q = n_q; jb.n_kv = n_kv;
    jb.d = head_dim; jb.scale = (double)scale; jb.rows = rows; jb.n_rows = n_rows;
    const int status = oracle_run(&jb, n_threads);
    free(first);
    return status;
}

/* Entry (i, j) of the unnormalised Walsh-Hadamard matrix of order 2^k: (-1)^popcount(i & j). */
static int hadamard_sign(uint32_t i, uint32_t j)
{
    uint32_t x = i & j;
    int parity = 0;
    while (x) { parity ^= 1; x &= x - 1; }
    return parity ? -1 : 1;
}

/*
 * oracle_fwht_undo_f64 -- back from the rotated basis: the rotation is
 * v_rot = H (s * v) / sqrt(D) with H the Walsh-Hadamard matrix (symmetric,
 * H H = D I) and s a vector of +-1, so v = s * (H v_rot) / sqrt(D)
 * (hf2q gemma4 batched_body.rs, the FWHT sign-undo after the attention).
 *   x, y  double [n_rows][D] (y may equal x); signs float +-1 [D]; D a power of two
 */
int oracle_fwht_undo_f64(const double *x, const float *signs, double *y, int64_t n_rows, int32_t head_dim)
{
    int64_t r;
    int32_t i, j;
    if (head_dim <= 0 || (head_dim & (head_dim - 1)) != 0 || n_rows < 0) return -1;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)head_dim);
    if (!tmp) return -2;
    const double inv = 1.0 / sqrt((double)head_dim);
    for (r = 0; r < n_rows; ++r) {
        const double *xr = x + r * head_dim;
        for (i = 0; i < head_dim; ++i) {
            double acc = 0.0;
            for (j = 0; j < head_dim; ++j) acc += hadamard_sign((uint32_t)i, (uint32_t)j) * xr[j];
            tmp[i] = (double)signs[i] * acc * inv;
        }
        memcpy(y + r * head_dim, tmp, sizeof(double) * (size_t)head_dim);
    }
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------
 * KV append: the step before the path.  Each new token's K is stored as fp16
 * and its V as fp16 or as symmetric int8 codes in blocks of 32 dims with one
 * fp16 scale (the library's int8 V format), into the cache row of its (slot,
 * position): row p for linear storage, row p mod capacity for a ring
 * (mlx-native flash_attn_vec_hybrid.metal, batched kernels: physical row of a
 * position; hf2q gemma4 batched_body.rs, the attention phase's KV encode:
 * F16 copy of K and quantisation of V per slot and position).
 *
 * Quantisation of one block b of 32 float values (every rounding decision in
 * IEEE single precision, round to nearest even):
 *   amax  = max_i |b_i|
 *   scale = fp16(amax / 127)
 *   code  = clamp(rint(b_i / (float)scale), -127, 127), or 0 when scale == 0
 * ------------------------------------------------------------------------ */

/* IEEE-754 single -> binary16, round to nearest, ties to even (from the
 * formats' definitions: 1 sign, 5 exponent bits with bias 15, 10 fraction
 * bits; subnormals below 2^-14; overflow to infinity). */
uint16_t oracle_float_to_half(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const uint32_t absx = x & 0x7fffffffu;
    if (absx >= 0x7f800000u) /* inf or NaN */
        return (uint16_t)(sign | 0x7c00u | (absx > 0x7f800000u ? 0x200u : 0u));
    const int e = (int)(absx >> 23) - 127; /* unbiased exponent */
    uint32_t mant = (absx & 0x7fffffu) | (absx >= 0x00800000u ? 0x800000u : 0u); /* 24-bit significand */
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    int shift; /* bits of the 24-bit significand dropped to reach the 11-bit (normal) or fewer (subnormal) */
    uint32_t exp_field;
    if (e >= -14) {
        shift = 13;
        exp_field = (uint32_t)(e + 15);
    } else {
        shift = 13 + (-14 - e); /* subnormal: value = m * 2^-24 */
        exp_field = 0;
        if (shift > 24) return sign; /* below half the smallest subnormal: +-0 */
    }
    uint32_t q = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    /* q carries the implicit bit for normals; a carry out of the significand bumps the exponent */
    uint32_t h;
    if (exp_field == 0) {
        h = q; /* may round up into the smallest normal: encoding 0x400 is exactly that */
    } else {
        h = ((exp_field << 10) + (q - 0x400u)); /* q in [0x400, 0x800]; 0x800 carries into the exponent */
        if (q == 0x800u) h = (exp_field + 1u) << 10;
        if (h >= 0x7c00u) h = 0x7c00u;
    }
    return (uint16_t)(sign | h);
}

/* Quantises one block of 32 values; returns the fp16 scale bits. */
static uint16_t oracle_quantize_block(const float *b, int8_t *codes)
{
    float amax = 0.0f;
    int i;
    for (i = 0; i < 32; ++i) {
        const float a = fabsf(b[i]);
        if (a > amax) amax = a;
    }
    const uint16_t s16 = oracle_float_to_half(amax / 127.0f);
    const float s = (float)oracle_half_to_double(s16);
    for (i = 0; i < 32; ++i) {
        if (s == 0.0f) {
            codes[i] = 0;
        } else {
            float c = rintf(b[i] / s);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            codes[i] = (int8_t)c;
        }
    }
    return s16;
}

static int check_append(const int32_t *slot_ids, const int32_t *positions, int32_t n_rows,
                        int32_t n_cache_slots, int32_t capacity, int32_t ring);

/* Exposed for pinning: quantises n_blocks blocks of 32 floats. */
void oracle_quantize_blocks(const float *v, int64_t n_blocks, int8_t *codes, uint16_t *scales)
{
    int64_t b;
    for (b = 0; b < n_blocks; ++b) scales[b] = oracle_quantize_block(v + b * 32, codes + b * 32);
}

/*
 * oracle_kv_append -- writes n_rows new tokens into a host copy of the cache.
 *   k_new, v_new  float [n_rows][n_kv][D]
 *   k_cache       fp16 bits [n_cache_slots][n_kv][capacity][D]
 *   v_cache       fp16 bits (v_scales == NULL) or int8 codes, same layout
 *   v_scales      fp16 bits [n_cache_slots][n_kv][capacity][D/32] or NULL
 * Returns 0, or -1 for invalid arguments (including two rows landing on one cache row).
 */
int oracle_kv_append(const float *k_new, const float *v_new, uint16_t *k_cache, void *v_cache,
                     uint16_t *v_scales, const int32_t *slot_ids, const int32_t *positions,
                     int32_t n_rows, int32_t n_cache_slots, int32_t capacity, int32_t ring,
                     int32_t n_kv, int32_t head_dim)
{
    int32_t i;
    if (n_rows < 0 || n_cache_slots < 0 || capacity <= 0 || n_kv <= 0 || head_dim <= 0) return -1;
    if (ring != 0 && ring != 1) return -1;
    if (v_scales != NULL && head_dim % 32 != 0) return -1;
    if (check_append(slot_ids, positions, n_rows, n_cache_slots, capacity, ring) != 0) return -1;
    const int32_t D = head_dim;
    for (i = 0; i < n_rows; ++i) {
        const int64_t phys = ring ? positions[i] % capacity : positions[i];
        int32_t h;
        for (h = 0; h < n_kv; ++h) {
            const int64_t row = ((int64_t)slot_ids[i] * n_kv + h) * capacity + phys;
            const float *ks = k_new + ((int64_t)i * n_kv + h) * D;
            const float *vs = v_new + ((int64_t)i * n_kv + h) * D;
            int32_t d;
            for (d = 0; d < D; ++d) k_cache[row * D + d] = oracle_float_to_half(ks[d]);
            if (v_scales == NULL) {
                uint16_t *vr = (uint16_t *)v_cache + row * D;
                for (d = 0; d < D; ++d) vr[d] = oracle_float_to_half(vs[d]);
            } else {
                int8_t *vr = (int8_t *)v_cache + row * D;
                int32_t b;
                for (b = 0; b < D / 32; ++b)
                    v_scales[row * (D / 32) + b] = oracle_quantize_block(vs + 32 * b, vr + 32 * b);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Codebook V: the fixed-capacity cache and the encode of new rows (the
 * hybrid regime's KV encode: hf2q gemma4 batched_body.rs, the attention
 * phase's F16 copy of K and FWHT-V encode per slot and position into packed
 * bytes plus norms; mlx-native flash_attn_vec_hybrid.metal, the TQ-HB V
 * layout and the D = 512 per-block norms that the encode must produce).  The
 * pages give the call and the layout it fills, not the encode's steps; the
 * plain reading, taken here, is to rotate the row, take each block's norm,
 * and quantise each normalised coordinate to its nearest level:
 *   y      = H (s * v) / sqrt(D)       (H by its entries, see hadamard_sign)
 *   norm_b = sqrt(sum_{i in block b} y_i^2),     blocks of B = min(D, 256)
 *   u_i    = y_i * sqrt(B) / norm_b              (0 when norm_b == 0)
 *   code_i = argmin_j |u_i - codebook[j]|, j < 2^bits, lowest j on a tie
 *            (0 when norm_b == 0: every level then decodes to 0)
 * so that codebook[code_i] * norm_b / sqrt(B) ~ y_i, the decode of
 * oracle_attend.  Norms are stored as float (rounded from double).
 * ------------------------------------------------------------------------ */

/* Encodes one row of D floats; u_out (may be NULL) receives the u_i in double. */
static int oracle_encode_row(const float *v, const float *signs, const float *codebook, int32_t n_levels,
                             int32_t D, uint8_t *codes, float *norms, double *u_out)
{
    const int32_t B = D < 256 ? D : 256;
    int32_t i, j, b;
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    if (!y) return -2;
    const double inv = 1.0 / sqrt((double)D);
    for (i = 0; i < D; ++i) {
        double acc = 0.0;
        for (j = 0; j < D; ++j) acc += hadamard_sign((uint32_t)i, (uint32_t)j) * (double)signs[j] * (double)v[j];
        y[i] = acc * inv;
    }
    for (b = 0; b < D / B; ++b) {
        double ss = 0.0;
        for (i = b * B; i < (b + 1) * B; ++i) ss += y[i] * y[i];
        const double nb = sqrt(ss);
        norms[b] = (float)nb;
        for (i = b * B; i < (b + 1) * B; ++i) {
            const double u = nb == 0.0 ? 0.0 : y[i] * sqrt((double)B) / nb;
            int32_t best = 0;
            if (nb != 0.0) {
                double dbest = fabs(u - (double)codebook[0]);
                for (j = 1; j < n_levels; ++j) {
                    const double dj = fabs(u - (double)codebook[j]);
                    if (dj < dbest) { dbest = dj; best = j; }
                }
            }
            codes[i] = (uint8_t)best;
            if (u_out) u_out[i] = u;
        }
    }
    free(y);
    return 0;
}

/*
 * oracle_codebook_encode_f64 -- the encode above on n_rows rows.
 *   v      float [n_rows][D]; signs float [D]; codebook float [2^bits]
 *   codes  uint8 [n_rows][D]; norms float [n_rows][D / B]; u double [n_rows][D] or NULL
 * D a power of two; bits 1..8.  Returns 0, -1 for invalid arguments, -2 for allocation failure.
 */
int oracle_codebook_encode_f64(const float *v, const float *signs, const float *codebook, int32_t bits,
                               int64_t n_rows, int32_t head_dim, uint8_t *codes, float *norms, double *u)
{
    int64_t r;
    if (head_dim <= 0 || (head_dim & (head_dim - 1)) != 0 || n_rows < 0) return -1;
    if (bits < 1 || bits > 8) return -1;
    const int32_t B = head_dim < 256 ? head_dim : 256;
    for (r = 0; r < n_rows; ++r) {
        const int rc = oracle_encode_row(v + r * head_dim, signs, codebook, 1 << bits, head_dim,
                                         codes + r * head_dim, norms + r * (head_dim / B),
                                         u ? u + r * head_dim : NULL);
        if (rc != 0) return rc;
    }
    return 0;
}

/* Checks of an append's placement shared by both V formats: every row names a
 * slot in range and a storable position, and no two rows share a cache row. */
static int check_append(const int32_t *slot_ids, const int32_t *positions, int32_t n_rows,
                        int32_t n_cache_slots, int32_t capacity, int32_t ring)
{
    int32_t i, j;
    for (i = 0; i < n_rows; ++i) {
        if (slot_ids[i] < 0 || slot_ids[i] >= n_cache_slots || positions[i] < 0) return -1;
        if (!ring && positions[i] >= capacity) return -1;
        for (j = 0; j < i; ++j) {
            const int64_t ri = ring ? positions[i] % capacity : positions[i];
            const int64_t rj = ring ? positions[j] % capacity : positions[j];
            if (slot_ids[i] == slot_ids[j] && ri == rj) return -1;
        }
    }
    return 0;
}

/*
 * oracle_kv_append_cb -- writes n_rows new tokens into a host copy of a cache
 * with codebook V: K as fp16, V encoded as above into the row of its (slot,
 * position) (row p linear, p mod capacity ring).
 *   k_new, v_new  float [n_rows][n_kv][D]; signs float [D]; codebook float [2^bits]
 *   k_cache fp16 bits, v_codes uint8 [n_cache_slots][n_kv][capacity][D];
 *   v_norms float [n_cache_slots][n_kv][capacity][D / B]
 *   u_out   double [n_rows][n_kv][D] or NULL: the normalised coordinates
 * Returns 0, -1 for invalid arguments (including two rows on one cache row), -2 on allocation failure.
 */
int oracle_kv_append_cb(const float *k_new, const float *v_new, const float *signs, const float *codebook,
                        int32_t bits, uint16_t *k_cache, uint8_t *v_codes, float *v_norms,
                        const int32_t *slot_ids, const int32_t *positions, int32_t n_rows,
                        int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t n_kv,
                        int32_t head_dim, double *u_out)
{
    int32_t i, h, d;
    if (n_rows < 0 || n_cache_slots < 0 || capacity <= 0 || n_kv <= 0) return -1;
    if (head_dim <= 0 || (head_dim & (head_dim - 1)) != 0) return -1;
    if (ring != 0 && ring != 1) return -1;
    if (bits < 1 || bits > 8) return -1;
    if (check_append(slot_ids, positions, n_rows, n_cache_slots, capacity, ring) != 0) return -1;
    const int32_t D = head_dim;
    const int32_t B = D < 256 ? D : 256;
    for (i = 0; i < n_rows; ++i) {
        const int64_t phys = ring ? positions[i] % capacity : positions[i];
        for (h = 0; h < n_kv; ++h) {
            const int64_t row = ((int64_t)slot_ids[i] * n_kv + h) * capacity + phys;
            const int64_t src = ((int64_t)i * n_kv + h) * D;
            for (d = 0; d < D; ++d) k_cache[row * D + d] = oracle_float_to_half(k_new[src + d]);
            const int rc = oracle_encode_row(v_new + src, signs, codebook, 1 << bits, D, v_codes + row * D,
                                             v_norms + row * (D / B), u_out ? u_out + src : NULL);
            if (rc != 0) return rc;
        }
    }
    return 0;
}

/*
 * oracle_attn_decode_cache_cb_f64 -- oracle_attn_decode_cache_f64 with codebook
 * V (decoded as in oracle_attn_decode_cb_f64; the result is in the rotated basis).
 *   v_codes uint8 [n_cache_slots][n_kv][capacity][D]; v_norms float [..][capacity][D / B]
 */
int oracle_attn_decode_cache_cb_f64(const uint16_t *q, const uint16_t *k, const uint8_t *v_codes,
                                    const float *v_norms, const float *codebook, int32_t codebook_bits,
                                    const int32_t *slot_ids, const int32_t *positions,
                                    int32_t n_queries, int32_t n_cache_slots, int32_t capacity,
                                    int32_t ring, int32_t window, double *out, int32_t n_q,
                                    int32_t n_kv, int32_t head_dim, float scale, const int32_t *rows,
                                    int64_t n_rows, int32_t n_threads)
{
    int32_t i;
    if (n_queries < 0 || n_cache_slots < 0 || capacity <= 0 || n_q <= 0 || n_kv <= 0 ||
        head_dim <= 0 || window < 0 || (ring != 0 && ring != 1))
        return -1;
    if (n_q % n_kv != 0) return -1;
    if (codebook_bits < 1 || codebook_bits > 8) return -1;
    const int32_t B = head_dim < 256 ? head_dim : 256;
    if (head_dim % B != 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (rows == NULL) n_rows = (int64_t)n_queries * n_q;
    if (n_rows == 0) return 0;
    for (i = 0; i < n_queries; ++i) {
        if (slot_ids[i] < 0 || slot_ids[i] >= n_cache_slots) return -1;
        if (positions[i] < 0 || (!ring && positions[i] >= capacity)) return -1;
    }
    if (check_rows(rows, n_rows, (int64_t)n_queries * n_q) != 0) return -1;

    oracle_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v_codes; jb.v_scales = NULL;
    jb.codebook = codebook; jb.v_norms = v_norms;
    jb.cb_mask = (1u << codebook_bits) - 1u; jb.cb_block = B;
    jb.slot_ids = slot_ids; jb.positions = positions; jb.capacity = capacity; jb.ring = ring;
    jb.window = window; jb.out = out; jb.n_slots = n_queries; jb.n_q = n_q; jb.n_kv = n_kv;
    jb.d = head_dim; jb.scale = (double)scale; jb.rows = rows; jb.n_rows = n_rows;
    return oracle_run(&jb, n_threads);
}
