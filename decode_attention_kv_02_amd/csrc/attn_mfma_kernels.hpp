// attn_mfma_kernels.hpp -- gfx950 partial kernel for up to 16 (query, head)
// columns per workgroup, on the matrix cores: 8 or 16 query heads of one kv
// head, every head of the kv head for each of a slot's draft queries (a
// speculative-verify step), or the 4 to 7 heads of one query.
//
// Same operation and partial format as attn_partial_kernel (one chunk of one
// (slot, kv head): out = O / S, or O and (M, S) for the log-sum-exp merge;
// mlx-native flash_attn_vec_hybrid.metal, flash_attn_vec_hybrid_batched_gqa_impl:
// every K and V row is read once for all the query heads of the group).  With
// 8 or more heads per kv head the per-lane dot products and V FMAs of the
// lane kernel make it VALU-bound, so here both products are MFMA tiles.
//
//  * The 4 waves split the chunk's keys (the pages' simdgroups splitting the
//    KV range, merged at the end): wave w takes the 16-key tiles w, w + 4,
//    w + 8, ... and runs its own online softmax, with no barrier until the
//    final merge of the 4 waves' (M, S, O) through LDS.
//  * S^T (16 keys x 16 heads) = K q^T on v_mfma_f32_16x16x32_f16: A = K rows
//    (key l%16, 8 dims per lane per step, one 16-byte load), B = q.  fp16
//    products are exact, the accumulation fp32.
//  * O^T (dims x heads) += V^T P^T on v_mfma_f32_16x16x16_f16, with both
//    operands straight from registers.  Lane l loads keys 4(l/16) + j,
//    j = 0..3, each EV consecutive dims starting at EV (l%16) (16 bytes); the
//    S^T accumulator gives it P of the same four keys for head l%16, which is
//    the B operand B[4(l/16) + j][l%16].  The A operand A[l%16][4(l/16) + j]
//    is then element e of load j, so instruction e covers the tile's 16 keys
//    for dims EV (l%16) + e: the same for every lane with that l%16, and the
//    accumulators cover every dim once.  Each V load reads 4 keys x 16 EV
//    contiguous bytes, whole cache lines; V is never staged in LDS.  P and V
//    enter as fp16 pairs hi + lo that carry about 22 bits (fp16 V as it is,
//    int8 code x scale exactly), the products are exact and the accumulation
//    fp32.
//  * Accumulator o[b EV + e] lane l component r holds head l%16, dim
//    BW b + 4 EV (l/16) + EV r + e (BW = 16 EV dims per load).
//  * At head_dim 512 the workgroup has 8 waves in two halves (mfma_dim_splits):
//    waves w and w + 4 take the same key tiles; each loads K for 256 of the
//    dims and sums its QK steps, the two halves of S^T are added through LDS
//    (both waves form lower + upper, the same bits), and each accumulates O
//    for 256 of the output dims.  Accumulators and V buffers halve, so two
//    waves run per SIMD instead of one (graph-replayed, 8 x 32768, 16 q / 2 kv
//    heads: codebook V 176.4 -> 145.3 us, int8 165.7 -> 150.9, fp16
//    174.0 -> 169.2).  Two sibling workgroups that each computed the whole
//    QK product measured 166.0 and 162.2 us (their second K read hit L2);
//    four, 1.8 times slower; a second K buffer spills.
//
// Lane layouts (checked on gfx950 with one-wave probes): 16x16x32 f16:
// A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]; 16x16x16 f16: A[l%16][4(l/16)+e],
// B[4(l/16)+e][l%16]; both C[4(l/16)+i][l%16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode_kernels.hpp"

namespace attn_decode_impl {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaKeys = 16;   // keys per tile (the MFMA M / N size)
constexpr float kLazyMax = 8.f; // log2 headroom of the softmax reference before a rescale

template <int D, int VF>
struct MfmaGeometry {
    static_assert(D >= 128 && D <= 512, "head_dim 128..512");
    static constexpr int KS = D / 32;                                    // QK steps = 16-byte K loads per lane
    static constexpr int DS = mfma_dim_splits(D);                       // waves sharing a key tile, by dims
    static constexpr int DH = D / DS;                                    // output dims of one wave
    static constexpr int THREADS = kThreads * DS;                        // DS groups of kWaves waves
    static constexpr int KW = KS / DS;                                   // QK steps of one wave
    static constexpr int EV = (VF == kVF16) ? 8 : (DH >= 256 ? 16 : 8);  // V elements per lane per load
    static constexpr int BW = 16 * EV;                                   // dims covered by one load
    static constexpr int NB = DH / BW;                                   // loads per key step
    static constexpr int VBYTES = EV * (VF == kVF16 ? 2 : 1);            // 16, or 8 (byte V at D = 128)
    static constexpr int NO = NB * EV;                                   // f32x4 accumulators = DH / 16
    static_assert(NO * 16 == DH, "accumulators cover every dim of the wave once");
    static_assert(VF != kVCB || (D < 256 ? D : 256) % BW == 0, "one codebook norm block per load");
    // Workgroups per CU the register allocation must allow: two (two waves per SIMD) for codebook
    // V at 256, where the bound measured faster (4 x 32768, 16 q / 2 kv heads: 46.8 -> 45.5 us);
    // elsewhere the compiler's own allocation, which allows two waves at 256 and one for fp16 V at
    // 512 (accumulators, K and V buffers need more than half the register file there).  The
    // 8-wave workgroups of the split run one per CU, two waves per SIMD.
    static constexpr int MIN_WG = (D == 256 && VF == kVCB) ? 2 : 1;
};

template <int D, int VF>
struct MKTile {
    uint4 k[MfmaGeometry<D, VF>::KW];   // key kb + l%16, dims 32 s + 8 (l/16) + [0, 8) of the wave's steps s
};

template <int D, int VF>
struct MVTile {
    uint4 v[4][MfmaGeometry<D, VF>::NB];     // step i: key kb + 4 (l/16) + i, dims BW b + EV (l%16) + [0, EV)
    float side[4][MfmaGeometry<D, VF>::NB];  // int8: scale of the lane's 32-dim block; codebook: its norm
};

__device__ __forceinline__ half8_t as_h8(const uint4 &u) { return __builtin_bit_cast(half8_t, u); }

// Four fp32 values as fp16 pairs: hi = fp16(x), lo = fp16(x - hi); hi + lo carries about 22 bits.
__device__ __forceinline__ void split_f16(const float (&x)[4], half4_t &hi, half4_t &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const _Float16 h = (_Float16)x[i];
        hi[i] = h;
        lo[i] = (_Float16)(x[i] - (float)h);
    }
}

// Spins of a wave waiting for its partner's half of a QK product (about a tenth of a second); past
// it the wave goes on and the workgroup writes NaN, so a fault shows in the results instead of
// hanging the GPU.
constexpr int kPairMaxSpins = 1 << 21;

template <int D, int VF, int NS>
__global__ __launch_bounds__((MfmaGeometry<D, VF>::THREADS), (MfmaGeometry<D, VF>::MIN_WG)) void attn_partial_mfma_kernel(const LaunchArgsT<NS> args) {
    using Geo = MfmaGeometry<D, VF>;
    constexpr int KW = Geo::KW, EV = Geo::EV, BW = Geo::BW, NB = Geo::NB, NO = Geo::NO;
    constexpr int DS = Geo::DS, DH = Geo::DH, NT = Geo::THREADS;
    constexpr int CB_B = D < 256 ? D : 256;   // codebook norm block
    static_assert(NT >= 256, "one thread per codebook table entry");

    const int item = xcd_item(blockIdx.x, args.n_items, args.n_sub);
    int si = upper_index(args.n_slots, item, [&](int i) { return args.key[i]; });
    si -= args.slot[si].lead_off;         // the query group's leader: its longest query
    const SlotDesc sd = args.slot[si];
    const int n_mem = sd.group_n;         // queries of the group (1 when alone); table entries si..
    const int local = item - sd.item_begin;
    const int sub = local % args.n_sub;
    const int t = local / args.n_sub;
    const int c = t % sd.n_chunks;
    const int kvh = t / sd.n_chunks;
    const int cbeg = sd.lo + c * sd.chunk;
    const int cend = min(cbeg + sd.chunk, sd.L);
    const int GB = args.G / args.n_sub;                 // heads per query of this block
    const int h0 = kvh * args.G + sub * GB;             // first head of the block (in the slot)
    const int64_t rowbase = sd.kv_row0 + (int64_t)kvh * sd.kv_stride;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
    const int w = wv % kWaves;   // the wave's stream of key tiles: w, w + 4, ...
    const int dh = wv / kWaves;  // with the split, its output dims [dh DH, dh DH + DH) and QK steps [dh KW, dh KW + KW)
    const int c16 = lane & 15;   // MFMA row / column of the lane
    const int g = lane >> 4;     // lane group
    // Column c16 is head h0 + c16 % GB of the group's query c16 / GB: GB = 8 or 16 heads of one
    // query, or every head of the kv head (GB = G < 8) for each of up to 16 / GB queries of one
    // slot (drafts of a speculative-verify step, or one query alone).  Each query masks the
    // positions past its own end; columns past the group's queries compute and are not written.
    const int mem = c16 / GB;
    const bool head_ok = mem < n_mem;
    const int mi = si + (head_ok ? mem : 0);
    const int m_L = args.slot[mi].L;
    const int m_nchunks = args.slot[mi].n_chunks;
    const int64_t m_part = args.slot[mi].part_row0;
    const int hh = c16 - mem * GB;
    const int64_t qrow = (int64_t)args.slot[mi].slot_idx * args.n_q + h0 + hh;
    const int cend_col = min(cbeg + sd.chunk, m_L);

    // q as the B operand of the QK steps: step s covers dims 32 s + 8 g + [0, 8), like the K loads.
    // Each wave holds the KW steps it computes in registers (32 per lane up to 128 dims; at 512
    // each wave of a pair takes 256 dims), except for fp16 V at head_dim 256, whose accumulators
    // and V buffers need the registers: there q sits in LDS (rows padded by 16 bytes so the 16
    // heads of one read fall in different banks) and is read again for every tile.  In registers
    // it saves those reads (graph-replayed, 8 x 32768 slots, 16 q / 2 kv heads at 512: codebook V
    // 144.1 -> 140.3 us, one slot 62.3 -> 54.9; int8 and fp16 V and byte V at 256 0.2-2%).
    constexpr bool QLDS = D >= 256 && DS == 1 && VF == kVF16;
    constexpr int QS = D + 8;                      // LDS row stride of q, in halves
    __shared__ uint16_t s_q[QLDS ? 16 * QS : 1];
    half8_t qf[QLDS ? 1 : KW];
    if constexpr (QLDS) {
        // the workgroup's threads fill 16 rows of D halves, 16 bytes per thread per pass
        for (int x = tid * 8; x < 16 * D; x += NT * 8) {
            const int hr = x / D, dd = x % D;   // row hr: column hr's query and head
            uint4 a = make_uint4(0, 0, 0, 0);
            if (hr / GB < n_mem) {
                const int64_t qr = (int64_t)args.slot[si + hr / GB].slot_idx * args.n_q + h0 + hr % GB;
                a = *(const uint4 *)(args.q + qr * D + dd);
            }
            *(uint4 *)(s_q + hr * QS + dd) = a;
        }
    } else {
#pragma unroll
        for (int s = 0; s < KW; ++s) {
            uint4 a = make_uint4(0, 0, 0, 0);
            if (head_ok) a = *(const uint4 *)(args.q + qrow * D + 32 * (KW * dh + s) + 8 * g);
            qf[s] = as_h8(a);
        }
    }

    // codebook V: 2^6 level[i & mask] / sqrt(B) as two fp16 terms, hi in the low half, lo in the
    // high.  The 2^6 is taken back from the block norm that scales P (below).  With p <= 2^8 the
    // pair p norm / 2^6 stays finite in fp16 for norms below 16376, and normal for weights
    // p >= 2^-8 / norm; the table stays finite for levels below 8192.
    __shared__ uint32_t s_cb[VF == kVCB ? 256 : 1];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    __shared__ f32x4_t s_o[DS][NO][64];            // one wave's accumulators per dim range, for the final merge
    // the split: each wave's half of S^T per tile (two tiles in turn) and the count of halves it has posted
    __shared__ f32x4_t s_x[DS > 1 ? kWaves * DS * 2 : 1][64];
    __shared__ int s_posted[DS > 1 ? kWaves * DS : 1];
    __shared__ int s_pair_late;   // a wave gave up waiting for its partner
    if constexpr (DS > 1) {
        if (tid < kWaves * DS) s_posted[tid] = 0;
        if (tid == 0) s_pair_late = 0;
    }

    // Cache row of a key of the chunk (keys past its end read its last key; they are masked).
    auto row_of = [&](int key) -> int64_t {
        int rc = (key < cend ? key : cend - 1) - sd.ring_base;
        if (rc >= sd.ring_cap) rc -= sd.ring_cap;
        return rowbase + rc;
    };
    // K: each load reads 64 bytes of 16 rows, so the two halves of a 128-byte line come
    // from consecutive steps; plain (cached) loads let the second half hit in L1, where
    // non-temporal ones measured 3-12% slower.  V reads whole lines and streams.
    auto load_k = [&](int kb, MKTile<D, VF> &f) {
        const uint16_t *kp = args.k + row_of(kb + c16) * D + 8 * g + 32 * KW * dh;
#pragma unroll
        for (int s = 0; s < KW; ++s) f.k[s] = *(const uint4 *)(kp + 32 * s);
    };
    auto load_v = [&](int kb, MVTile<D, VF> &f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = row_of(kb + 4 * g + i);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int d0 = dh * DH + BW * b + EV * c16;
                if constexpr (VF == kVF16) {
                    f.v[i][b] = load_stream16((const uint16_t *)args.v + row * D + d0);
                } else {
                    const uint8_t *vp = (const uint8_t *)args.v + row * D + d0;
                    if constexpr (Geo::VBYTES == 16) {
                        f.v[i][b] = load_stream16(vp);
                    } else {
                        const uint2 x = *(const uint2 *)vp;
                        f.v[i][b] = make_uint4(x.x, x.y, 0, 0);
                    }
                    if constexpr (VF == kVI8)
                        f.side[i][b] = h2f(((const uint16_t *)args.vs)[row * (D / 32) + d0 / 32]);
                    else
                        f.side[i][b] = ((const float *)args.vs)[row * (D / CB_B) + d0 / CB_B];
                }
            }
        }
    };

    float m = -INFINITY, l = 0.f;   // running max (log2 domain) and this lane's part of the sum, head c16
    f32x4_t o[NO];
#pragma unroll
    for (int j = 0; j < NO; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float sl2 = args.scale_log2;

    // S^T of one tile of 16 keys (with the split: this wave's steps, then the sum with the
    // partner wave's steps through LDS; both waves form lower half + upper half, the same bits)
    int posted = 0;   // halves this wave has posted
    bool late = false;
    auto qk = [&](const MKTile<D, VF> &kt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KW; ++s) {
            half8_t qb;
            if constexpr (QLDS) qb = as_h8(*(const uint4 *)(s_q + c16 * QS + 32 * (KW * dh + s) + 8 * g));
            else qb = qf[s];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(kt.k[s]), qb, acc, 0, 0, 0);
        }
        if constexpr (DS > 1) {
            const int mine = (w * DS + dh) * 2 + (posted & 1), theirs = (w * DS + (dh ^ 1)) * 2 + (posted & 1);
            s_x[mine][lane] = acc;
            ++posted;
            __hip_atomic_store(&s_posted[w * DS + dh], posted, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            int spins = 0;
            while (__hip_atomic_load(&s_posted[w * DS + (dh ^ 1)], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
                       posted && spins < kPairMaxSpins) {
                __builtin_amdgcn_s_sleep(1);
                ++spins;
            }
            late |= spins >= kPairMaxSpins;
            const f32x4_t other = s_x[theirs][lane];
            acc = dh == 0 ? acc + other : other + acc;
        }
        return acc;
    };
    // The rest of the tile from kb: online softmax, O^T += V^T P^T.
    auto step = [&](int kb, const f32x4_t acc, const MVTile<D, VF> &vt) {
        float sc[4], p[4];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = (kb + 4 * g + i) < cend_col ? acc[i] * sl2 : -INFINITY;
            mt = fmaxf(mt, sc[i]);
        }
        mt = fmaxf(mt, shfl_xor_f32(mt, 16));
        mt = fmaxf(mt, shfl_xor_f32(mt, 32));
        // The reference m (log2 domain) moves only when a logit passes it by more than
        // kLazyMax, so the weights stay <= 2^kLazyMax and the accumulators are rescaled
        // rarely (O and S share the reference, so O / S is unchanged).
        if (__builtin_amdgcn_ballot_w64(mt > m + kLazyMax) != 0) {
            const float mx = fmaxf(m, mt);
            const float alpha = fast_exp2(m - ((mx == -INFINITY) ? 0.f : mx));
            l *= alpha;
#pragma unroll
            for (int j = 0; j < NO; ++j) o[j] *= alpha;
            m = mx;
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(sc[i] - ms);
            psum += p[i];
        }
        l += psum;

        if constexpr (VF == kVF16) {
            // fp16 V on v_mfma_f32_16x16x16_f16: one product covers the tile's 16 keys.  A is
            // V^T: lane l supplies A[l%16][4(l/16) + j], keys 4(l/16) + j, which are exactly its
            // loads j = 0..3, so element e of those four loads is its A operand for instruction e.
            // B is P^T straight from the S^T accumulator (keys 4(l/16) + j of head l%16), as two
            // fp16 terms, hi + lo, which carry about 22 bits of each weight; the products are
            // exact and the accumulation fp32.
            half4_t ph, pl;
            split_f16(p, ph, pl);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const half8_t v0 = as_h8(vt.v[0][b]), v1 = as_h8(vt.v[1][b]);
                const half8_t v2 = as_h8(vt.v[2][b]), v3 = as_h8(vt.v[3][b]);
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const half4_t a = {v0[e], v1[e], v2[e], v3[e]};
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, ph, o[b * EV + e], 0, 0, 0);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pl, o[b * EV + e], 0, 0, 0);
                }
            }
        } else if constexpr (VF == kVCB) {
            // Codebook V on the same products.  The table gives each level as hi + lo (about 22
            // bits).  The 16 dims of one instruction lie in one norm block (min(D, 256) dims, one
            // load), so the norm belongs to the key alone and scales P once per load, which is
            // then split the same way.  x p = xh ph + xh pl + xl ph, leaving out xl pl (about
            // 2^-22 of the product).
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float pn[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) pn[j] = p[j] * (vt.side[j][b] * (1.f / 64.f));
                half4_t ph, pl;
                split_f16(pn, ph, pl);
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    uint32_t t[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 &u = vt.v[j][b];
                        const uint32_t wd = (e / 4 == 0) ? u.x : (e / 4 == 1) ? u.y : (e / 4 == 2) ? u.z : u.w;
                        t[j] = s_cb[(wd >> (8 * (e % 4))) & 0xFF];
                    }
                    // low halves (hi terms) of keys 0..3, then high halves (lo terms)
                    const uint2 ah = make_uint2(__builtin_amdgcn_perm(t[1], t[0], 0x05040100u),
                                                __builtin_amdgcn_perm(t[3], t[2], 0x05040100u));
                    const uint2 al = make_uint2(__builtin_amdgcn_perm(t[1], t[0], 0x07060302u),
                                                __builtin_amdgcn_perm(t[3], t[2], 0x07060302u));
                    const half4_t xh = __builtin_bit_cast(half4_t, ah), xl = __builtin_bit_cast(half4_t, al);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, ph, o[b * EV + e], 0, 0, 0);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, pl, o[b * EV + e], 0, 0, 0);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xl, ph, o[b * EV + e], 0, 0, 0);
                }
            }
        } else {
            // int8 V on the same products, exactly: the block scale is an fp16 value and the code
            // a small integer, so hi = fp16(code scale) and lo = fma(code, scale, -hi) (the
            // residual, exact in fp16) sum to code scale exactly, for |code scale| up to 65504
            // (V within fp16's range).  Keys 0, 1 and 2, 3 of the lane
            // go through packed fp16 arithmetic side by side, already in the A operand's order.
            half4_t ph, pl;
            split_f16(p, ph, pl);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const half2_t s01 = {(_Float16)vt.side[0][b], (_Float16)vt.side[1][b]};
                const half2_t s23 = {(_Float16)vt.side[2][b], (_Float16)vt.side[3][b]};
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    _Float16 c[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 &u = vt.v[j][b];
                        const uint32_t wd = (e / 4 == 0) ? u.x : (e / 4 == 1) ? u.y : (e / 4 == 2) ? u.z : u.w;
                        c[j] = (_Float16)(int)(int8_t)(wd >> (8 * (e % 4)));
                    }
                    const half2_t c01 = {c[0], c[1]}, c23 = {c[2], c[3]};
                    const half2_t h01 = c01 * s01, h23 = c23 * s23;
                    const half2_t l01 = __builtin_elementwise_fma(c01, s01, -h01);
                    const half2_t l23 = __builtin_elementwise_fma(c23, s23, -h23);
                    const half4_t xh = {h01[0], h01[1], h23[0], h23[1]};
                    const half4_t xl = {l01[0], l01[1], l23[0], l23[1]};
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, ph, o[b * EV + e], 0, 0, 0);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, pl, o[b * EV + e], 0, 0, 0);
                    o[b * EV + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(xl, ph, o[b * EV + e], 0, 0, 0);
                }
            }
        }
    };

    const int ntiles = (cend - cbeg + kMfmaKeys - 1) / kMfmaKeys;
    MKTile<D, VF> kt;
    MVTile<D, VF> va, vb;
    int tl = w;
    if (tl < ntiles) {
        load_k(cbeg + tl * kMfmaKeys, kt);
        load_v(cbeg + tl * kMfmaKeys, va);
    }
    if constexpr (VF == kVCB) {
        if (tid < 256) {
            const float x = args.codebook[tid & args.cb_mask] * args.cb_scale * 64.f;
            const _Float16 h = (_Float16)x, lo = (_Float16)(x - (float)h);
            s_cb[tid] = (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
        }
    }
    if constexpr (VF == kVCB || QLDS || DS > 1) __syncthreads();
    // K: one buffer, refilled as soon as the QK steps have read it; V: two buffers.
    for (; tl < ntiles; tl += 2 * kWaves) {
        f32x4_t acc = qk(kt);
        const bool more1 = tl + kWaves < ntiles;
        if (more1) {
            load_k(cbeg + (tl + kWaves) * kMfmaKeys, kt);
            load_v(cbeg + (tl + kWaves) * kMfmaKeys, vb);
        }
        step(cbeg + tl * kMfmaKeys, acc, va);
        if (!more1) break;
        acc = qk(kt);
        if (tl + 2 * kWaves < ntiles) {
            load_k(cbeg + (tl + 2 * kWaves) * kMfmaKeys, kt);
            load_v(cbeg + (tl + 2 * kWaves) * kMfmaKeys, va);
        }
        step(cbeg + (tl + kWaves) * kMfmaKeys, acc, vb);
    }

    // merge the 4 tile streams: M = max of their maxima, each stream's O and S scaled by 2^(m_w - M)
    // (with the split both waves of a stream hold the same m and l)
    l += shfl_xor_f32(l, 16);
    l += shfl_xor_f32(l, 32);
    if (g == 0 && dh == 0) {
        s_m[w][c16] = m;
        s_l[w][c16] = l;
    }
    if constexpr (DS > 1) {
        if (late) s_pair_late = 1;
    }
    __syncthreads();
    float M = s_m[0][c16];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][c16]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) L += s_l[ww][c16] * fast_exp2(s_m[ww][c16] - Ms);
    const float f = fast_exp2(m - Ms);
#pragma unroll
    for (int j = 0; j < NO; ++j) o[j] *= f;
    // ((o3 + o2) + o1) + o0 through one LDS buffer per dim range, in a fixed order
#pragma unroll
    for (int ww = kWaves - 1; ww >= 1; --ww) {
        if (w == ww) {
#pragma unroll
            for (int j = 0; j < NO; ++j) {
                if (ww < kWaves - 1) o[j] += s_o[dh][j][lane];
                s_o[dh][j][lane] = o[j];
            }
        }
        __syncthreads();
    }
    // a group member whose last chunk is before c has nothing here
    if (w != 0 || !head_ok || c >= m_nchunks) return;   // no barriers follow
#pragma unroll
    for (int j = 0; j < NO; ++j) o[j] += s_o[dh][j][lane];

    float *op;
    float scale_out = 1.f;
    bool failed = false;
    if constexpr (DS > 1) failed = s_pair_late != 0;
    if (m_nchunks == 1) {
        op = args.out + qrow * D + dh * DH;
        scale_out = (L == 0.f) ? 0.f : 1.f / L;
    } else {
        const int64_t prow = m_part + (int64_t)(h0 + hh) * m_nchunks + c;
        op = args.ws_o + prow * D + dh * DH;
        if (g == 0 && dh == 0) {
            args.ws_ml[prow * 2 + 0] = failed ? NAN : M;
            args.ws_ml[prow * 2 + 1] = failed ? NAN : L;
        }
    }
    if (failed) scale_out = NAN;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *dst = op + BW * b + 4 * EV * g + EV * r;
#pragma unroll
            for (int e = 0; e < EV; e += 4)
                *(float4 *)(dst + e) = make_float4(o[b * EV + e][r] * scale_out, o[b * EV + e + 1][r] * scale_out,
                                                   o[b * EV + e + 2][r] * scale_out, o[b * EV + e + 3][r] * scale_out);
        }
    }
}

}  // namespace attn_decode_impl
