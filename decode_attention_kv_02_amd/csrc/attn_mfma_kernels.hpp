// attn_mfma_kernels.hpp -- gfx950 partial kernel for GQA groups of 8 or 16
// query heads per workgroup, on the matrix cores.
//
// Same operation and partial format as attn_partial_kernel (one chunk of one
// (slot, kv head): out = O / S, or O and (M, S) for the log-sum-exp merge;
// mlx-native flash_attn_vec_hybrid.metal, flash_attn_vec_hybrid_batched_gqa_impl:
// every K and V row is read once for all the query heads of the group).  With
// 8 or more heads per kv head the per-lane dot products and V FMAs of the
// lane kernel make it VALU-bound (rocprof: 205 VALU instructions per KV row at
// 8 heads, 74% busy, 37% of HBM peak), so here both products are MFMA tiles:
//
//  * The 4 waves split head_dim: wave w owns dims [w D/4, (w+1) D/4).  For a
//    tile of 16 keys each wave computes its part of S^T (16 keys x 16 heads)
//    with v_mfma_f32_16x16x16_f16 (A = K rows, B = q; fp16 products are exact,
//    fp32 accumulation), the 4 parts are added in LDS in a fixed order, and
//    every wave then holds the same S^T and runs the same online softmax
//    (running max M and sum S per head, log2 domain).
//  * O^T (dims x heads) += V^T P^T with v_mfma_f32_16x16x4_f32: the A operand
//    is V (dequantised to fp32 in an LDS tile, exact for every V format), the
//    B operand is P straight from the S^T accumulator registers (lane l holds
//    keys 4(l/16)+i of head l%16, exactly the B layout of step i), so P never
//    leaves the registers and stays fp32.  Each lane's O values belong to one
//    head, so rescaling by exp(M_old - M_new) needs no cross-lane traffic.
//  * Each wave writes the dims it owns; M and S are the same in every wave.
//
// Lane layouts (checked on gfx950): 16x16x16 f16: A[l%16][4(l/16)+e],
// B[4(l/16)+e][l%16]; 16x16x4 f32: A[l%16][l/16], B[l/16][l%16]; both
// C[4(l/16)+i][l%16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode_kernels.hpp"

namespace attn_decode_impl {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaKeys = 16;   // keys per tile (the MFMA M / N size)

template <int D>
struct MfmaGeometry {
    static constexpr int DW = D / kWaves;   // dims per wave
    static constexpr int NT = DW / 16;      // 16-dim tiles per wave: QK k-steps and PV output tiles
    static constexpr int KL = DW / 32;      // 16-byte K (and fp16 V) loads per lane per key tile
    static constexpr int VB = DW / 4;       // bytes of int8 / codebook V per lane per key tile
    static constexpr int VS = DW + 4;       // LDS row stride (floats) of the V tile: keys 4 apart land 16 banks apart
    static_assert(D >= 128 && D <= 512, "head_dim 128..512");
};

// Registers of one key tile for one lane: key row l%16, the lane group's dims.
template <int D>
struct MFrag {
    uint4 k[MfmaGeometry<D>::KL];
    uint4 v[MfmaGeometry<D>::KL];   // fp16 V: like k; byte formats use the first VB bytes
    float side[2];                  // int8: fp16 scale of each 16-dim piece; codebook: the norm
};

__device__ __forceinline__ half4_t as_h4(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(half4_t, make_uint2(lo, hi));
}

template <int D, int VF>
__global__ __launch_bounds__(kThreads) void attn_partial_mfma_kernel(const LaunchArgs args) {
    using Geo = MfmaGeometry<D>;
    constexpr int DW = Geo::DW, NT = Geo::NT, KL = Geo::KL, VB = Geo::VB, VS = Geo::VS;
    constexpr int CB_B = D < 256 ? D : 256;   // codebook norm block
    static_assert(kThreads == 256, "one thread per codebook table entry");

    const int item = xcd_item(blockIdx.x, args.n_items, args.n_sub);
    const int si = upper_index(args.n_slots, item, [&](int i) { return args.slot[i].item_begin; });
    const SlotDesc sd = args.slot[si];   // no query groups on this path
    const int local = item - sd.item_begin;
    const int sub = local % args.n_sub;
    const int t = local / args.n_sub;
    const int c = t % sd.n_chunks;
    const int kvh = t / sd.n_chunks;
    const int cbeg = sd.lo + c * sd.chunk;
    const int cend = min(cbeg + sd.chunk, sd.L);
    const int GB = args.G / args.n_sub;                 // heads of this block: 8 or 16
    const int h0 = kvh * args.G + sub * GB;             // first head of the block (in the slot)
    const int64_t rowbase = sd.kv_row0 + (int64_t)kvh * sd.kv_stride;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c16 = lane & 15;   // MFMA row / column of the lane
    const int g = lane >> 4;     // lane group
    const int dw0 = w * DW;      // first dim of this wave
    const bool head_ok = c16 < GB;
    const int64_t qrow = (int64_t)sd.slot_idx * args.n_q + h0 + c16;

    // q as the B operand of the QK tiles: step 2j covers dims dw0 + 32j + 8g + [0, 4),
    // step 2j+1 dims dw0 + 32j + 8g + [4, 8) (the K loads use the same mapping)
    half4_t qf[NT];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (head_ok) a = *(const uint4 *)(args.q + qrow * D + dw0 + 32 * j + 8 * g);
        qf[2 * j] = as_h4(a.x, a.y);
        qf[2 * j + 1] = as_h4(a.z, a.w);
    }

    __shared__ float s_cb[VF == kVCB ? 256 : 1];    // codebook V: level[i & mask] / sqrt(B)
    __shared__ float s_v[kWaves][kMfmaKeys][VS];    // each wave's V tile, fp32
    __shared__ f32x4_t s_s[2][kWaves][64];          // the waves' parts of S^T, by tile parity

    // Loads of the tile starting at key kb: lane l reads key kb + l%16 (clamped
    // to the chunk's last key past its end; those keys are masked).
    auto load = [&](int kb, MFrag<D> &f) {
        const int key = kb + c16;
        int rc = (key < cend ? key : cend - 1) - sd.ring_base;
        if (rc >= sd.ring_cap) rc -= sd.ring_cap;
        const int64_t row = rowbase + rc;
        const uint16_t *kp = args.k + row * D + dw0 + 8 * g;
#pragma unroll
        for (int j = 0; j < KL; ++j) f.k[j] = load_stream16(kp + 32 * j);
        if constexpr (VF == kVF16) {
            const uint16_t *vp = (const uint16_t *)args.v + row * D + dw0 + 8 * g;
#pragma unroll
            for (int j = 0; j < KL; ++j) f.v[j] = load_stream16(vp + 32 * j);
        } else {
            // VB = 32: dims 16g + [0,16) and 64 + 16g + [0,16); 16: 16g + [0,16); 8: 8g + [0,8)
            const uint8_t *vp = (const uint8_t *)args.v + row * D + dw0;
            if constexpr (VB == 32) {
                f.v[0] = load_stream16(vp + 16 * g);
                f.v[1] = load_stream16(vp + 64 + 16 * g);
            } else if constexpr (VB == 16) {
                f.v[0] = load_stream16(vp + 16 * g);
            } else {
                const uint2 x = *(const uint2 *)(vp + 8 * g);
                f.v[0] = make_uint4(x.x, x.y, 0, 0);
            }
            if constexpr (VF == kVI8) {
                const uint16_t *sp = (const uint16_t *)args.vs + row * (D / 32);
                if constexpr (VB == 32) {
                    f.side[0] = h2f(sp[(dw0 + 16 * g) / 32]);
                    f.side[1] = h2f(sp[(dw0 + 64 + 16 * g) / 32]);
                } else {
                    f.side[0] = h2f(sp[(dw0 + (VB == 16 ? 16 : 8) * g) / 32]);
                }
            } else {
                f.side[0] = ((const float *)args.vs)[row * (D / CB_B) + dw0 / CB_B];
            }
        }
    };

    // This lane's key row of the wave's V tile, dequantised to fp32, into LDS.
    auto stage_v = [&](const MFrag<D> &f) {
        float *rowp = &s_v[w][c16][0];
        if constexpr (VF == kVF16) {
#pragma unroll
            for (int j = 0; j < KL; ++j) {
                const uint32_t wd[4] = {f.v[j].x, f.v[j].y, f.v[j].z, f.v[j].w};
                float x[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[2 * q] = h2f((uint16_t)(wd[q] & 0xFFFF));
                    x[2 * q + 1] = h2f((uint16_t)(wd[q] >> 16));
                }
                *(float4 *)(rowp + 32 * j + 8 * g) = make_float4(x[0], x[1], x[2], x[3]);
                *(float4 *)(rowp + 32 * j + 8 * g + 4) = make_float4(x[4], x[5], x[6], x[7]);
            }
        } else {
            constexpr int PIECES = VB == 32 ? 2 : 1;        // 16-byte pieces (VB = 8: one half piece)
            constexpr int WORDS = VB == 8 ? 2 : 4;          // 32-bit words of codes per piece
#pragma unroll
            for (int pc = 0; pc < PIECES; ++pc) {
                const uint32_t wd[4] = {f.v[pc].x, f.v[pc].y, f.v[pc].z, f.v[pc].w};
                const int d0 = VB == 32 ? 64 * pc + 16 * g : (VB == 16 ? 16 * g : 8 * g);
                const float sc = VF == kVI8 ? f.side[pc] : f.side[0];
#pragma unroll
                for (int q = 0; q < WORDS; ++q) {
                    float x[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t code = (wd[q] >> (8 * b)) & 0xFF;
                        if constexpr (VF == kVI8) x[b] = (float)(int8_t)code * sc;
                        else x[b] = s_cb[code] * sc;
                    }
                    *(float4 *)(rowp + d0 + 4 * q) = make_float4(x[0], x[1], x[2], x[3]);
                }
            }
        }
    };

    float m = -INFINITY, l = 0.f;   // running max (log2 domain) and this lane's part of the sum, head c16
    f32x4_t o[NT];                  // O^T: o[tt][i] = dim dw0 + 16 tt + 4g + i of head c16
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) o[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float sl2 = args.scale_log2;

    // One tile: QK part -> LDS, V tile -> LDS, barrier, whole S^T, softmax, PV.
    auto step = [&](int tile, int kb, const MFrag<D> &f) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            acc = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(f.k[j].x, f.k[j].y), qf[2 * j], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x16f16(as_h4(f.k[j].z, f.k[j].w), qf[2 * j + 1], acc, 0, 0, 0);
        }
        s_s[tile & 1][w][lane] = acc;
        stage_v(f);
        __syncthreads();
        f32x4_t sv = s_s[tile & 1][0][lane];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) sv += s_s[tile & 1][ww][lane];

        // online softmax over the tile's keys kb + 4g + i of head c16
        float s[4], p[4];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = (kb + 4 * g + i) < cend ? sv[i] * sl2 : -INFINITY;
            mt = fmaxf(mt, s[i]);
        }
        mt = fmaxf(mt, shfl_xor_f32(mt, 16));
        mt = fmaxf(mt, shfl_xor_f32(mt, 32));
        const float mx = fmaxf(m, mt);
        const float ms = (mx == -INFINITY) ? 0.f : mx;
        const float alpha = fast_exp2(m - ms);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(s[i] - ms);
            psum += p[i];
        }
        l = l * alpha + psum;
        m = mx;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) o[tt] *= alpha;

        // O^T += V^T P^T, 4 keys per MFMA: step i takes keys 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const float a = s_v[w][4 * g + i][16 * tt + c16];
                o[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[i], o[tt], 0, 0, 0);
            }
        }
    };

    const int ntiles = (cend - cbeg + kMfmaKeys - 1) / kMfmaKeys;   // the same in every wave
    MFrag<D> fa, fb;
    if (ntiles > 0) load(cbeg, fa);
    if constexpr (VF == kVCB) {
        s_cb[tid] = args.codebook[tid & args.cb_mask] * args.cb_scale;
        __syncthreads();
    }
    for (int tl = 0; tl < ntiles; tl += 2) {
        if (tl + 1 < ntiles) load(cbeg + (tl + 1) * kMfmaKeys, fb);
        step(tl, cbeg + tl * kMfmaKeys, fa);
        if (tl + 1 >= ntiles) break;
        if (tl + 2 < ntiles) load(cbeg + (tl + 2) * kMfmaKeys, fa);
        step(tl + 1, cbeg + (tl + 1) * kMfmaKeys, fb);
    }

    // the sum over the tile keys of the 4 lane groups of head c16
    l += shfl_xor_f32(l, 16);
    l += shfl_xor_f32(l, 32);
    if (!head_ok) return;   // no barriers follow
    if (sd.n_chunks == 1) {
        float *op = args.out + qrow * D + dw0 + 4 * g;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            float4 r;
            r.x = (l == 0.f) ? 0.f : o[tt][0] / l;
            r.y = (l == 0.f) ? 0.f : o[tt][1] / l;
            r.z = (l == 0.f) ? 0.f : o[tt][2] / l;
            r.w = (l == 0.f) ? 0.f : o[tt][3] / l;
            *(float4 *)(op + 16 * tt) = r;
        }
    } else {
        const int64_t prow = sd.part_row0 + (int64_t)(h0 + c16) * sd.n_chunks + c;
        float *op = args.ws_o + prow * D + dw0 + 4 * g;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            *(float4 *)(op + 16 * tt) = make_float4(o[tt][0], o[tt][1], o[tt][2], o[tt][3]);
        if (w == 0 && g == 0) {
            args.ws_ml[prow * 2 + 0] = m;
            args.ws_ml[prow * 2 + 1] = l;
        }
    }
}

}  // namespace attn_decode_impl
