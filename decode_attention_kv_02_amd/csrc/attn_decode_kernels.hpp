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
//    A row is read by R = head_dim/16 lanes with 16-byte loads (a wave loads
//    64/R consecutive rows per instruction, fully coalesced); the QK dot uses
//    v_dot2_f32_f16 on the fp16 pairs and an all-reduce over the R lanes made
//    of DPP row ops (quad_perm, row_half_mirror, row_mirror) plus one swizzle
//    at R = 32.  Each lane group keeps its own fp32 online softmax (running
//    max M and sum S in the log2 domain) and accumulates its 16 output dims;
//    at the end the lane groups are merged with cross-lane shuffles and the
//    4 waves through LDS.  A slot with one chunk writes out = O / S directly
//    (S == 0, an empty slot, writes zeros); otherwise O and (M, S) go to the
//    workspace.
//  * attn_combine_kernel: one workgroup per (slot, query head) whose slot has
//    several chunks: M* = max_c M_c, S* = sum_c S_c 2^(M_c - M*),
//    out = sum_c O_c 2^(M_c - M*) / S*.
//
// The logits are kept in the log2 domain (scale * log2 e folded into the
// scale), so every exponential is one v_exp_f32; exp(x - m) = 2^((x - m) log2 e).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_decode_impl {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct SlotDesc {
    int64_t kv_row0;    // row (position) index of (slot, kv head 0, pos 0) in the packed cache
    int64_t part_row0;  // first partial row of the slot, -1 when it has one chunk
    int32_t L;          // slot length: row stride between kv heads of the slot
    int32_t lo;         // first attended position
    int32_t chunk;      // positions per chunk
    int32_t n_chunks;   // chunks of the slot
    int32_t item_begin; // first partial workgroup of the slot in this launch
    int32_t comb_begin; // first combine workgroup of the slot in this launch
};

struct LaunchArgs {
    const uint16_t *q;      // fp16 [n_slots_total][n_q][D]
    const uint16_t *k;      // fp16 packed cache
    const void *v;          // fp16 or int8 packed cache
    const uint16_t *vs;     // fp16 scales or null
    float *out;             // fp32 [n_slots_total][n_q][D]
    float *ws_o;            // partial O rows [part_rows][D]
    float *ws_ml;           // partial (M, S) [part_rows][2]
    int32_t n_slots;        // slots in this launch
    int32_t slot0;          // global index of the launch's first slot
    int32_t n_q;
    int32_t G;              // query heads per kv head
    int32_t n_sub;          // G / GB
    float scale_log2;       // scale * log2(e)
    int32_t n_items;
    int32_t n_comb;
    SlotDesc slot[64];
};

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---------------------------------------------------------------- partial kernel

template <int D>
struct Geometry {
    static constexpr int R = D / 16;                        // lanes per KV row (16 dims each)
    static constexpr int P = 64 / R;                        // rows per wave load
    static constexpr int U = (D == 512) ? 4 : (16 / P);     // loads per wave iteration
    static constexpr int RW = P * U;                        // rows per wave iteration
    static constexpr int HALF = D / 2;
};

template <int D, int GB, bool VINT8>
__global__ __launch_bounds__(kThreads) void attn_partial_kernel(const LaunchArgs args) {
    using Geo = Geometry<D>;
    constexpr int R = Geo::R, P = Geo::P, U = Geo::U, RW = Geo::RW, HALF = Geo::HALF;

    const int item = blockIdx.x;
    const int si = upper_index(args.n_slots, item, [&](int i) { return args.slot[i].item_begin; });
    const SlotDesc sd = args.slot[si];
    const int local = item - sd.item_begin;
    const int sub = local % args.n_sub;
    const int t = local / args.n_sub;
    const int c = t % sd.n_chunks;
    const int kvh = t / sd.n_chunks;
    const int cbeg = sd.lo + c * sd.chunk;
    const int cend = min(cbeg + sd.chunk, sd.L);
    const int h0 = kvh * args.G + sub * GB;            // first query head of the block (in the slot)
    const int64_t slot_g = (int64_t)args.slot0 + si;  // global slot index
    const int64_t rowbase = sd.kv_row0 + (int64_t)kvh * sd.L;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int rg = lane / R;   // lane group = row within a wave load
    const int sl = lane % R;   // lane within the group

    // q fragment of each head: dims [sl*8, sl*8+8) and [HALF + sl*8, HALF + sl*8 + 8)
    half2_t qv[GB][8];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        const uint16_t *qp = args.q + (slot_g * args.n_q + h0 + g) * D;
        const uint4 a = *(const uint4 *)(qp + sl * 8);
        const uint4 b = *(const uint4 *)(qp + HALF + sl * 8);
        qv[g][0] = as_h2(a.x); qv[g][1] = as_h2(a.y); qv[g][2] = as_h2(a.z); qv[g][3] = as_h2(a.w);
        qv[g][4] = as_h2(b.x); qv[g][5] = as_h2(b.y); qv[g][6] = as_h2(b.z); qv[g][7] = as_h2(b.w);
    }

    float m[GB], l[GB], o[GB][16];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) o[g][i] = 0.f;
    }

    const float sl2 = args.scale_log2;
    const uint16_t *kbase = args.k + rowbase * D;

    for (int wb = cbeg + w * RW; wb < cend; wb += kWaves * RW) {
        // ---- issue every load of the iteration
        uint4 ka[U], kb[U];
        uint4 va[U], vb[U];      // fp16 V: two 16-byte halves; int8 V: codes in va
        uint16_t vsc[U];
        int rowv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = wb + u * P + rg;
            rowv[u] = row;
            const int rc = row < cend ? row : cend - 1;
            const uint16_t *kp = kbase + (int64_t)rc * D;
            ka[u] = *(const uint4 *)(kp + sl * 8);
            kb[u] = *(const uint4 *)(kp + HALF + sl * 8);
            if constexpr (VINT8) {
                const int8_t *vp = (const int8_t *)args.v + (rowbase + rc) * D;
                va[u] = *(const uint4 *)(vp + sl * 16);
                vsc[u] = args.vs[(rowbase + rc) * (D / 32) + (sl >> 1)];
            } else {
                const uint16_t *vp = (const uint16_t *)args.v + (rowbase + rc) * D;
                va[u] = *(const uint4 *)(vp + sl * 8);
                vb[u] = *(const uint4 *)(vp + HALF + sl * 8);
            }
        }

        // ---- logits (log2 domain)
        float s[U][GB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                float acc = 0.f;
                acc = __builtin_amdgcn_fdot2(as_h2(ka[u].x), qv[g][0], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ka[u].y), qv[g][1], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ka[u].z), qv[g][2], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(ka[u].w), qv[g][3], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(kb[u].x), qv[g][4], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(kb[u].y), qv[g][5], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(kb[u].z), qv[g][6], acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(kb[u].w), qv[g][7], acc, false);
                acc = group_sum<R>(acc);
                s[u][g] = rowv[u] < cend ? acc * sl2 : -INFINITY;
            }
        }

        // ---- V rows as fp32 (shared by the GB heads)
        float vf[U][16];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (VINT8) {
                const uint32_t wd[4] = {va[u].x, va[u].y, va[u].z, va[u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vf[u][4 * j + 0] = (float)(int8_t)(wd[j]);
                    vf[u][4 * j + 1] = (float)(int8_t)(wd[j] >> 8);
                    vf[u][4 * j + 2] = (float)(int8_t)(wd[j] >> 16);
                    vf[u][4 * j + 3] = (float)(int8_t)(wd[j] >> 24);
                }
            } else {
                const uint32_t wd[8] = {va[u].x, va[u].y, va[u].z, va[u].w, vb[u].x, vb[u].y, vb[u].z, vb[u].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    vf[u][2 * j + 0] = h2f((uint16_t)(wd[j] & 0xFFFF));
                    vf[u][2 * j + 1] = h2f((uint16_t)(wd[j] >> 16));
                }
            }
        }

        // ---- online softmax + V accumulation, per head
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
            const float ms = (mx == -INFINITY) ? 0.f : mx;
            const float alpha = fast_exp2(m[g] - ms);
            float p[U];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = fast_exp2(s[u][g] - ms);
                psum += p[u];
            }
            l[g] = l[g] * alpha + psum;
            m[g] = mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) o[g][i] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float wgt = p[u];
                if constexpr (VINT8) wgt *= h2f(vsc[u]);
#pragma unroll
                for (int i = 0; i < 16; ++i) o[g][i] = fmaf(wgt, vf[u][i], o[g][i]);
            }
        }
    }

    // ---- merge the P lane groups of the wave (lanes lane ^ off share the dims)
#pragma unroll
    for (int off = R; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
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
    __shared__ float s_o[kWaves][GB][D];
    __shared__ float s_ml[kWaves][GB][2];
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            if constexpr (VINT8) {
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

    const bool single = sd.n_chunks == 1;
    for (int idx = tid; idx < GB * D; idx += kThreads) {
        const int g = idx / D;
        const int d = idx - g * D;
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
        if (single) {
            args.out[(slot_g * args.n_q + h0 + g) * D + d] = (lsum == 0.f) ? 0.f : acc / lsum;
        } else {
            const int64_t prow = sd.part_row0 + (int64_t)(h0 + g) * sd.n_chunks + c;
            args.ws_o[prow * D + d] = acc;
            if (d == 0) {
                args.ws_ml[prow * 2 + 0] = mx;
                args.ws_ml[prow * 2 + 1] = lsum;
            }
        }
    }
}

// ---------------------------------------------------------------- combine kernel

constexpr int kCombineMaxChunks = 4096;

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

template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const LaunchArgs args) {
    __shared__ float s_w[kCombineMaxChunks];
    __shared__ float s_red[kWaves];

    const int row = blockIdx.x;
    const int si = upper_index(args.n_slots, row, [&](int i) { return args.slot[i].comb_begin; });
    const SlotDesc sd = args.slot[si];
    const int h = row - sd.comb_begin;
    const int nc = sd.n_chunks;
    const int64_t base = sd.part_row0 + (int64_t)h * nc;
    const int64_t slot_g = (int64_t)args.slot0 + si;
    const int tid = threadIdx.x;
    const int w = tid >> 6;

    // M* over chunks
    float mx = -INFINITY;
    for (int c = tid; c < nc; c += kThreads) mx = fmaxf(mx, args.ws_ml[(base + c) * 2]);
    mx = wave_max(mx);
    if ((tid & 63) == 0) s_red[w] = mx;
    __syncthreads();
    mx = s_red[0];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mx = fmaxf(mx, s_red[ww]);
    const float ms = (mx == -INFINITY) ? 0.f : mx;
    __syncthreads();

    // chunk weights 2^(M_c - M*) and S*
    float ls = 0.f;
    for (int c = tid; c < nc; c += kThreads) {
        const float wc = fast_exp2(args.ws_ml[(base + c) * 2] - ms);
        s_w[c] = wc;
        ls += wc * args.ws_ml[(base + c) * 2 + 1];
    }
    ls = wave_sum(ls);
    if ((tid & 63) == 0) s_red[w] = ls;
    __syncthreads();
    float lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) lsum += s_red[ww];

    float *dst = args.out + (slot_g * args.n_q + h) * D;
    for (int d = tid; d < D; d += kThreads) {
        float acc = 0.f;
        const float *src = args.ws_o + base * D + d;
        for (int c = 0; c < nc; ++c) acc = fmaf(s_w[c], src[(int64_t)c * D], acc);
        dst[d] = (lsum == 0.f) ? 0.f : acc / lsum;
    }
}

}  // namespace attn_decode_impl
