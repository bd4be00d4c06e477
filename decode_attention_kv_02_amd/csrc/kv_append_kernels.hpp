// kv_append_kernels.hpp -- gfx950 kernel that writes new tokens into the KV cache.
//
// The step before decode attention (hf2q gemma4 batched_body.rs, the
// attention phase's KV encode: an F16 copy of K and the quantisation of V,
// per slot and position; mlx-native flash_attn_vec_hybrid.metal, batched
// kernels: the physical row of a position).  Each new token's K is stored as
// fp16 and its V as fp16 or as symmetric int8 codes in blocks of 32 dims with
// one fp16 scale per block:
//     scale = fp16(max|v| / 127),  code = clamp(rint(v / scale), -127, 127)
// (codes 0 when the scale is 0).  Every rounding decision is made in IEEE
// single precision: the divisions are the correctly rounded fp32 divide,
// rint rounds half to even, and the fp16 conversions round to nearest even.
//
// Codebook V (the hybrid regime's FWHT-V encode; the TQ-HB layout of
// mlx-native flash_attn_vec_hybrid.metal with its D = 512 per-block norms):
// the row is rotated, y = H (s * v) / sqrt(D), one fp32 norm is kept per
// block of B = min(D, 256) coordinates, and each coordinate is stored as the
// index of the level nearest to u = y * sqrt(B) / norm (the first index on a
// tie, 0 when the norm is 0).  The levels must increase; the nearest one is
// found by binary search over the midpoints of neighbouring levels, which
// every workgroup first stages in LDS.  All of it in fp32.
//
// One wave per (new row, kv head); each lane owns D/64 consecutive dims, so a
// block of 32 dims spans 2048/D lanes and its max |v| is an all-reduce over
// those lanes; a codebook block spans B/(D/64) lanes and its norm is an
// all-reduce over those.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode_kernels.hpp"
#include "fwht_kernels.hpp"

namespace attn_decode_impl {

// New rows reach the kernel as runs: rows of one slot whose cache rows follow one another
// (consecutive positions, no ring wrap).  A decode step is one run per slot; appending a
// prompt's rows to one slot is one run, two across a ring wrap.
constexpr int kAppendMaxRuns = 240;   // runs per launch (run table passed by value, < 4 KiB)

struct AppendRun {
    int64_t cache_row0;   // (slot * n_kv) * capacity + physical row of the run's first row
    int32_t row_begin;    // the run's first row, counted from the launch's first row
    int32_t pad;
};

struct AppendArgs {
    const float *k_new;        // [n_rows][n_kv][D]
    const float *v_new;        // [n_rows][n_kv][D]
    uint16_t *k_cache;         // fp16 [n_cache_slots][n_kv][capacity][D]
    void *v_cache;             // fp16 or int8, same layout
    uint16_t *v_scales;        // int8 V: fp16 [..][D/32]
    float *v_norms;            // codebook V: fp32 [..][D/B]
    const float *signs;        // codebook V: the rotation's sign flips [D]
    const float *codebook;     // codebook V: increasing levels [2^cb_bits]
    int32_t cb_bits;
    float inv_sqrt_d;          // codebook V: 1 / sqrt(D)
    int32_t n_rows;            // rows in this launch
    int32_t n_kv;
    int32_t capacity;
    int32_t row0;              // index of the launch's first row in k_new / v_new
    int32_t n_runs;            // runs in this launch (run i covers rows [row_begin_i, row_begin_i+1))
    int32_t pad0;
    AppendRun run[kAppendMaxRuns];
};

__device__ __forceinline__ float lane_max_xor(float x, int mask) {
    const int lane = __lane_id();
    return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2,
                                                                           __builtin_bit_cast(int, x))));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);   // v_cvt_f16_f32: round to nearest even
}

// E consecutive floats / halves / bytes moved with the widest aligned access.
template <int E>
__device__ __forceinline__ void load_f32(const float *p, float (&x)[E]) {
    if constexpr (E % 4 == 0) {
#pragma unroll
        for (int j = 0; j < E; j += 4) {
            const float4 t = *(const float4 *)(p + j);
            x[j] = t.x; x[j + 1] = t.y; x[j + 2] = t.z; x[j + 3] = t.w;
        }
    } else if constexpr (E == 2) {
        const float2 t = *(const float2 *)p;
        x[0] = t.x; x[1] = t.y;
    } else {
        x[0] = p[0];
    }
}

template <int E>
__device__ __forceinline__ void store_f16(uint16_t *p, const float (&x)[E]) {
    uint16_t h[E];
#pragma unroll
    for (int i = 0; i < E; ++i) h[i] = f32_to_f16_bits(x[i]);
    if constexpr (E == 8) {
        *(uint4 *)p = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16,
                                 h[4] | (uint32_t)h[5] << 16, h[6] | (uint32_t)h[7] << 16);
    } else if constexpr (E == 4) {
        *(uint2 *)p = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
    } else if constexpr (E == 2) {
        *(uint32_t *)p = h[0] | (uint32_t)h[1] << 16;
    } else {
        p[0] = h[0];
    }
}

template <int E>
__device__ __forceinline__ void store_i8(int8_t *p, const int8_t (&c)[E]) {
    uint32_t w[(E + 3) / 4] = {};
#pragma unroll
    for (int i = 0; i < E; ++i) w[i / 4] |= (uint32_t)(uint8_t)c[i] << (8 * (i % 4));
    if constexpr (E == 8) {
        *(uint2 *)p = make_uint2(w[0], w[1]);
    } else if constexpr (E == 4) {
        *(uint32_t *)p = w[0];
    } else if constexpr (E == 2) {
        *(uint16_t *)p = (uint16_t)w[0];
    } else {
        p[0] = c[0];
    }
}

template <int E>
__device__ __forceinline__ void store_u8(uint8_t *p, const uint8_t (&c)[E]) {
    uint32_t w[(E + 3) / 4] = {};
#pragma unroll
    for (int i = 0; i < E; ++i) w[i / 4] |= (uint32_t)c[i] << (8 * (i % 4));
    if constexpr (E == 8) {
        *(uint2 *)p = make_uint2(w[0], w[1]);
    } else if constexpr (E == 4) {
        *(uint32_t *)p = w[0];
    } else if constexpr (E == 2) {
        *(uint16_t *)p = (uint16_t)w[0];
    } else {
        p[0] = c[0];
    }
}

template <int D, int VF>
__global__ __launch_bounds__(256) void kv_append_kernel(const AppendArgs args) {
    constexpr int E = D / 64;          // dims per lane
    constexpr int LPB = 32 / E;        // lanes per 32-dim block (int8 V)
    constexpr int CB_B = D < 256 ? D : 256;
    constexpr int LPN = CB_B / E;      // lanes per norm block (codebook V): 64, or 32 at D = 512
    __shared__ float s_mid[VF == kVCB ? 255 : 1];
    if constexpr (VF == kVCB) {
        const int n_mid = (1 << args.cb_bits) - 1;
        for (int j = threadIdx.x; j < n_mid; j += 256) s_mid[j] = 0.5f * (args.codebook[j] + args.codebook[j + 1]);
        __syncthreads();
    }
    const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, kv head) of this wave
    if (unit >= args.n_rows * args.n_kv) return;             // whole wave leaves; no barriers follow
    const int lane = threadIdx.x & 63;
    const int r = unit / args.n_kv;
    const int h = unit - r * args.n_kv;
    int lo = 0, hi = args.n_runs - 1;   // the run holding row r: largest row_begin <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (args.run[mid].row_begin <= r) lo = mid; else hi = mid - 1;
    }
    const int64_t src = ((int64_t)(args.row0 + r) * args.n_kv + h) * D + lane * E;
    const int64_t dst_row = args.run[lo].cache_row0 + (r - args.run[lo].row_begin) + (int64_t)h * args.capacity;

    float kx[E], vx[E];
    load_f32<E>(args.k_new + src, kx);
    load_f32<E>(args.v_new + src, vx);
    store_f16<E>(args.k_cache + dst_row * D + lane * E, kx);

    if constexpr (VF == kVF16) {
        store_f16<E>((uint16_t *)args.v_cache + dst_row * D + lane * E, vx);
    } else if constexpr (VF == kVI8) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(vx[i]));
#pragma unroll
        for (int m = 1; m < LPB; m <<= 1) amax = lane_max_xor(amax, m);
        const uint16_t s16 = f32_to_f16_bits(amax / 127.0f);
        const float s = (float)__builtin_bit_cast(_Float16, s16);
        int8_t codes[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            float c = 0.f;
            if (s != 0.f) c = fminf(fmaxf(rintf(vx[i] / s), -127.f), 127.f);
            codes[i] = (int8_t)c;
        }
        store_i8<E>((int8_t *)args.v_cache + dst_row * D + lane * E, codes);
        if (lane % LPB == 0) args.v_scales[dst_row * (D / 32) + (lane * E) / 32] = s16;
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i) vx[i] *= args.signs[lane * E + i];
        fwht_wave<E>(vx, lane);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            vx[i] *= args.inv_sqrt_d;
            ss += vx[i] * vx[i];
        }
        // xor butterflies: both lanes of a pair add the same two numbers, so the
        // whole block ends with one bitwise-identical sum
#pragma unroll
        for (int m = 1; m < LPN; m <<= 1) ss += fwht_shfl_xor(ss, m);
        const float norm = sqrtf(ss);
        const float to_u = norm > 0.f ? sqrtf((float)CB_B) / norm : 0.f;
        uint8_t codes[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float u = vx[i] * to_u;
            int lo = 0;
            if (norm > 0.f)
                for (int step = 1 << (args.cb_bits - 1); step > 0; step >>= 1)
                    if (u > s_mid[lo + step - 1]) lo += step;
            codes[i] = (uint8_t)lo;
        }
        store_u8<E>((uint8_t *)args.v_cache + dst_row * D + lane * E, codes);
        if (lane % LPN == 0) args.v_norms[dst_row * (D / CB_B) + lane / LPN] = norm;
    }
}

}  // namespace attn_decode_impl
