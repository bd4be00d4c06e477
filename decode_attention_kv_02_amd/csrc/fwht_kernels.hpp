// fwht_kernels.hpp -- gfx950 kernel that takes attention outputs back from the
// rotated basis of codebook V.
//
// Codebook V is stored rotated, v_rot = H (s * v) / sqrt(D), with H the
// Walsh-Hadamard matrix of order D (symmetric, H H = D I) and s a vector of
// +-1 sign flips (mlx-native flash_attn_vec_hybrid.metal, the codebook V
// layout; hf2q gemma4 batched_body.rs, the FWHT sign-undo after the
// attention).  Attention is linear in V, so its output is rotated the same
// way, and
//     y = s * (H x) / sqrt(D)
// recovers it.  H x is computed by the fast transform: log2(D) butterfly
// stages, stage h mapping (x[i], x[i + h]) to (x[i] + x[i + h], x[i] - x[i + h])
// for every i with bit h clear.
//
// One wave per row; lane l holds the E = D/64 consecutive elements
// [l*E, l*E + E).  The stages with h < E stay inside a lane; the stage with
// h = E * 2^k pairs lane l with lane l ^ 2^k (a cross-lane shuffle).  The
// same butterflies rotate new V rows when they are encoded (kv append).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_decode_impl {

__device__ __forceinline__ float fwht_shfl_xor(float x, int mask) {
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// H v (unnormalised) for the row spread over the wave, E elements per lane.
template <int E>
__device__ __forceinline__ void fwht_wave(float (&v)[E], int lane) {
    static_assert(E >= 1 && (E & (E - 1)) == 0, "D is a power of two, 64..512");
    // stages inside the lane
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
    // stages across lanes: the lane with the bit clear keeps the sum, the other the difference
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float other = fwht_shfl_xor(v[i], m);
            v[i] = upper ? other - v[i] : v[i] + other;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void fwht_undo_kernel(const float *x, const float *signs, float *y,
                                                        int64_t n_rows, float inv_sqrt_d) {
    constexpr int E = D / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;   // the whole wave leaves; no barriers follow
    const int lane = threadIdx.x & 63;
    const float *xr = x + row * D + lane * E;
    float v[E];
#pragma unroll
    for (int i = 0; i < E; i += (E >= 4 ? 4 : E)) {
        if constexpr (E >= 4) {
            const float4 t = *(const float4 *)(xr + i);
            v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
        } else if constexpr (E == 2) {
            const float2 t = *(const float2 *)xr;
            v[0] = t.x; v[1] = t.y;
        } else {
            v[0] = xr[0];
        }
    }
    fwht_wave<E>(v, lane);
    float *yr = y + row * D + lane * E;
#pragma unroll
    for (int i = 0; i < E; ++i) yr[i] = v[i] * signs[lane * E + i] * inv_sqrt_d;
}

}  // namespace attn_decode_impl
