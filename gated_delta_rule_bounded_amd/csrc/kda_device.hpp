// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef float floatx4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the top half of the
// fp32 bits).  Narrowing rounds to nearest, ties to even; NaN stays a quiet
// NaN; values that round past the largest finite bf16 become inf.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Eight bf16 values packed in a uint4 (16 bytes, one vector load).
__device__ __forceinline__ void unpack8(const uint4 &p, float (&f)[8]) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = f32_to_bf16(f[2 * i]) | (f32_to_bf16(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoid_fast(float x) {
    return 1.0f / (1.0f + exp2_fast(-x * kLog2e));
}

// 16x16x4 fp32 MFMA: D[m][n] = sum_k A[m][k] B[k][n] + C[m][n].
// Lane l supplies A[l%16][l/16] and B[l/16][l%16]; on return lane l holds
// D[4*(l/16) + i][l%16] in element i.
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float get4(const float4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace kda
