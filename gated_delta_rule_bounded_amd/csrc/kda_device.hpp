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

// 16-byte accesses through addresses read from device pointer tables (states,
// snapshots, conv windows).  The compiler cannot infer that such an address
// is global memory and would use flat instructions, which the wave's LDS
// wait counter also tracks, so an LDS wait would also wait for them; these
// go through global-address-space pointers (the tables hold device-memory
// addresses by contract).
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) uintx4 guintx4;
__device__ __forceinline__ uint4 gload16(const void *p) {
    return __builtin_bit_cast(uint4, *(const guintx4 *)(p));
}
__device__ __forceinline__ void gstore16(void *p, const uint4 &v) {
    *(guintx4 *)(p) = __builtin_bit_cast(uintx4, v);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoid_fast(float x) {
    return 1.0f / (1.0f + exp2_fast(-x * kLog2e));
}

// softplus(z) = log(1 + e^z), with e^z and log on the transcendental unit:
// log1p(y) is taken as log(u) * y / (u - 1), u = 1 + y (exact for the
// rounding of u, so small y keeps its relative accuracy; u == 1 means
// log1p(y) = y to within rounding); z > 20 returns z as the pages' threshold.
__device__ __forceinline__ float softplus_fast(float z) {
    const float y = exp2_fast(z * kLog2e);
    const float u = 1.0f + y;
    const float l1p = u == 1.0f ? y : __builtin_amdgcn_logf(u) * 0.69314718055994531f * (y / (u - 1.0f));
    return z > 20.0f ? z : l1p;
}

// The bounded log-decay of one channel ("Glm5NextKdaWeights" page, a_log per
// head and dt_bias per channel): g = -exp(a_log) * softplus(x + dt_bias),
// with rate = exp(a_log) from decay_rate.  kda_gate and the projection
// epilogue of the block decode both form it here.
__device__ __forceinline__ float decay_rate(float a_log) { return exp2_fast(a_log * kLog2e); }
__device__ __forceinline__ float log_decay(float x, float dt_bias, float rate) {
    return -rate * softplus_fast(x + dt_bias);
}

// 16x16x4 fp32 MFMA: D[m][n] = sum_k A[m][k] B[k][n] + C[m][n].
// Lane l supplies A[l%16][l/16] and B[l/16][l%16]; on return lane l holds
// D[4*(l/16) + i][l%16] in element i.
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA with fp32 accumulation: lane l supplies A[l%16][8*(l/16)+j]
// and B[8*(l/16)+j][l%16] for j = 0..7; the result layout is that of mfma4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split fp32 values into bf16 hi = rne(x) and lo = rne(x - hi): hi + lo
// carries x to about 2^-16 relative, so hi*hi + hi*lo + lo*hi gives an
// fp32-grade product on the bf16 matrix units.  Pairs are packed as the
// matrix units read them (element 2i in the low half of 32-bit word i).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
}
// x - hi is exact in fp32; it is formed on the bf16 dot-product unit as
// (-1, 0) . (hi_a, hi_b) + a (products of bf16 values are exact), one
// instruction per value instead of a widening and a subtraction.  The pair
// (-1, 0) (bits 0x0000bf80) goes through a scalar register: as an immediate
// the compiler encodes it as the inline constant -1.0, which the hardware
// expands to the bits 0xbf800000, i.e. the pair (0, -1) (checked on gfx950).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    const bf16x2 h = __builtin_convertvector(floatx2{a, b}, bf16x2);
    hi = __builtin_bit_cast(uint32_t, h);
    uint32_t m1_lo = 0x0000bf80u;   // (-1, 0)
    asm("" : "+s"(m1_lo));
    const float la = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1_lo), a, false);
    const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, bf16x2{(__bf16)0.0f, (__bf16)-1.0f}, b, false);
    lo = pk_bf16(la, lb);
}
// four values -> 8 bytes hi, 8 bytes lo
__device__ __forceinline__ void split4(const float4 &x, uint2 &hi, uint2 &lo) {
    split2(x.x, x.y, hi.x, lo.x);
    split2(x.z, x.w, hi.y, lo.y);
}
// eight values (a then b) -> one 16x16x32 operand each for hi and lo
__device__ __forceinline__ void split8(const float4 &a, const float4 &b, bf16x8 &hi, bf16x8 &lo) {
    uint2 ha, la, hb, lb;
    split4(a, ha, la);
    split4(b, hb, lb);
    hi = __builtin_bit_cast(bf16x8, make_uint4(ha.x, ha.y, hb.x, hb.y));
    lo = __builtin_bit_cast(bf16x8, make_uint4(la.x, la.y, lb.x, lb.y));
}

__device__ __forceinline__ float get4(const float4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace kda
