// Per-row device code shared by the stage kernels and the fused block-decode
// mixer, so that every kernel that runs a stage runs the same instructions on
// the same values (and gives the same bits).
#pragma once

#include "kda_device.hpp"

namespace kda {

constexpr int kConvKC = 4;   // conv taps (the "Glm5NextKdaWeights" page, conv: [conv_dim, 4])

// The taps of channels c0 .. c0 + 7: wt[e][j] = w[c0 + e][j], as loaded
// (four 16-byte pieces) and unpacked.
__device__ __forceinline__ void conv_taps_load(const uint16_t *__restrict__ w, int64_t c0,
                                               uint4 (&raw)[kConvKC])
{
    const uint4 *wp = reinterpret_cast<const uint4 *>(w + c0 * kConvKC);
#pragma unroll
    for (int p = 0; p < kConvKC; ++p) raw[p] = wp[p];
}
__device__ __forceinline__ void conv_taps_unpack(const uint4 (&raw)[kConvKC], float (&wt)[8][kConvKC])
{
    float f[8];
#pragma unroll
    for (int p = 0; p < kConvKC; ++p) {
        unpack8(raw[p], f);   // channels 2p, 2p+1, each kConvKC taps
#pragma unroll
        for (int e = 0; e < 8; ++e) wt[(p * 8 + e) / kConvKC][(p * 8 + e) % kConvKC] = f[e];
    }
}
__device__ __forceinline__ void conv_taps(const uint16_t *__restrict__ w, int64_t c0,
                                          float (&wt)[8][kConvKC])
{
    uint4 raw[kConvKC];
    conv_taps_load(w, c0, raw);
    conv_taps_unpack(raw, wt);
}

// One row of conv + SiLU + (q and k sections) L2 for this lane's 8
// channels: win holds the last kConvKC pre-conv rows (newest last), LANES
// adjacent lanes (aligned) hold the head's channels of the section.
//   pre = sum_j w[c][j] * win[j][c];  s = pre * sigmoid(pre)
//   q, k: s /= sqrt(sum over the head's channels of s^2 + eps)
// exp, reciprocal and rsqrt on the transcendental unit; one bf16 rounding.
template <int LANES>
__device__ __forceinline__ uint4 conv_row(const uint4 (&win)[kConvKC],
                                          const float (&wt)[8][kConvKC], bool normalise,
                                          float eps)
{
    float xv[kConvKC][8];
#pragma unroll
    for (int j = 0; j < kConvKC; ++j) unpack8(win[j], xv[j]);
    float s[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float pre = wt[e][0] * xv[0][e];
#pragma unroll
        for (int j = 1; j < kConvKC; ++j) pre = __builtin_fmaf(wt[e][j], xv[j][e], pre);
        s[e] = pre * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-pre * kLog2e));
        ss = __builtin_fmaf(s[e], s[e], ss);
    }
#pragma unroll
    for (int off = 1; off < LANES; off <<= 1) ss += __shfl_xor(ss, off);
    if (normalise) {
        const float inv = __builtin_amdgcn_rsqf(ss + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] *= inv;
    }
    return pack8(s);
}

// Sigmoid-gated RMSNorm of 8 consecutive channels of one (row, head), the
// head's D / 8 lanes adjacent and aligned:
//   out = bf16( x * rsqrt(mean x^2 + eps) * w * sigmoid(gate) )
template <int D>
__device__ __forceinline__ uint4 gated_norm8(const float (&xv)[8], const uint4 &gate,
                                             const uint4 &w, float eps)
{
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(xv[e], xv[e], ss);
#pragma unroll
    for (int off = 1; off < D / 8; off <<= 1) ss += __shfl_xor(ss, off);
    const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
    float g[8], wv[8], o[8];
    unpack8(gate, g);
    unpack8(w, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        o[e] = xv[e] * r * wv[e] * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-g[e] * kLog2e));
    return pack8(o);
}

}  // namespace kda
