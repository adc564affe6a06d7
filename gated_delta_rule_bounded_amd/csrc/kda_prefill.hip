// Chunked KDA prefill from a carried state ("Glm5NextKdaLayer" page, prefill
// and prefill_with_pad_fill; "Glm5NextKdaWorkspace" page, fields q_f32, gate,
// beta, core).
//
// The token-serial recurrence (per head, S[i][j], i = key channel):
//   S <- diag(e^{g_t}) S;  u_t = b_t (v_t - S^T k_t);  S <- S + k_t u_t^T;
//   o_t = scale S^T q_t
// is rewritten exactly over chunks of C tokens.  With G the in-chunk inclusive
// cumulative log-decay (per channel), for rows r, s of one chunk:
//   A[r][s] = sum_d k_r k_s e^{G_r - G_s}  (s <  r)      decayed key Gram matrix
//   P[r][s] = sum_d q_r k_s e^{G_r - G_s}  (s <= r)      decayed query-key scores
//   Tb      = (I + diag(b) A)^{-1} diag(b)                 UT transform of the chain
//   X       = V - (K e^{G}) S                              residual against the carried S
//   U       = Tb X                                         corrected writes u_r
//   O       = scale ((Q e^{G}) S + P U)
//   S'      = diag(e^{G_C}) S + (K e^{G_C - G})^T U
// (Expanding u_r = b_r (v_r - k_r^T-weighted prediction) row by row gives
// (I + diag(b) A) U = diag(b) X, the WY/UT form named on the "Glm5NextLayer"
// page, write-on-accept section, as the table-form WY.)
//
// Kernel split, designed for gfx950:
//   kda_chunk_prep  — one workgroup per (chunk, head), all chunks in parallel:
//                     cumulative decay, A and P on fp32 MFMA, the 64x64
//                     unit-lower-triangular inverse by 16x16 blocks (forward
//                     substitution on the diagonal blocks, MFMA for the rest).
//                     Writes Tb and P (C x C each) to the workspace.
//   kda_chunk_fwd   — one workgroup per (head, 16-column slice of the value
//                     axis); walks the chunks in order with its D x 16 state
//                     slice in registers.  Per chunk: two D-deep MFMA products
//                     against S, two C-deep triangular products, the rank-C
//                     state update, all fp32 MFMA.
// Decay factors are always formed as 2^{x} with x <= 0 except on a diagonal
// 16x16 block, where the factor is split around the block's last row and the
// positive exponent is bounded by the block's decay span; a block whose span
// could overflow fp32 takes an exact pairwise path instead.
//
// Rows t >= T (the pad tail) are replaced by zero (k, q, v, beta) and zero
// log-decay by a select at load time, never by arithmetic with their bits, so
// poison in the tail cannot change a single bit of the result.  Chunks wholly
// past T are not visited; core rows >= T are not written.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kPadK = 4;            // LDS row padding (floats) of [C][D] tiles
constexpr int kPadC = 4;            // ... of [C][C] tiles
constexpr int kPad16 = 4;           // ... of [rows][16] tiles
constexpr float kSpanLimit = 86.0f; // log2 units: largest diagonal-block decay span factored

template <int D, int C>
struct PrefCfg {
    static constexpr int kNW = C / 16;   // waves per workgroup: wave w owns chunk rows 16w..16w+15
    static constexpr int kDT = D / 16;   // 16-wide channel tiles
    static constexpr int kThreads = kNW * kWave;
};

__device__ __forceinline__ float4 shfl4(const float4 &v, int src) {
    return make_float4(__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src));
}
__device__ __forceinline__ float4 add4(const float4 &a, const float4 &b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 sub4(const float4 &a, const float4 &b) {
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 mul4(const float4 &a, const float4 &b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 exp2_4(const float4 &a) {
    return make_float4(exp2_fast(a.x), exp2_fast(a.y), exp2_fast(a.z), exp2_fast(a.w));
}
__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// Load this lane's A-layout slice of chunk row (channels 16*t8 + 4*lg .. +3
// for every tile t8) of k, q and the gate.  The loads are unconditional: a
// chunk never extends past T_pad rows, so every row it touches is in bounds;
// rows past T are replaced afterwards by select_rows.  Keeping the loads free
// of branches and arithmetic lets them stay in flight across other work.
template <int D>
__device__ __forceinline__ void load_rows(const float *__restrict__ q, const float *__restrict__ k,
                                          const float *__restrict__ gate, int64_t roff, int lg,
                                          float4 (&K)[D / 16], float4 (&Q)[D / 16],
                                          float4 (&G)[D / 16])
{
#pragma unroll
    for (int t8 = 0; t8 < D / 16; ++t8) {
        const int d0 = 16 * t8 + 4 * lg;
        K[t8] = *reinterpret_cast<const float4 *>(k + roff + d0);
        Q[t8] = *reinterpret_cast<const float4 *>(q + roff + d0);
        G[t8] = *reinterpret_cast<const float4 *>(gate + roff + d0);
    }
}

// Rows past T become k = q = 0 and zero log-decay (a select, so the bits they
// held never reach the arithmetic); the gate is scaled to log2 units.
template <int D>
__device__ __forceinline__ void select_rows(bool valid, float4 (&K)[D / 16], float4 (&Q)[D / 16],
                                            float4 (&G)[D / 16])
{
#pragma unroll
    for (int t8 = 0; t8 < D / 16; ++t8) {
        const float4 g = G[t8];
        K[t8] = valid ? K[t8] : zero4();
        Q[t8] = valid ? Q[t8] : zero4();
        G[t8] = valid ? make_float4(g.x * kLog2e, g.y * kLog2e, g.z * kLog2e, g.w * kLog2e)
                      : zero4();
    }
}

// Row shift within each 16-lane DPP row; lanes shifted in from outside the
// row read 0.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf,
                                                      true));
}

// In-chunk inclusive prefix over rows of the log2 gate, in two phases so the
// cross-wave exchange can share a barrier with other work.  Wave w owns chunk
// rows 16w + lr (lr = lane % 16, one DPP row of the wave); for channel tile
// t8 the lane holds channels 16*t8 + 4*lg .. +3.
//   scan_local: Hillis-Steele over the 16 lanes of each row (DPP row shifts),
//               then (NW > 1) the wave's row totals to s_tot.
//   scan_carry: after a barrier, add the totals of the preceding waves in wave
//               order; Gend = the chunk's last row (the chunk total).
// Both prefill kernels use these with the same layout, so they see bitwise the
// same cumulative decay.
template <int D, int NW>
__device__ __forceinline__ void scan_local(float4 (&G)[D / 16], float *s_tot, int w, int lane)
{
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t8 = 0; t8 < D / 16; ++t8) {
        float4 g = G[t8];
        g = add4(g, make_float4(row_shr<1>(g.x), row_shr<1>(g.y), row_shr<1>(g.z), row_shr<1>(g.w)));
        g = add4(g, make_float4(row_shr<2>(g.x), row_shr<2>(g.y), row_shr<2>(g.z), row_shr<2>(g.w)));
        g = add4(g, make_float4(row_shr<4>(g.x), row_shr<4>(g.y), row_shr<4>(g.z), row_shr<4>(g.w)));
        g = add4(g, make_float4(row_shr<8>(g.x), row_shr<8>(g.y), row_shr<8>(g.z), row_shr<8>(g.w)));
        G[t8] = g;
        if (NW > 1 && lr == 15)
            *reinterpret_cast<float4 *>(s_tot + w * D + 16 * t8 + 4 * lg) = g;
    }
}

template <int D, int NW>
__device__ __forceinline__ void scan_carry(float4 (&G)[D / 16], float4 (&Gend)[D / 16],
                                           const float *s_tot, int w, int lane)
{
    const int lg = lane >> 4;
    if constexpr (NW > 1) {
#pragma unroll
        for (int t8 = 0; t8 < D / 16; ++t8) {
            float4 tot[NW];
#pragma unroll
            for (int ww = 0; ww < NW; ++ww)
                tot[ww] = *reinterpret_cast<const float4 *>(s_tot + ww * D + 16 * t8 + 4 * lg);
            float4 run = zero4(), carry = zero4();
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                if (ww == w) carry = run;   // w is wave-uniform: a scalar branch
                run = add4(run, tot[ww]);
            }
            G[t8] = add4(G[t8], carry);
            Gend[t8] = run;
        }
    } else {
#pragma unroll
        for (int t8 = 0; t8 < D / 16; ++t8) Gend[t8] = shfl4(G[t8], (lane & 48) | 15);
    }
}

template <int D, int NW>
__device__ __forceinline__ void chunk_cumsum(float4 (&G)[D / 16], float4 (&Gend)[D / 16],
                                             float *s_tot, int w, int lane)
{
    scan_local<D, NW>(G, s_tot, w, lane);
    if (NW > 1) __syncthreads();
    scan_carry<D, NW>(G, Gend, s_tot, w, lane);
}

// ---------------------------------------------------------------------------
// kda_chunk_prep: per (chunk n, head h) -> Tb = (I + diag(b) A)^{-1} diag(b)
// and P (masked lower triangle), both [C][C] fp32 in the workspace.
// ---------------------------------------------------------------------------
template <int D, int C>
__global__ __launch_bounds__(C / 16 * 64) void kda_chunk_prep_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ gate,
    const float *__restrict__ beta, int T, int H, float *__restrict__ Tb_out,
    float *__restrict__ P_out)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    const int n = blockIdx.x, h = blockIdx.y;
    // wave index, uniform across the wave (scalar register)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int rl = 16 * w + lr;
    const int64_t tg = (int64_t)n * C + rl;
    const bool valid = tg < T;
    const int64_t roff = (tg * H + h) * D;

    __shared__ __align__(16) float s_tot[NW * D];
    __shared__ __align__(16) float s_kc[C][D + kPadK];
    __shared__ __align__(16) float s_M[C][C + kPadC];
    __shared__ __align__(16) float s_T[C][C + kPadC];
    __shared__ float s_beta[C];

    float4 K[DT], Q[DT], G[DT], Gend[DT];
    load_rows<D>(q, k, gate, roff, lg, K, Q, G);
    const float braw = beta[tg * H + h];
    select_rows<D>(valid, K, Q, G);
    if (lg == 0) s_beta[rl] = valid ? braw : 0.f;
    chunk_cumsum<D, NW>(G, Gend, s_tot, w, lane);

    // Column operand Kc = K e^{G_last - G}, relative to the last row of this
    // wave's 16-row block (all factors <= 1); also the block's decay span.
    float span = 0.f;
    float4 Gl[DT];
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) {
        Gl[t8] = shfl4(G[t8], (lane & 48) | 15);
        const float4 Gf = shfl4(G[t8], lane & 48);
        const float4 e = exp2_4(sub4(Gl[t8], G[t8]));
        *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = mul4(K[t8], e);
        span = fmaxf(span, fmaxf(fmaxf(Gf.x - Gl[t8].x, Gf.y - Gl[t8].y),
                                 fmaxf(Gf.z - Gl[t8].z, Gf.w - Gl[t8].w)));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) span = fmaxf(span, __shfl_xor(span, off));
    const bool diag_ok = span <= kSpanLimit;
    __syncthreads();

    // Block row w of A and P: tiles (w, bj) for bj <= w.  Row operand relative
    // to the last row of block bj: exponent G_r - G_ref <= 0 off the diagonal,
    // in [0, span] on it.
    floatx4 Aacc[NW], Pacc[NW];
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) {
        Aacc[bj] = floatx4{0.f, 0.f, 0.f, 0.f};
        Pacc[bj] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (bj > w || (bj == w && !diag_ok)) continue;
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            float4 ref = Gl[t8];
            if (bj < w) {
                ref = zero4();
#pragma unroll
                for (int ww = 0; ww <= bj; ++ww)
                    ref = add4(ref, *reinterpret_cast<const float4 *>(s_tot + ww * D + 16 * t8 + 4 * lg));
            }
            const float4 e = exp2_4(sub4(G[t8], ref));
            const float4 kr = mul4(K[t8], e), qr = mul4(Q[t8], e);
            const float4 kc = *reinterpret_cast<const float4 *>(&s_kc[16 * bj + lr][16 * t8 + 4 * lg]);
            Aacc[bj] = mfma4(kr.x, kc.x, Aacc[bj]);
            Pacc[bj] = mfma4(qr.x, kc.x, Pacc[bj]);
            Aacc[bj] = mfma4(kr.y, kc.y, Aacc[bj]);
            Pacc[bj] = mfma4(qr.y, kc.y, Pacc[bj]);
            Aacc[bj] = mfma4(kr.z, kc.z, Aacc[bj]);
            Pacc[bj] = mfma4(qr.z, kc.z, Pacc[bj]);
            Aacc[bj] = mfma4(kr.w, kc.w, Aacc[bj]);
            Pacc[bj] = mfma4(qr.w, kc.w, Pacc[bj]);
        }
    }

    // Exact pairwise diagonal block when its span is too wide to factor.
    if (__syncthreads_or(!diag_ok)) {
        if (!diag_ok) {
#pragma unroll
            for (int t8 = 0; t8 < DT; ++t8)
                *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = G[t8];
        }
        __syncthreads();
        if (!diag_ok) {
            float da[4], dp[4];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int r = 16 * w + 4 * lg + vv, s = 16 * w + lr;
                float a = 0.f, p = 0.f;
                const int64_t tr = (int64_t)n * C + r, ts = (int64_t)n * C + s;
                if (s <= r && ts < T) {
                    const float *kr = k + (tr * H + h) * D, *qr = q + (tr * H + h) * D;
                    const float *ks = k + (ts * H + h) * D;
                    const bool rv = tr < T;
                    for (int d = 0; d < D; ++d) {
                        const float e = exp2_fast(s_kc[r][d] - s_kc[s][d]);
                        const float kse = ks[d] * e;
                        if (rv) {
                            a = __builtin_fmaf(kr[d], kse, a);
                            p = __builtin_fmaf(qr[d], kse, p);
                        }
                    }
                }
                da[vv] = a;
                dp[vv] = p;
            }
#pragma unroll
            for (int bj = 0; bj < NW; ++bj)
                if (bj == w) Aacc[bj] = floatx4{da[0], da[1], da[2], da[3]},
                             Pacc[bj] = floatx4{dp[0], dp[1], dp[2], dp[3]};
        }
    }

    // Masked tiles: M = diag(b) A (strictly lower) to LDS, P to the workspace.
    float *Pn = P_out + ((int64_t)n * H + h) * C * C;
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) {
        if (bj > w) continue;
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            const int r = 16 * w + 4 * lg + vv, s = 16 * bj + lr;
            float a = Aacc[bj][vv], p = Pacc[bj][vv];
            if (bj == w) {
                if (s >= r) a = 0.f;
                if (s > r) p = 0.f;
            }
            s_M[r][s] = s_beta[r] * a;
            Pn[(int64_t)r * C + s] = p;
        }
    }
    __syncthreads();

    // T = (I + M)^{-1}, M strictly lower.  Diagonal 16x16 blocks by forward
    // substitution (lane lr solves column lr), then block levels
    // T_ij = -T_ii sum_{m=j}^{i-1} M_im T_mj on MFMA.
    {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc = __builtin_fmaf(-s_M[16 * w + r][16 * w + s], x[s], acc);
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r >> 2) == lg) s_T[16 * w + r][16 * w + lr] = x[r];
    }
    __syncthreads();
    for (int lev = 1; lev < NW; ++lev) {
        if (w >= lev) {
            const int i = w, j = w - lev;
            floatx4 X = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < i; ++m) {
                const float4 ma = *reinterpret_cast<const float4 *>(&s_M[16 * i + lr][16 * m + 4 * lg]);
                X = mfma4(ma.x, s_T[16 * m + 4 * lg + 0][16 * j + lr], X);
                X = mfma4(ma.y, s_T[16 * m + 4 * lg + 1][16 * j + lr], X);
                X = mfma4(ma.z, s_T[16 * m + 4 * lg + 2][16 * j + lr], X);
                X = mfma4(ma.w, s_T[16 * m + 4 * lg + 3][16 * j + lr], X);
            }
            const float4 ta = *reinterpret_cast<const float4 *>(&s_T[16 * i + lr][16 * i + 4 * lg]);
            floatx4 Y = {0.f, 0.f, 0.f, 0.f};
            Y = mfma4(ta.x, X[0], Y);
            Y = mfma4(ta.y, X[1], Y);
            Y = mfma4(ta.z, X[2], Y);
            Y = mfma4(ta.w, X[3], Y);
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) s_T[16 * i + 4 * lg + vv][16 * j + lr] = -Y[vv];
        }
        __syncthreads();
    }

    // Tb = T diag(b), lower block triangle of block row w.
    float *Tn = Tb_out + ((int64_t)n * H + h) * C * C;
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) {
        if (bj > w) continue;
        const int s = 16 * bj + lr;
        const float bs = s_beta[s];
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            const int r = 16 * w + 4 * lg + vv;
            Tn[(int64_t)r * C + s] = s_T[r][s] * bs;
        }
    }
}

// ---------------------------------------------------------------------------
// kda_chunk_fwd: per (head h, value slice j0..j0+15), serial over chunks.
//
// Software pipeline: the global loads of chunk n+1 (this wave's 16 rows of
// k, q, gate, the v slice, and its rows of Tb and P) are issued at the top of
// iteration n and consumed after its last barrier, so their latency overlaps
// the MFMA work of chunk n.  The in-chunk scan of chunk n+1 shares that last
// barrier with the state broadcast, leaving three barriers per chunk:
//   B1  X rows and Kd rows visible      (U needs X of waves <= w)
//   B2  U rows visible                  (P U and the state update need U)
//   B3  new state slice and scan totals visible
// ---------------------------------------------------------------------------
template <int D, int C>
struct FwdRows {
    float4 K[D / 16], Q[D / 16], G[D / 16];   // A-layout row slices of k, q, gate
    float V[4];                               // v[16w + 4lg + i][j0 + lr]
    float4 Tb[C / 16], P[C / 16];             // Tb, P row 16w + lr, columns 16w2 + 4lg ..
};

template <int D, int C>
__device__ __forceinline__ void fwd_load(FwdRows<D, C> &R, const float *__restrict__ q,
                                         const float *__restrict__ k, const float *__restrict__ v,
                                         const float *__restrict__ gate,
                                         const float *__restrict__ Tb,
                                         const float *__restrict__ Pm, int n, int T, int H, int h,
                                         int j0, int w, int lr, int lg)
{
    constexpr int NW = C / 16;
    const int64_t tg = (int64_t)n * C + 16 * w + lr;
    load_rows<D>(q, k, gate, (tg * H + h) * D, lg, R.K, R.Q, R.G);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t tr = (int64_t)n * C + 16 * w + 4 * lg + i;
        R.V[i] = v[(tr * H + h) * D + j0 + lr];
    }
    // the blocks above the diagonal are loaded (in bounds) but never used
    const int64_t toff = (((int64_t)n * H + h) * C + 16 * w + lr) * C + 4 * lg;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
        R.Tb[w2] = *reinterpret_cast<const float4 *>(Tb + toff + 16 * w2);
        R.P[w2] = *reinterpret_cast<const float4 *>(Pm + toff + 16 * w2);
    }
}

// Pad-row selects of a loaded chunk (see select_rows), applied when the
// chunk's values are first used.
template <int D, int C>
__device__ __forceinline__ void fwd_select(FwdRows<D, C> &R, int n, int T, int w, int lr, int lg)
{
    select_rows<D>((int64_t)n * C + 16 * w + lr < T, R.K, R.Q, R.G);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        R.V[i] = ((int64_t)n * C + 16 * w + 4 * lg + i < T) ? R.V[i] : 0.f;
}

template <int D, int C>
__global__ __launch_bounds__(C / 16 * 64) void kda_chunk_fwd_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ gate, float *__restrict__ state, float *__restrict__ core,
    const float *__restrict__ Tb, const float *__restrict__ Pm, int T, int NC, int H,
    float scale)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    // all value slices of one head share an XCD (workgroups are dealt to the
    // 8 XCDs round-robin), so they share that XCD's L2 copy of q/k/gate/Tb/P
    const int h = blockIdx.x % H, jt = blockIdx.x / H, j0 = 16 * jt;
    // wave index, uniform across the wave (scalar register)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int rl = 16 * w + lr;

    __shared__ __align__(16) float s_tot[NW * D];
    __shared__ __align__(16) float s_kd[C][D + kPadK];
    __shared__ float s_x[C][16 + kPad16];
    __shared__ float s_u[C][16 + kPad16];
    __shared__ float s_S[D][16 + kPad16];

    // S slice in MFMA output layout: Sr[t8][i] = S[16*t8 + 4*lg + i][j0 + lr]
    float *__restrict__ Sg = state + (int64_t)h * D * D;
    floatx4 Sr[DT];
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sr[t8][i] = Sg[(int64_t)(16 * t8 + 4 * lg + i) * D + j0 + lr];

    FwdRows<D, C> R;
    float4 Kg[DT], Qg[DT], Gend[DT];
    float V[4];
    float4 TbR[NW], PR[NW];

    // chunk 0: load, scan, operands
    fwd_load<D, C>(R, q, k, v, gate, Tb, Pm, 0, T, H, h, j0, w, lr, lg);
    fwd_select<D, C>(R, 0, T, w, lr, lg);
    scan_local<D, NW>(R.G, s_tot, w, lane);
    if (NW > 1) __syncthreads();

    for (int n = 0; n < NC; ++n) {
        // ---- operands of chunk n from R (its scan totals are in s_tot) ----
        scan_carry<D, NW>(R.G, Gend, s_tot, w, lane);
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            const float4 ed = exp2_4(sub4(Gend[t8], R.G[t8]));
            *reinterpret_cast<float4 *>(&s_kd[rl][16 * t8 + 4 * lg]) = mul4(R.K[t8], ed);
            const float4 eg = exp2_4(R.G[t8]);
            Kg[t8] = mul4(R.K[t8], eg);
            Qg[t8] = mul4(R.Q[t8], eg);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) V[i] = R.V[i];
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            TbR[w2] = R.Tb[w2];
            PR[w2] = R.P[w2];
        }
        // ---- prefetch chunk n+1 ----
        if (n + 1 < NC) fwd_load<D, C>(R, q, k, v, gate, Tb, Pm, n + 1, T, H, h, j0, w, lr, lg);

        // X = V - (K e^G) S ;  QS = (Q e^G) S   (rows 16w.., D-deep products)
        floatx4 X = {V[0], V[1], V[2], V[3]}, QS = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            X = mfma4(-Kg[t8].x, Sr[t8][0], X);
            QS = mfma4(Qg[t8].x, Sr[t8][0], QS);
            X = mfma4(-Kg[t8].y, Sr[t8][1], X);
            QS = mfma4(Qg[t8].y, Sr[t8][1], QS);
            X = mfma4(-Kg[t8].z, Sr[t8][2], X);
            QS = mfma4(Qg[t8].z, Sr[t8][2], QS);
            X = mfma4(-Kg[t8].w, Sr[t8][3], X);
            QS = mfma4(Qg[t8].w, Sr[t8][3], QS);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s_x[16 * w + 4 * lg + i][lr] = X[i];
        __syncthreads();   // B1

        // U = Tb X  (block row w, lower triangle)
        floatx4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            if (w2 > w) continue;
            U = mfma4(TbR[w2].x, s_x[16 * w2 + 4 * lg + 0][lr], U);
            U = mfma4(TbR[w2].y, s_x[16 * w2 + 4 * lg + 1][lr], U);
            U = mfma4(TbR[w2].z, s_x[16 * w2 + 4 * lg + 2][lr], U);
            U = mfma4(TbR[w2].w, s_x[16 * w2 + 4 * lg + 3][lr], U);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s_u[16 * w + 4 * lg + i][lr] = U[i];
        __syncthreads();   // B2

        // O = scale (QS + P U)
        floatx4 O = QS;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            if (w2 > w) continue;
            O = mfma4(PR[w2].x, s_u[16 * w2 + 4 * lg + 0][lr], O);
            O = mfma4(PR[w2].y, s_u[16 * w2 + 4 * lg + 1][lr], O);
            O = mfma4(PR[w2].z, s_u[16 * w2 + 4 * lg + 2][lr], O);
            O = mfma4(PR[w2].w, s_u[16 * w2 + 4 * lg + 3][lr], O);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t tr = (int64_t)n * C + 16 * w + 4 * lg + i;
            if (tr < T) core[(tr * H + h) * D + j0 + lr] = scale * O[i];
        }

        // S' = diag(e^{G_C}) S + Kd^T U for the channel tiles this wave owns
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            if (t8 % NW != w) continue;
            const float4 ec = exp2_4(Gend[t8]);
            floatx4 acc = {Sr[t8][0] * ec.x, Sr[t8][1] * ec.y, Sr[t8][2] * ec.z, Sr[t8][3] * ec.w};
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma4(s_kd[16 * w2 + 4 * lg + kk][16 * t8 + lr],
                                s_u[16 * w2 + 4 * lg + kk][lr], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) s_S[16 * t8 + 4 * lg + i][lr] = acc[i];
        }
        // in-row scan of chunk n+1 (its loads were issued above)
        if (n + 1 < NC) {
            fwd_select<D, C>(R, n + 1, T, w, lr, lg);
            scan_local<D, NW>(R.G, s_tot, w, lane);
        }
        __syncthreads();   // B3
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sr[t8][i] = s_S[16 * t8 + 4 * lg + i][lr];
    }

#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) {
        if (t8 % NW != w) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) Sg[(int64_t)(16 * t8 + 4 * lg + i) * D + j0 + lr] = Sr[t8][i];
    }
}

size_t prefill_workspace_bytes(int T_pad, int heads, int head_dim, int chunk)
{
    (void)head_dim;
    // Tb and P: [T_pad/chunk, heads, chunk, chunk] fp32 each
    return 2 * (size_t)(T_pad / chunk) * heads * chunk * chunk * sizeof(float);
}

template <int D, int C>
static hipError_t prepare_t(const float *q, const float *k, const float *gate,
                            const float *beta, int T, int T_pad, int H, void *workspace,
                            hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    float *Tb = static_cast<float *>(workspace);
    float *Pm = Tb + (size_t)(T_pad / C) * H * C * C;
    hipLaunchKernelGGL((kda_chunk_prep_kernel<D, C>), dim3(NC, H), dim3(PrefCfg<D, C>::kThreads),
                       0, stream, q, k, gate, beta, T, H, Tb, Pm);
    return hipGetLastError();
}

template <int D, int C>
static hipError_t forward_t(const float *q, const float *k, const float *v, const float *gate,
                            float *state, float *core, int T, int T_pad, int H, float scale,
                            const void *workspace, hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    const float *Tb = static_cast<const float *>(workspace);
    const float *Pm = Tb + (size_t)(T_pad / C) * H * C * C;
    hipLaunchKernelGGL((kda_chunk_fwd_kernel<D, C>), dim3(H * PrefCfg<D, C>::kDT),
                       dim3(PrefCfg<D, C>::kThreads), 0, stream, q, k, v, gate, state, core, Tb,
                       Pm, T, NC, H, scale);
    return hipGetLastError();
}

#define KDA_PREFILL_DISPATCH(FN, ...)                                        \
    (head_dim == 128 && chunk == 64)   ? FN<128, 64>(__VA_ARGS__)            \
    : (head_dim == 128 && chunk == 16) ? FN<128, 16>(__VA_ARGS__)            \
    : (head_dim == 16 && chunk == 64)  ? FN<16, 64>(__VA_ARGS__)             \
                                       : FN<16, 16>(__VA_ARGS__)

hipError_t launch_kda_prefill_prepare(const float *q, const float *k, const float *gate,
                                      const float *beta, int T, int T_pad, int heads,
                                      int head_dim, int chunk, void *workspace,
                                      hipStream_t stream)
{
    return KDA_PREFILL_DISPATCH(prepare_t, q, k, gate, beta, T, T_pad, heads, workspace, stream);
}

hipError_t launch_kda_prefill_forward(const float *q, const float *k, const float *v,
                                      const float *gate, float *state, float *core, int T,
                                      int T_pad, int heads, int head_dim, int chunk, float scale,
                                      const void *workspace, hipStream_t stream)
{
    return KDA_PREFILL_DISPATCH(forward_t, q, k, v, gate, state, core, T, T_pad, heads, scale,
                                workspace, stream);
}

hipError_t launch_kda_prefill(const float *q, const float *k, const float *v,
                              const float *gate, const float *beta, float *state,
                              float *core, int T, int T_pad, int heads, int head_dim,
                              int chunk, float scale, void *workspace, hipStream_t stream)
{
    hipError_t e = launch_kda_prefill_prepare(q, k, gate, beta, T, T_pad, heads, head_dim, chunk,
                                              workspace, stream);
    if (e != hipSuccess) return e;
    return launch_kda_prefill_forward(q, k, v, gate, state, core, T, T_pad, heads, head_dim,
                                      chunk, scale, workspace, stream);
}

}  // namespace kda
