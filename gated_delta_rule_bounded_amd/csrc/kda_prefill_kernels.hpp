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
#pragma once

#include <algorithm>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kPadK = 4;            // LDS row padding (floats) of [C][D] tiles
constexpr int kPadC = 4;            // ... of [C][C] tiles
constexpr int kPad16 = 4;           // ... of [rows][16] tiles
constexpr float kSpanLimit = 86.0f; // log2 units: largest diagonal-block decay span factored

// ---------------------------------------------------------------------------
// Several sequences in one launch ("Glm5NextLayer" page, batched and varlen
// linear-attention prefill: one state pointer per sequence, the sequences'
// tokens back to back, row offsets cu_seqlens).  Sequence s owns rows
// [cu[s], cu[s+1]) of the row arrays and the dense run of operand blocks that
// follows the blocks of sequences 0..s-1.  A workgroup maps itself onto its
// sequence and then runs exactly the single-sequence code: the rows of the
// next sequence past the end of its last chunk are pad rows to it, replaced
// at load time like any pad tail.  A launch covers the global chunks
// [seg_lo, seg_hi) only (a cache-sized segment); a sequence that straddles a
// segment boundary continues in the next launch from the state the previous
// one stored, on the same chunk grid, so the result does not depend on the
// segmentation.  cu == nullptr: one sequence, the plain arguments apply.
//
// The lengths live in device memory.  Every launch of a call sizes its grid
// by the segment alone (a prepare workgroup per chunk of the segment, a walk
// workgroup per sequence in it), and each workgroup finds its sequence:
//   at most kWave sequences: from cu directly, one lane per sequence (a load
//     and a prefix sum across the wave);
//   more: in tables that a small plan kernel (one workgroup, once per call)
//     builds from cu, with a few reads, whatever the number of sequences.
// Plan layout, int32:
//   seq_of[total_chunks]  sequence owning global chunk g (-1: no sequence)
//   chunk0[B]             first global chunk of sequence s (chunks of the
//                         sequences before it; total_chunks + 1 when past it)
//   rank[B + 1]           walked sequences before s (rank[B]: all of them)
//   by_rank[B]            the r-th walked sequence
// A sequence is walked when it has chunks and they fit: nch <= max_chunks
// and chunk0 + nch <= total_chunks; one that does not fit is skipped.
// ---------------------------------------------------------------------------
struct Varlen {
    const int32_t *cu;      // [B + 1] row offsets, or nullptr
    float *const *states;   // [B] state pointers (forward)
    int64_t rows;           // rows held by the row arrays
    int32_t B;              // sequences
    int32_t max_chunks;     // chunks of the longest sequence
    int32_t total_chunks;   // chunks of all sequences
    int32_t seg_lo, seg_hi; // global chunks of this launch; block 0 of the workspace = seg_lo
    const int32_t *plan;    // the plan kernel's tables (B > kWave), else nullptr
    int32_t *status;        // report word (B <= kWave; the plan kernel reports otherwise)
};

inline size_t varlen_plan_ints(int B, int total_chunks)
{
    return (size_t)total_chunks + 3 * (size_t)B + 1;
}

struct SeqSpan {
    int64_t row0, chunk0;
    int T, nch;
    bool ok;   // walked: inside the workspace and max_chunks
};

// Rows of sequence i, clamped to [0, rows): the same clamp for every i, so
// chunk offsets and chunk counts agree between all workgroups.
__device__ __forceinline__ void seq_rows(const int32_t *cu, int64_t rows, int i, int64_t &lo,
                                         int64_t &hi)
{
    lo = min(max((int64_t)cu[i], (int64_t)0), rows);
    hi = min(max((int64_t)cu[i + 1], lo), rows);
}

template <int C>
__device__ __forceinline__ SeqSpan seq_span(const Varlen &vl, int s, int64_t chunk0)
{
    SeqSpan r;
    int64_t hi;
    seq_rows(vl.cu, vl.rows, s, r.row0, hi);
    r.T = (int)(hi - r.row0);
    r.nch = (r.T + C - 1) / C;
    r.chunk0 = chunk0;
    r.ok = r.nch <= vl.max_chunks && r.chunk0 + r.nch <= vl.total_chunks;
    return r;
}

// At most kWave sequences: lane i's view of sequence i (chunk offset, chunk
// count, walked), the same on every wave of every workgroup.
struct WaveSeq {
    int64_t c0;
    int nch;
    bool walk;
};

template <int C>
__device__ __forceinline__ WaveSeq wave_seq(const Varlen &vl)
{
    const int lane = threadIdx.x & 63;
    int64_t nch = 0;
    if (lane < vl.B) {
        int64_t lo, hi;
        seq_rows(vl.cu, vl.rows, lane, lo, hi);
        nch = (hi - lo + C - 1) / C;
    }
    int64_t inc = nch;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int64_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    WaveSeq w;
    w.c0 = inc - nch;
    w.nch = (int)nch;
    w.walk = nch > 0 && nch <= vl.max_chunks && w.c0 + nch <= vl.total_chunks;
    return w;
}

// Report bits (the KDA_REPORT_* values of kda.h) of a call of at most kWave
// sequences, from one workgroup of its first launch: a sequence skipped
// because its chunks do not fit max_chunks / total_chunks, and offsets that
// had to be clamped, ORed into the caller's word with a vector atomic.
__device__ __forceinline__ void wave_report(const Varlen &vl, const WaveSeq &w, bool leader)
{
    if (vl.status == nullptr || vl.seg_lo != 0 || !leader || threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    bool skipped = false, clamped = false;
    if (lane < vl.B) {
        const int64_t a = vl.cu[lane], b = vl.cu[lane + 1];
        skipped = !(w.nch <= vl.max_chunks && w.c0 + w.nch <= vl.total_chunks);
        clamped = a < 0 || b < a || b > vl.rows;
    }
    const int32_t bits = (__ballot(skipped) ? kReportSeqSkipped : 0) |
                         (__ballot(clamped) ? kReportRowsClamped : 0);
    if (lane == 0 && bits) atomicOr(vl.status, bits);
}

// The sequence of the prepare workgroup for global chunk g: false when no
// walked sequence owns the chunk.  leader: this workgroup reports for a call
// of at most kWave sequences.
template <int C>
__device__ __forceinline__ bool chunk_span(const Varlen &vl, int64_t g, SeqSpan &sp, bool leader)
{
    if (vl.plan == nullptr) {
        const WaveSeq w = wave_seq<C>(vl);
        wave_report(vl, w, leader);
        const uint64_t m = __ballot(w.nch > 0 && w.c0 <= g && g < w.c0 + w.nch);
        if (m == 0) return false;
        const int s = __builtin_ctzll(m);
        sp = seq_span<C>(vl, s, __shfl(w.c0, s));
        return sp.ok;
    }
    const int s = vl.plan[g];
    if (s < 0) return false;
    sp = seq_span<C>(vl, s, vl.plan[vl.total_chunks + s]);
    return sp.ok;
}

// The y-th walked sequence with chunks in [seg_lo, seg_hi): false past the
// last one.  s is its index.
template <int C>
__device__ __forceinline__ bool walker_span(const Varlen &vl, int y, int &s, SeqSpan &sp)
{
    if (vl.plan == nullptr) {
        const WaveSeq w = wave_seq<C>(vl);
        const uint64_t m = __ballot(w.walk && w.c0 < vl.seg_hi && w.c0 + w.nch > vl.seg_lo);
        if (y >= __popcll(m)) return false;
        const int lane = threadIdx.x & 63;
        const bool mine = ((m >> lane) & 1) && __popcll(m & ((uint64_t(1) << lane) - 1)) == y;
        s = __builtin_ctzll(__ballot(mine));
        sp = seq_span<C>(vl, s, __shfl(w.c0, s));
        return sp.ok;
    }
    const int32_t *rank = vl.plan + vl.total_chunks + vl.B;
    const int32_t *by_rank = rank + vl.B + 1;
    const int s_lo = vl.plan[vl.seg_lo], s_hi = vl.plan[vl.seg_hi - 1];
    if (s_lo < 0) return false;   // the segment is past the last sequence
    const int r = rank[s_lo] + y;
    if (r >= (s_hi < 0 ? rank[vl.B] : rank[s_hi + 1])) return false;
    s = by_rank[r];
    sp = seq_span<C>(vl, s, vl.plan[vl.total_chunks + s]);
    return sp.ok;
}

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

// Where the prepare kernels read q, k and v.  BF = false: fp32 arrays
// [rows, H, D] (the core entry points; ld = H * D).  BF = true: the bf16 conv
// output rows [rows, ld] holding q | k | v sections (the block prefill), read
// directly: the widening to fp32 is exact, so either source gives the same
// bits.  gate and beta are always fp32 [rows, H, D] / [rows, H].
template <bool BF>
struct QkvSrc {
    const void *q, *k, *v;
    int64_t ld;   // elements per row
    __device__ __forceinline__ float4 load4(const void *base, int64_t row, int64_t col) const {
        if constexpr (BF) {
            const uint2 u = *reinterpret_cast<const uint2 *>(
                static_cast<const uint16_t *>(base) + row * ld + col);
            return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
        } else {
            return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + row * ld + col);
        }
    }
    __device__ __forceinline__ float load1(const void *base, int64_t row, int64_t col) const {
        if constexpr (BF)
            return bf16_to_f32(static_cast<const uint16_t *>(base)[row * ld + col]);
        else
            return static_cast<const float *>(base)[row * ld + col];
    }
    __host__ __device__ __forceinline__ void advance(int64_t rows) {   // move every section down
        const int64_t e = rows * ld * (BF ? 2 : 4);
        q = static_cast<const char *>(q) + e;
        k = static_cast<const char *>(k) + e;
        v = static_cast<const char *>(v) + e;
    }
};

// This lane's A-layout slice of chunk row tg (channels 16*t8 + 4*lg .. +3 of
// head h, every tile t8) of k, q and the gate, from either source.  The loads
// are unconditional: a chunk never extends past the rows that exist, and rows
// past T are replaced afterwards by select_rows.  Keeping the loads free of
// branches and arithmetic lets them stay in flight across other work.
template <int D, bool BF>
__device__ __forceinline__ void load_rows_src(const QkvSrc<BF> &src, const float *__restrict__ gate,
                                              int64_t tg, int h, int H, int lg,
                                              float4 (&K)[D / 16], float4 (&Q)[D / 16],
                                              float4 (&G)[D / 16])
{
    const int64_t goff = (tg * H + h) * D;
    // the gate first: the in-chunk scan needs only it, so it can start while
    // k and q are still arriving
#pragma unroll
    for (int t8 = 0; t8 < D / 16; ++t8)
        G[t8] = *reinterpret_cast<const float4 *>(gate + goff + 16 * t8 + 4 * lg);
#pragma unroll
    for (int t8 = 0; t8 < D / 16; ++t8) {
        const int d0 = 16 * t8 + 4 * lg;
        K[t8] = src.load4(src.k, tg, (int64_t)h * D + d0);
        Q[t8] = src.load4(src.q, tg, (int64_t)h * D + d0);
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
// Per-chunk operand block in the workspace, for chunk n and head h at
// float offset ((n*H + h) * kSize).  All parts are fp32:
//   W   [C x D]  Tb (K e^{G})          U'  [C x D]  Tb V
//   Qg  [C x D]  Q e^{G}               Kd  [C x D]  K e^{G_C - G}
//   P   [C x C]  decayed scores (lower triangle incl. diagonal)
//   Ec  [D]      e^{G_C}
// with Tb = (I + diag(b) A)^{-1} diag(b).  Rows past T are exactly zero in
// W, U', Qg, Kd and P (their k, q, v and beta were replaced by zero).
//
// The matrices are stored in fragment order: a fragment is what one wave
// holds after one 16-byte-per-lane load (64 lanes x 4 floats), and it is
// stored as 1 KiB of consecutive memory, so every load of the forward pass
// is a fully contiguous 1 KiB read (row-strided 64-byte pieces read from L2
// at well under a third of that rate).  With lane = 16*lg + lr:
//   W, Qg  fragment (w, t8):  X[16w + lr][16t8 + 4lg + i]
//   U'     fragment (jt, w):  U'[16w + 4lg + i][16jt + lr]
//   P      fragment (w, w2):  P[16w + lr][16w2 + 4lg + i]
//   Kd     fragment (t8, w2): Kd[16w2 + 4lg + i][16t8 + lr]
// for i = 0..3, i.e. exactly the register layout of the MFMA operand or
// accumulator that consumes it.
//
// Split form (kSplit: D and C multiples of 32).  W, Qg, P and Kd are the
// left operands of the forward pass's products; there they are stored as
// bf16 pairs hi = rne(x), lo = rne(x - hi), so each product runs on the bf16
// matrix units as hi*hi + hi*lo + lo*hi with fp32 accumulation (the dropped
// lo*lo term and lo's rounding are both near 2^-16 relative).  A pair
// fragment (a, kb) covers the two fp32 fragments (a, 2kb) and (a, 2kb+1): lane
// l holds their eight values in that order, as bf16x8 hi at float offset
// 4l and lo at 256 + 4l of the 2 KiB pair fragment.  For the 16x16x32 bf16
// MFMA this is a fixed permutation of the 32-deep contraction index, and the
// right operand (the state S, the corrected writes U) is split the same way
// from the same two fp32 fragments, so the products are unchanged.  The block
// layout and size are those of the fp32 form; U' and Ec stay fp32.
// ---------------------------------------------------------------------------
template <int D, int C>
struct Blk {
    static constexpr int NW = C / 16, DT = D / 16;
    static constexpr int kW = 0, kU = C * D, kQ = 2 * C * D, kKd = 3 * C * D;
    static constexpr int kP = 4 * C * D, kEc = 4 * C * D + C * C;
    static constexpr int kSize = 4 * C * D + C * C + D;
    static constexpr bool kSplit = (D % 32 == 0) && (C % 32 == 0);
    // float offset of fragment (a, b) of a part with nb fragments per a
    static __device__ __forceinline__ int frag(int a, int b, int nb) { return (a * nb + b) * 256; }
    // float offset of pair fragment (a, kb) of a part with nkb pairs per a
    static __device__ __forceinline__ int pfrag(int a, int kb, int nkb) { return (a * nkb + kb) * 512; }
};

// Store this lane's share of a pair fragment: fp32 fragments x0, x1 split
// into bf16 hi / lo halves (see Blk).
__device__ __forceinline__ void store_pair(float *dst, int lane, const float4 &x0, const float4 &x1)
{
    bf16x8 hi, lo;
    split8(x0, x1, hi, lo);
    *reinterpret_cast<bf16x8 *>(dst + 4 * lane) = hi;
    *reinterpret_cast<bf16x8 *>(dst + 256 + 4 * lane) = lo;
}
__device__ __forceinline__ float4 f4(const floatx4 &a) { return make_float4(a[0], a[1], a[2], a[3]); }

// T = (I + M)^{-1} for the strictly lower C x C matrix M in s_M, into the
// lower block triangle of s_T (blocks above the diagonal are not written).
// Diagonal 16x16 blocks by forward substitution (wave w solves block w, lane
// lr column lr), then block levels T_ij = -T_ii sum_{m=j}^{i-1} M_im T_mj on
// fp32 MFMA, one level per barrier.  Ends with a barrier.
template <int C>
__device__ __forceinline__ void invert_unit_lower(const float (*__restrict__ s_M)[C + kPadC],
                                                  float (*__restrict__ s_T)[C + kPadC], int w,
                                                  int lane)
{
    constexpr int NW = C / 16;
    const int lr = lane & 15, lg = lane >> 4;
    {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; s4 < r; s4 += 4) {
                const float4 m = *reinterpret_cast<const float4 *>(&s_M[16 * w + r][16 * w + s4]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (s4 + i < r) acc = __builtin_fmaf(-get4(m, i), x[s4 + i], acc);
            }
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
}

// ---------------------------------------------------------------------------
// kda_chunk_prep: one workgroup per (chunk n, head h), all chunks in parallel;
// fp32 fragments and fp32 MFMA, for the shapes without a split form.
// ---------------------------------------------------------------------------
template <int D, int C, bool BF>
__global__ __launch_bounds__(C / 16 * 64) void kda_chunk_prep_kernel(
    QkvSrc<BF> src, const float *__restrict__ gate, const float *__restrict__ beta, int T, int H,
    float *__restrict__ ws, const Varlen vl)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    using B = Blk<D, C>;
    // several sequences: x is the chunk of the segment
    int n = blockIdx.x;
    const int h = blockIdx.y;
    int64_t nblk = n, tmax = (int64_t)1 << 62;   // operand block index; last row that exists
    if (vl.cu) {
        SeqSpan sp;
        if (!chunk_span<C>(vl, vl.seg_lo + nblk, sp, blockIdx.x == 0 && blockIdx.y == 0))
            return;   // uniform over the workgroup
        n = (int)(vl.seg_lo + nblk - sp.chunk0);
        const int64_t r0 = sp.row0 * H;
        src.advance(sp.row0);
        gate += r0 * D, beta += r0;
        T = sp.T;
        tmax = vl.rows - 1 - sp.row0;
    }
    // wave index, uniform across the wave (scalar register)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int rl = 16 * w + lr;
    const int64_t tg = min((int64_t)n * C + rl, tmax);   // rows past T are replaced
    const bool valid = (int64_t)n * C + rl < T;
    float *__restrict__ blk = ws + (nblk * H + h) * B::kSize;

    __shared__ __align__(16) float s_tot[NW * D];
    __shared__ __align__(16) float s_kc[C][D + kPadK];   // Kc, then Kg, then V
    __shared__ __align__(16) float s_M[C][C + kPadC];
    __shared__ __align__(16) float s_T[C][C + kPadC];
    __shared__ __align__(16) float s_beta[C];

    // Register lifetimes are kept short so two workgroups fit on a CU: Q e^G,
    // e^{G_C} and Kd = K e^{G_C - G} are formed right after the scan, K e^G
    // goes to LDS right after the A/P products, v is loaded only for U'.
    float4 K[DT], Q[DT], G[DT], Kd[DT];
    load_rows_src<D, BF>(src, gate, tg, h, H, lg, K, Q, G);
    const float braw = beta[tg * H + h];
    select_rows<D>(valid, K, Q, G);
    if (lg == 0) s_beta[rl] = valid ? braw : 0.f;
    {
        float4 Gend[DT];
        chunk_cumsum<D, NW>(G, Gend, s_tot, w, lane);
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            *reinterpret_cast<float4 *>(blk + B::kQ + B::frag(w, t8, DT) + 4 * lane) =
                mul4(Q[t8], exp2_4(G[t8]));
            Kd[t8] = mul4(K[t8], exp2_4(sub4(Gend[t8], G[t8])));
            if (w == 0 && lr == 0)
                *reinterpret_cast<float4 *>(blk + B::kEc + 16 * t8 + 4 * lg) = exp2_4(Gend[t8]);
        }
    }

    // Column operand Kc = K e^{G_last - G}, relative to the last row of this
    // wave's 16-row block (all factors <= 1); also the block's decay span.
    float span = 0.f;
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) {
        const float4 Gl = shfl4(G[t8], (lane & 48) | 15);
        const float4 Gf = shfl4(G[t8], lane & 48);
        const float4 e = exp2_4(sub4(Gl, G[t8]));
        *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = mul4(K[t8], e);
        span = fmaxf(span, fmaxf(fmaxf(Gf.x - Gl.x, Gf.y - Gl.y), fmaxf(Gf.z - Gl.z, Gf.w - Gl.w)));
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
            float4 ref = zero4();
            if (bj == w) {
                ref = shfl4(G[t8], (lane & 48) | 15);
            } else {
                ref = zero4();
#pragma unroll
                for (int ww = 0; ww <= bj; ++ww)
                    ref = add4(ref, *reinterpret_cast<const float4 *>(s_tot + ww * D + 16 * t8 + 4 * lg));
            }
            const float4 e = exp2_4(sub4(G[t8], ref));
            const float4 kr = mul4(K[t8], e), qr = mul4(Q[t8], e);
            const float4 kc = *reinterpret_cast<const float4 *>(&s_kc[16 * bj + lr][16 * t8 + 4 * lg]);
            // A tile (rows r) and P tile transposed (rows s): the swapped
            // operand order leaves P^T in the fragment order of P
            Aacc[bj] = mfma4(kr.x, kc.x, Aacc[bj]);
            Pacc[bj] = mfma4(kc.x, qr.x, Pacc[bj]);
            Aacc[bj] = mfma4(kr.y, kc.y, Aacc[bj]);
            Pacc[bj] = mfma4(kc.y, qr.y, Pacc[bj]);
            Aacc[bj] = mfma4(kr.z, kc.z, Aacc[bj]);
            Pacc[bj] = mfma4(kc.z, qr.z, Pacc[bj]);
            Aacc[bj] = mfma4(kr.w, kc.w, Aacc[bj]);
            Pacc[bj] = mfma4(kc.w, qr.w, Pacc[bj]);
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
            // sum_d x_r[d] k_s[d] e^{G_r[d] - G_s[d]} for one (r, s) of this
            // block, with x = k (A) or q (P); rows past T contribute zero
            auto pair = [&](int r, int sc, const void *x) {
                float acc = 0.f;
                const int64_t tr = (int64_t)n * C + r, ts = (int64_t)n * C + sc;
                if (sc <= r && tr < T && ts < T) {
                    const int64_t c0 = (int64_t)h * D;
                    for (int d = 0; d < D; ++d)
                        acc = __builtin_fmaf(src.load1(x, tr, c0 + d),
                                             src.load1(src.k, ts, c0 + d) *
                                                 exp2_fast(s_kc[r][d] - s_kc[sc][d]),
                                             acc);
                }
                return acc;
            };
            float da[4], dp[4];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                da[vv] = pair(16 * w + 4 * lg + vv, 16 * w + lr, src.k);   // A tile layout
                dp[vv] = pair(16 * w + lr, 16 * w + 4 * lg + vv, src.q);   // P^T tile layout
            }
#pragma unroll
            for (int bj = 0; bj < NW; ++bj)
                if (bj == w) Aacc[bj] = floatx4{da[0], da[1], da[2], da[3]},
                             Pacc[bj] = floatx4{dp[0], dp[1], dp[2], dp[3]};
        }
    }

    // Masked tiles: M = diag(b) A (strictly lower) to LDS; P to the workspace
    // as fragments (w, bj), the blocks above the diagonal as zeros so the
    // forward pass can run the whole block row without branching.
    float *Pf = blk + B::kP;
    float4 pv[NW];
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) {
        pv[bj] = zero4();
        if (bj <= w) {
            float pe[4];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int r = 16 * w + 4 * lg + vv, sc = 16 * bj + lr;
                float a = Aacc[bj][vv];
                if (bj == w && sc >= r) a = 0.f;
                s_M[r][sc] = s_beta[r] * a;
                // P^T element: s = 16bj + 4lg + vv, r = 16w + lr
                pe[vv] = (bj == w && 4 * lg + vv > lr) ? 0.f : Pacc[bj][vv];
            }
            pv[bj] = make_float4(pe[0], pe[1], pe[2], pe[3]);
        }
        *reinterpret_cast<float4 *>(Pf + B::frag(w, bj, NW) + 4 * lane) = pv[bj];
    }
    __syncthreads();
    // Kg = K e^G into LDS as the left operand of W^T = Kg^T Tb^T (the fallback
    // is done with s_kc; the inversion's barriers order this before its use)
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8)
        *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = mul4(K[t8], exp2_4(G[t8]));

    invert_unit_lower<C>(s_M, s_T, w, lane);

    // W = Tb Kg, then U' = Tb V, then the Kd fragments: wave w owns channel
    // tiles t8 = w (mod NW), all row blocks (balanced across waves).
    // Tb = T diag(b) is formed on the fly from s_T and s_beta.  W is computed
    // transposed (operands swapped), which leaves each output tile in W's
    // fragment order; U' in its natural orientation is already in U''s.
    constexpr int TG = 1;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int g = 0; g < DT / TG; ++g) {
            if (g % NW != w) continue;
#pragma unroll
            for (int bi = 0; bi < NW; ++bi) {
                floatx4 acc[TG];
#pragma unroll
                for (int u = 0; u < TG; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w2 = 0; w2 <= bi; ++w2) {
                    const float4 ta = mul4(
                        *reinterpret_cast<const float4 *>(&s_T[16 * bi + lr][16 * w2 + 4 * lg]),
                        *reinterpret_cast<const float4 *>(&s_beta[16 * w2 + 4 * lg]));
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                        for (int u = 0; u < TG; ++u) {
                            const float x = s_kc[16 * w2 + 4 * lg + kk][16 * (TG * g + u) + lr];
                            acc[u] = pass == 0 ? mfma4(x, get4(ta, kk), acc[u])
                                               : mfma4(get4(ta, kk), x, acc[u]);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < TG; ++u) {
                    float *dst = pass == 0 ? blk + B::kW + B::frag(bi, TG * g + u, DT)
                                           : blk + B::kU + B::frag(TG * g + u, bi, NW);
                    *reinterpret_cast<float4 *>(dst + 4 * lane) = f4(acc[u]);
                }
            }
        }
        __syncthreads();
        if (pass == 0) {   // next right operand: V
#pragma unroll
            for (int t8 = 0; t8 < DT; ++t8) {
                const float4 vv = src.load4(src.v, tg, (int64_t)h * D + 16 * t8 + 4 * lg);
                *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = valid ? vv : zero4();
            }
        } else {           // then Kd, to be transposed into its fragments
#pragma unroll
            for (int t8 = 0; t8 < DT; ++t8)
                *reinterpret_cast<float4 *>(&s_kc[rl][16 * t8 + 4 * lg]) = Kd[t8];
        }
        __syncthreads();
    }
    // Kd fragments (t8, w2): a transpose of the 16 x 16 tiles through LDS
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) {
        if ((t8 / TG) % NW != w) continue;
        float4 kv[NW];
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            kv[w2] = make_float4(s_kc[16 * w2 + 4 * lg + 0][16 * t8 + lr],
                                 s_kc[16 * w2 + 4 * lg + 1][16 * t8 + lr],
                                 s_kc[16 * w2 + 4 * lg + 2][16 * t8 + lr],
                                 s_kc[16 * w2 + 4 * lg + 3][16 * t8 + lr]);
            *reinterpret_cast<float4 *>(blk + B::kKd + B::frag(t8, w2, NW) + 4 * lane) = kv[w2];
        }
    }
}

// ---------------------------------------------------------------------------
// kda_chunk_prep_split: the split form of kda_chunk_prep (D, C multiples of
// 32), one workgroup per (chunk n, head h).  Every product runs on the
// 16x16x32 bf16 MFMA as hi*hi + hi*lo + lo*hi (fp32 accumulation); operands
// are in the pair order of Blk, so a lane's eight values of a 32-deep block
// are its elements of fp32 tiles 2kb and 2kb+1.
//
// Decay references.  With R_b the cumulative log-decay at the end of 16-row
// block b (R_{-1} = 0) and G_r the cumulative log-decay of row r (both per
// channel), a row r of block w and a row s of block bj <= w give
//   e^{G_r - G_s} = e^{G_r - R_{w-1}} * e^{R_{w-1} - R_{bj-1}} * e^{R_{bj-1} - G_s}
// with the first two factors <= 1 and the third >= 1 but bounded by block
// bj's own decay span (for a decay gate, G <= 0 per token).  So the row operands are K e^{G - R_{w-1}} and
// Q e^{G - R_{w-1}} (one exponential per element, formed once), the column
// operand of block bj is K e^{R_{bj-1} - G} (once per row), and the middle
// factor is a per-channel table entry applied to the column operand of an
// off-diagonal tile.  Q e^G, K e^G and Kd follow from the same two
// exponentials and per-channel tables.  A block whose span exceeds
// kBlockSpanLog2 (a decay beyond e^{-66} within 16 tokens), or any growing
// (positive) log-gate, would push a factor out of range: such a chunk takes
// the exact pairwise sum for every entry of A and P instead (slow, correct
// for any gate).
// ---------------------------------------------------------------------------
constexpr float kBlockSpanLog2 = 96.0f;

// LDS of one prepare unit (one chunk of one head) in the split form.
template <int D, int C>
struct __align__(16) PrepSplitLds {
    static constexpr int NW = C / 16;
    // s_xbuf, fp32: first Kd^T, then the column operand K e^{R_{w-1} - G} as
    // rows (or, on the pairwise path, the cumulative log-decay rows), then
    // the right operands of the W and U' passes transposed: (K e^G)^T, V^T.
    // A transposed operand is read as two 16-byte pieces per lane.
    static constexpr int kXRow = C * (D + kPadK), kXCol = D * (C + kPadC);
    float s_tot[NW * D];
    float s_beta[C];
    float s_xbuf[kXRow > kXCol ? kXRow : kXCol];
    float s_M[C][C + kPadC];
    float s_T[C][C + kPadC];
    float s_tab[2 * NW + NW * (NW - 1) / 2 + 1][D];
    int s_bad[NW];
};

// One prepare unit: chunk n of head h into its operand block `blk`, by the
// C/16 waves whose unit-local thread indices are tid = 0 .. 64*C/16 - 1.
// Rows past T are replaced (tmax: the last row that exists).  Every thread
// of the workgroup passes the same barriers whatever its unit does, so a
// workgroup may run several units side by side.  W_LDS: W and U' go to the
// unit's own LDS instead of the block, in the block's layouts (C*D floats
// each: W from the start of L.s_M running on into L.s_T, U' from the start
// of L.s_xbuf), for a walk by the same workgroup right after; they are
// there once the unit's caller has passed a barrier.
template <int D, int C, bool BF, bool W_LDS = false>
__device__ __forceinline__ void prep_split_unit(const QkvSrc<BF> &src, const float *__restrict__ gate,
                                                const float *__restrict__ beta, int T, int H,
                                                float *__restrict__ blk, int n, int h,
                                                int64_t tmax, int tid, PrepSplitLds<D, C> &L)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    constexpr int KD = DT / 2, KC = NW / 2;   // 32-deep blocks over D and over C
    using B = Blk<D, C>;
    static_assert(B::kSplit, "split operand blocks need D, C multiples of 32");
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int rl = 16 * w + lr;
    const int64_t tg = min((int64_t)n * C + rl, tmax);   // rows past T are replaced
    const bool valid = (int64_t)n * C + rl < T;

    float *__restrict__ s_tot = L.s_tot;
    float *__restrict__ s_beta = L.s_beta;
    auto s_x = reinterpret_cast<float (*)[D + kPadK]>(L.s_xbuf);    // rows [C][D]
    auto s_xT = reinterpret_cast<float (*)[C + kPadC]>(L.s_xbuf);   // transposed [D][C]
    auto &s_M = L.s_M;
    auto &s_T = L.s_T;
    auto &s_tab = L.s_tab;

    float4 K[DT], Q[DT], G[DT];
    load_rows_src<D, BF>(src, gate, tg, h, H, lg, K, Q, G);
    const float braw = beta[tg * H + h];
    if ((int64_t)(n + 1) * C <= T) {   // a whole chunk (uniform): no row to replace
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8)
            G[t8] = make_float4(G[t8].x * kLog2e, G[t8].y * kLog2e, G[t8].z * kLog2e, G[t8].w * kLog2e);
    } else {
        select_rows<D>(valid, K, Q, G);
    }
    if (lg == 0) s_beta[rl] = valid ? braw : 0.f;
    // G: inclusive cumulative log-decay within this wave's block (relative
    // to R_{w-1}); the block totals go to s_tot
    scan_local<D, NW>(G, s_tot, w, lane);
    __syncthreads();
    // Per-channel tables from the block totals, and the span check.  Rows:
    //   w            e^{R_{w-1}}                (Q e^G, K e^G from the row operands)
    //   NW + w       e^{R_{NW-1} - R_{w-1}}     (Kd from the column operand)
    //   2NW + w(w-1)/2 + bj   e^{R_{w-1} - R_{bj-1}}, bj < w   (off-diagonal tiles)
    //   kRowEc       e^{R_{NW-1}} = e^{G_C}     (also stored as Ec)
    constexpr int kRowF = 2 * NW, kRowEc = 2 * NW + NW * (NW - 1) / 2, kRows = kRowEc + 1;
    {
        // a thread takes one channel d and every kParts-th row (kParts threads
        // share a channel when the workgroup has more threads than channels)
        constexpr int NT = NW * kWave, kParts = NT >= D ? NT / D : 1;
        const int part = NT >= D ? tid / D : 0;
        for (int d = NT >= D ? tid % D : tid; d < D; d += NT >= D ? D : NT) {
            float R[NW + 1];   // R[b + 1] = R_b
            R[0] = 0.f;
#pragma unroll
            for (int b = 0; b < NW; ++b) R[b + 1] = R[b] + s_tot[b * D + d];
#pragma unroll
            for (int row = 0; row < kRows; ++row) {
                if (row % kParts != part) continue;
                float x;
                if (row < NW) {
                    x = R[row];
                } else if (row < kRowF) {
                    x = R[NW] - R[row - NW];
                } else if (row < kRowEc) {
                    int ww = 1, r0 = row - kRowF;   // row = kRowF + ww(ww-1)/2 + r0, r0 < ww
                    while (r0 >= ww) r0 -= ww++;
                    x = R[ww] - R[r0];
                } else {
                    x = R[NW];
                }
                const float ex = exp2_fast(x);
                s_tab[row][d] = ex;
                if (row == kRowEc) blk[B::kEc + d] = ex;
            }
        }
    }
    bool bad = false;
    // every factor stays in range when each in-block cumulative log-decay lies
    // in [-kBlockSpanLog2, 0] (always true of a decay gate whose blocks span
    // less than the limit)
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) {
        const float4 g = G[t8];
        bad |= fminf(fminf(g.x, g.y), fminf(g.z, g.w)) < -kBlockSpanLog2 ||
               fmaxf(fmaxf(g.x, g.y), fmaxf(g.z, g.w)) > 0.f;
    }
    // the unit's waves OR their flags through LDS (a workgroup may hold
    // several units; each decides for its own chunk)
    bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) L.s_bad[w] = bad ? 1 : 0;
    __syncthreads();
    bool wide = false;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) wide |= L.s_bad[ww] != 0;
    auto tab4 = [&](int row, int c) { return *reinterpret_cast<const float4 *>(&s_tab[row][c]); };

    // Row operands B = K e^{G - R_{w-1}}, Qb = Q e^{G - R_{w-1}} (split), the
    // column operand Kc = K e^{R_{w-1} - G} (fp32 rows, later), and from them
    // Q e^G (stored), K e^G (fp32, the right operand of W) and
    // Kd = K e^{G_C - G} (rows, transposed into its pair fragments through
    // s_x first)
    auto x_operand = [&](int t8, int kb2, bf16x8 &xh, bf16x8 &xl) {
        // this lane's X[s(kb2, lg, j)][16t8 + lr] from X^T in s_xT
        const int s0 = 32 * kb2 + 4 * lg, c = 16 * t8 + lr;
        split8(*reinterpret_cast<const float4 *>(&s_xT[c][s0]),
               *reinterpret_cast<const float4 *>(&s_xT[c][s0 + 16]), xh, xl);
    };
    auto put_T = [&](int t8, const float4 &x) {   // this lane's row piece into X^T
        const int c = 16 * t8 + 4 * lg;
        s_xT[c + 0][rl] = x.x;
        s_xT[c + 1][rl] = x.y;
        s_xT[c + 2][rl] = x.z;
        s_xT[c + 3][rl] = x.w;
    };
    bf16x8 Bh[KD], Bl[KD], Qh[KD], Ql[KD];
    float4 Kc[DT], Kg[DT];
#pragma unroll
    for (int kb = 0; kb < KD; ++kb) {
        float4 b2[2], qb2[2], qg[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t8 = 2 * kb + u, c = 16 * t8 + 4 * lg;
            const float4 e = exp2_4(G[t8]);
            const float4 ei = exp2_4(make_float4(-G[t8].x, -G[t8].y, -G[t8].z, -G[t8].w));
            b2[u] = mul4(K[t8], e);
            qb2[u] = mul4(Q[t8], e);
            Kc[t8] = mul4(K[t8], ei);
            const float4 pw = tab4(w, c);
            qg[u] = mul4(qb2[u], pw);
            Kg[t8] = mul4(b2[u], pw);
            if (!wide) {
                put_T(t8, mul4(Kc[t8], tab4(NW + w, c)));   // Kd = K e^{R_{w-1} - G} e^{G_C - R_{w-1}}
            } else {
                // e^{-G} may overflow here: Kd = K e^{(G_C - R_{w-1}) - G}, exponent <= 0
                float4 x = zero4();
#pragma unroll
                for (int b = 0; b < NW; ++b)
                    if (b >= w) x = add4(x, *reinterpret_cast<const float4 *>(&s_tot[b * D + c]));
                put_T(t8, mul4(K[t8], exp2_4(sub4(x, G[t8]))));
            }
        }
        split8(b2[0], b2[1], Bh[kb], Bl[kb]);
        split8(qb2[0], qb2[1], Qh[kb], Ql[kb]);
        store_pair(blk + B::kQ + B::pfrag(w, kb, KD), lane, qg[0], qg[1]);
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < KD; ++g) {
        if (g % NW != w) continue;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kb2 = 0; kb2 < KC; ++kb2) {
                bf16x8 xh, xl;
                x_operand(2 * g + u, kb2, xh, xl);
                float *dst = blk + B::kKd + B::pfrag(2 * g + u, kb2, KC);
                *reinterpret_cast<bf16x8 *>(dst + 4 * lane) = xh;
                *reinterpret_cast<bf16x8 *>(dst + 256 + 4 * lane) = xl;
            }
    }
    __syncthreads();
    if (!wide) {
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) *reinterpret_cast<float4 *>(&s_x[rl][16 * t8 + 4 * lg]) = Kc[t8];
    } else {   // the chunk-relative cumulative log-decay rows, for the pairwise sums
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            float4 g = G[t8];
#pragma unroll
            for (int b = 0; b < NW; ++b)
                if (b < w) g = add4(g, *reinterpret_cast<const float4 *>(&s_tot[b * D + 16 * t8 + 4 * lg]));
            *reinterpret_cast<float4 *>(&s_x[rl][16 * t8 + 4 * lg]) = g;
        }
    }
    __syncthreads();

    // Block row w of A (tile layout: element i is A[16w + 4lg + i][16bj + lr])
    // and of P (fragment layout: element i is P[16w + lr][16bj + 4lg + i]).
    floatx4 Aacc[NW], Pacc[NW];
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) Aacc[bj] = Pacc[bj] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (!wide) {
#pragma unroll
        for (int bj = 0; bj < NW; ++bj) {
            if (bj > w) continue;
            const int frow = kRowF + w * (w - 1) / 2 + bj;   // used only when bj < w
#pragma unroll
            for (int kb = 0; kb < KD; ++kb) {
                // column operand: block bj's K e^{R_{bj-1} - G}, times e^{R_{w-1} - R_{bj-1}}
                const int c0 = 32 * kb + 4 * lg;
                float4 x0 = *reinterpret_cast<const float4 *>(&s_x[16 * bj + lr][c0]);
                float4 x1 = *reinterpret_cast<const float4 *>(&s_x[16 * bj + lr][c0 + 16]);
                if (bj < w) {
                    x0 = mul4(x0, tab4(frow, c0));
                    x1 = mul4(x1, tab4(frow, c0 + 16));
                }
                bf16x8 ch, cl;
                split8(x0, x1, ch, cl);
                Aacc[bj] = mfma_bf16(Bh[kb], ch, Aacc[bj]);
                Pacc[bj] = mfma_bf16(ch, Qh[kb], Pacc[bj]);
                Aacc[bj] = mfma_bf16(Bh[kb], cl, Aacc[bj]);
                Pacc[bj] = mfma_bf16(ch, Ql[kb], Pacc[bj]);
                Aacc[bj] = mfma_bf16(Bl[kb], ch, Aacc[bj]);
                Pacc[bj] = mfma_bf16(cl, Qh[kb], Pacc[bj]);
            }
        }
    } else {
        // sum_d x_r[d] k_s[d] e^{G_r[d] - G_s[d]} for one (r, s) of the chunk,
        // x = k (A) or q (P); rows past T contribute zero
        auto pair = [&](int r, int sc, const void *x) {
            float acc = 0.f;
            const int64_t tr = (int64_t)n * C + r, ts = (int64_t)n * C + sc;
            if (sc <= r && tr < T && ts < T) {
                const int64_t c0 = (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    acc = __builtin_fmaf(src.load1(x, tr, c0 + d),
                                         src.load1(src.k, ts, c0 + d) *
                                             exp2_fast(s_x[r][d] - s_x[sc][d]),
                                         acc);
            }
            return acc;
        };
#pragma unroll
        for (int bj = 0; bj < NW; ++bj) {
            if (bj > w) continue;
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                Aacc[bj][vv] = pair(16 * w + 4 * lg + vv, 16 * bj + lr, src.k);
                Pacc[bj][vv] = pair(16 * w + lr, 16 * bj + 4 * lg + vv, src.q);
            }
        }
    }

    // M = diag(b) A, strictly lower, to LDS; P as pair fragments (blocks above
    // the diagonal as zeros; a 32-column fragment wholly above the diagonal,
    // 32 kb > 16 w + 15, is neither stored nor read)
    float4 pv[NW];
#pragma unroll
    for (int bj = 0; bj < NW; ++bj) {
        pv[bj] = zero4();
        if (bj <= w) {
            float pe[4];
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int r = 16 * w + 4 * lg + vv, sc = 16 * bj + lr;
                float a = Aacc[bj][vv];
                if (bj == w && sc >= r) a = 0.f;
                s_M[r][sc] = s_beta[r] * a;
                pe[vv] = (bj == w && 4 * lg + vv > lr) ? 0.f : Pacc[bj][vv];
            }
            pv[bj] = make_float4(pe[0], pe[1], pe[2], pe[3]);
        }
        if (bj % 2 == 1 && bj - 1 <= w)
            store_pair(blk + B::kP + B::pfrag(w, bj / 2, KC), lane, pv[bj - 1], pv[bj]);
    }
    __syncthreads();   // s_M complete; s_x free
    // V now, for the U' pass (its latency hidden behind the inversion and W)
    float4 Vr[DT];
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) Vr[t8] = src.load4(src.v, tg, (int64_t)h * D + 16 * t8 + 4 * lg);
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8) put_T(t8, Kg[t8]);   // (K e^G)^T, right operand of W

    invert_unit_lower<C>(s_M, s_T, w, lane);   // ends with a barrier: s_T and s_x visible

    // W = Tb Kg, then U' = Tb V (Tb = T diag(b)).  Wave
    // w owns the channel-tile pairs g = w (mod NW).  The Tb operand of row
    // block bi over rows 32kb2.. is read from s_T rows (zero where the 16-row
    // block lies above the diagonal, which s_T does not hold); the right
    // operand X (K e^G, then V) is gathered from the s_x rows, transposed.
    auto tb_operand = [&](int bi, int kb2, bf16x8 &th, bf16x8 &tl) {
        const int s0 = 32 * kb2 + 4 * lg;
        const float4 t0 = mul4(*reinterpret_cast<const float4 *>(&s_T[16 * bi + lr][s0]),
                               *reinterpret_cast<const float4 *>(&s_beta[s0]));
        const float4 t1 = (2 * kb2 + 1 <= bi)
                              ? mul4(*reinterpret_cast<const float4 *>(&s_T[16 * bi + lr][s0 + 16]),
                                     *reinterpret_cast<const float4 *>(&s_beta[s0 + 16]))
                              : zero4();
        split8(t0, t1, th, tl);
    };
    // the Tb operands, shared by both passes
    bf16x8 tbh[NW][KC], tbl[NW][KC];
#pragma unroll
    for (int bi = 0; bi < NW; ++bi)
#pragma unroll
        for (int kb2 = 0; kb2 <= bi / 2; ++kb2) tb_operand(bi, kb2, tbh[bi][kb2], tbl[bi][kb2]);
    [[maybe_unused]] float4 up_keep[W_LDS ? NW : 1][2];
    if constexpr (W_LDS) {
        static_assert(C * D <= 2 * C * (C + kPadC) && C * D <= PrepSplitLds<D, C>::kXRow &&
                          KD == NW, "W and U' fit in LDS; one channel-tile pair per wave");
        __syncthreads();   // every read of s_T done before W overwrites it
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int g = 0; g < KD; ++g) {
            if (g % NW != w) continue;
            bf16x8 xh[2][KC], xl[2][KC];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int kb2 = 0; kb2 < KC; ++kb2) x_operand(2 * g + u, kb2, xh[u][kb2], xl[u][kb2]);
#pragma unroll
            for (int bi = 0; bi < NW; ++bi) {
                floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int kb2 = 0; kb2 <= bi / 2; ++kb2) {
                    const bf16x8 th = tbh[bi][kb2], tl = tbl[bi][kb2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if (pass == 0) {   // W^T tile (t8, bi) = X^T Tb^T: W's fragment order
                            acc[u] = mfma_bf16(xh[u][kb2], th, acc[u]);
                            acc[u] = mfma_bf16(xh[u][kb2], tl, acc[u]);
                            acc[u] = mfma_bf16(xl[u][kb2], th, acc[u]);
                        } else {           // U' tile = Tb X: U''s fragment order
                            acc[u] = mfma_bf16(th, xh[u][kb2], acc[u]);
                            acc[u] = mfma_bf16(th, xl[u][kb2], acc[u]);
                            acc[u] = mfma_bf16(tl, xh[u][kb2], acc[u]);
                        }
                    }
                }
                if (pass == 0) {
                    if constexpr (W_LDS)
                        store_pair(&L.s_M[0][0] + B::pfrag(bi, g, KD), lane, f4(acc[0]), f4(acc[1]));
                    else
                        store_pair(blk + B::kW + B::pfrag(bi, g, KD), lane, f4(acc[0]), f4(acc[1]));
                } else {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if constexpr (W_LDS)
                            up_keep[bi][u] = f4(acc[u]);
                        else
                            *reinterpret_cast<float4 *>(blk + B::kU + B::frag(2 * g + u, bi, NW) + 4 * lane) = f4(acc[u]);
                    }
                }
            }
        }
        if (pass == 0) {
            __syncthreads();
#pragma unroll
            for (int t8 = 0; t8 < DT; ++t8)
                put_T(t8, valid ? Vr[t8] : zero4());
            __syncthreads();
        }
    }
    if constexpr (W_LDS) {
        __syncthreads();   // every read of V^T in s_xbuf done before U' overwrites it
#pragma unroll
        for (int bi = 0; bi < NW; ++bi)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                *reinterpret_cast<float4 *>(L.s_xbuf + B::frag(2 * w + u, bi, NW) + 4 * lane) = up_keep[bi][u];
    }
}


template <int D, int C, bool BF>
__global__ __launch_bounds__(C / 16 * 64) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_prep_split_kernel(
    QkvSrc<BF> src, const float *__restrict__ gate, const float *__restrict__ beta, int T, int H,
    float *__restrict__ ws, const Varlen vl)
{
    using B = Blk<D, C>;
    // heads fastest in the grid (a round of resident workgroups reads whole
    // token rows and writes adjacent operand blocks): heads in x, chunks in
    // y (for several sequences, the chunks of the segment)
    int n = (int)blockIdx.y;
    const int h = (int)blockIdx.x;
    int64_t nblk = n, tmax = (int64_t)1 << 62;   // operand block index; last row that exists
    if (vl.cu) {
        SeqSpan sp;
        if (!chunk_span<C>(vl, vl.seg_lo + nblk, sp, blockIdx.x == 0 && blockIdx.y == 0))
            return;   // uniform over the workgroup
        n = (int)(vl.seg_lo + nblk - sp.chunk0);
        const int64_t r0 = sp.row0 * H;
        src.advance(sp.row0);
        gate += r0 * D, beta += r0;
        T = sp.T;
        tmax = vl.rows - 1 - sp.row0;
    }
    __shared__ PrepSplitLds<D, C> L;
    prep_split_unit<D, C, BF>(src, gate, beta, T, H, ws + (nblk * H + h) * B::kSize, n, h, tmax,
                              (int)threadIdx.x, L);
}

// ---------------------------------------------------------------------------
// kda_chunk_fwd: per (head h, value slice j0..j0+15), serial over chunks.
// Wave w owns chunk rows 16w..16w+15; the state slice S[:, j0..j0+15] lives
// in registers of every wave in MFMA output layout.  Per chunk:
//   U  = U' - W S            (D-deep, this wave's rows)
//   QS = Qg S                (D-deep)
//   -- B1: U rows visible --
//   O  = scale (QS + P U)    (lower block triangle)
//   S' = Ec * S + KdT U      (C-deep, channel tiles t8 = w mod NW)
//   -- B2: new state slice visible --
// Every operand arrives pre-laid-out from kda_chunk_prep.  Loads of chunk
// n+1's operands are issued as soon as chunk n's copy of that operand has
// been consumed (rolling prefetch), so they overlap the rest of the chunk.
// ---------------------------------------------------------------------------
template <int D, int C>
__global__ __launch_bounds__(C / 16 * 64) void kda_chunk_fwd_kernel(
    const float *__restrict__ ws, float *__restrict__ state, float *__restrict__ core, int T,
    int NC, int H, float scale, const Varlen vl)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    constexpr int OWN = (DT + NW - 1) / NW;   // channel tiles per wave in the state update
    using B = Blk<D, C>;
    // all value slices of one head share an XCD (workgroups are dealt to the
    // 8 XCDs round-robin), so they share that XCD's L2 copy of the operands
    const int h = blockIdx.x % H, jt = blockIdx.x / H, j0 = 16 * jt;
    if (vl.cu) {   // the blockIdx.y-th sequence of the segment: its state and chunks here
        int s;
        SeqSpan sp;
        if (!walker_span<C>(vl, blockIdx.y, s, sp)) return;   // uniform over the workgroup
        const int64_t g0 = max(sp.chunk0, (int64_t)vl.seg_lo);
        const int64_t g1 = min(sp.chunk0 + sp.nch, (int64_t)vl.seg_hi);
        if (g0 >= g1) return;
        const int c0 = (int)(g0 - sp.chunk0);   // first chunk of the sequence walked here
        state = vl.states[s];
        core += (sp.row0 + (int64_t)c0 * C) * H * D;
        ws += (g0 - vl.seg_lo) * H * B::kSize;
        NC = (int)(g1 - g0);
        T = min(sp.T - c0 * C, NC * C);
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;

    __shared__ float s_u[C][16 + kPad16];
    __shared__ float s_S[D][16 + kPad16];

    // S slice in MFMA output layout: Sr[t8][i] = S[16*t8 + 4*lg + i][j0 + lr]
    // (through a global-space pointer, as in walk_split)
    typedef __attribute__((address_space(1))) float gfloat;
    gfloat *__restrict__ Sg = (gfloat *)(state + (int64_t)h * D * D);
    floatx4 Sr[DT];
#pragma unroll
    for (int t8 = 0; t8 < DT; ++t8)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sr[t8][i] = Sg[(int64_t)(16 * t8 + 4 * lg + i) * D + j0 + lr];

    // the state tiles this wave updates (t8 = w + NW*o; a wave with no tile
    // of its own, possible only when D/16 < C/16, repeats the last tile and
    // writes the same values as its owner)
    auto own_tile = [&](int o) { return min(w + NW * o, DT - 1); };
    floatx4 Sown[OWN];
#pragma unroll
    for (int o = 0; o < OWN; ++o)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Sown[o][i] = Sg[(int64_t)(16 * own_tile(o) + 4 * lg + i) * D + j0 + lr];

    auto block = [&](int n) { return ws + ((int64_t)n * H + h) * B::kSize; };
    // One chunk's operands in registers (A layout unless noted).
    struct Ops {
        float4 Wr[DT], Qr[DT], Pr[NW], Kd[OWN][NW], Ec[OWN];
        float4 Up;     // U'[16w + 4lg + i][j0 + lr], i = 0..3
    };
    auto load_ops = [&](Ops &R, const float *b) {
        R.Up = *reinterpret_cast<const float4 *>(b + B::kU + B::frag(jt, w, NW) + 4 * lane);
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8) {
            R.Wr[t8] = *reinterpret_cast<const float4 *>(b + B::kW + B::frag(w, t8, DT) + 4 * lane);
            R.Qr[t8] = *reinterpret_cast<const float4 *>(b + B::kQ + B::frag(w, t8, DT) + 4 * lane);
        }
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
            R.Pr[w2] = *reinterpret_cast<const float4 *>(b + B::kP + B::frag(w, w2, NW) + 4 * lane);
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
            const int t8 = own_tile(o);
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2)
                R.Kd[o][w2] = *reinterpret_cast<const float4 *>(b + B::kKd + B::frag(t8, w2, NW) + 4 * lane);
            R.Ec[o] = *reinterpret_cast<const float4 *>(b + B::kEc + 16 * t8 + 4 * lg);
        }
    };

    Ops X, Y;
    load_ops(X, block(0));
    // Drain the prologue's loads once; inside the loop the only loads in
    // flight are the next chunk's, issued a whole chunk before their use.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // One chunk: consume `cur`, prefetch chunk n+1 into `nxt`.  The two
    // operand sets alternate (the loop is unrolled by two), so no register
    // copies tie the prefetch to a wait.  The body has no branches (a branch
    // splits it into blocks across which the compiler's wait counting turns
    // conservative).  LAST adds the row guard on the output store: only the
    // last chunk can hold rows >= T.
    auto chunk = [&](int n, Ops &cur, Ops &nxt, auto last) {
        constexpr bool LAST = decltype(last)::value;
        // U = U' - W S = -(W S - U') ;  QS = Qg S.  U' is consumed before
        // its register is reloaded.  Each product runs as two independent
        // accumulators (even / odd channel tiles), four chains interleaved.
        // The next chunk's operands are loaded in small groups between the
        // MFMA groups (same order as load_ops), so the memory pipeline is fed
        // steadily instead of stalling the wave on one burst of loads.
        const float *bn = block(min(n + 1, NC - 1));   // the last chunk reloads itself
        floatx4 WS0 = {-cur.Up.x, -cur.Up.y, -cur.Up.z, -cur.Up.w};
        floatx4 WS1 = {0.f, 0.f, 0.f, 0.f}, QS0 = WS1, QS1 = WS1;
        __builtin_amdgcn_sched_barrier(0);
        nxt.Up = *reinterpret_cast<const float4 *>(bn + B::kU + B::frag(jt, w, NW) + 4 * lane);
#pragma unroll
        for (int t8 = 0; t8 < DT; t8 += 2) {
#pragma unroll
            for (int u = 0; u < 2 && t8 + u < DT; ++u) {
                nxt.Wr[t8 + u] = *reinterpret_cast<const float4 *>(bn + B::kW + B::frag(w, t8 + u, DT) + 4 * lane);
                nxt.Qr[t8 + u] = *reinterpret_cast<const float4 *>(bn + B::kQ + B::frag(w, t8 + u, DT) + 4 * lane);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                WS0 = mfma4(get4(cur.Wr[t8], i), Sr[t8][i], WS0);
                QS0 = mfma4(get4(cur.Qr[t8], i), Sr[t8][i], QS0);
                if (t8 + 1 < DT) {
                    WS1 = mfma4(get4(cur.Wr[t8 + 1], i), Sr[t8 + 1][i], WS1);
                    QS1 = mfma4(get4(cur.Qr[t8 + 1], i), Sr[t8 + 1][i], QS1);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s_u[16 * w + 4 * lg + i][lr] = -(WS0[i] + WS1[i]);
        __syncthreads();   // B1: U rows visible

        // O = scale (QS + P U) and S' = Ec * S + KdT U for the owned tiles,
        // interleaved: P U and each owned tile's product run as two chains
        // (even / odd 16-row blocks of U).  P's blocks above the diagonal are
        // zero.
        float uk[NW][4];
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) uk[w2][kk] = s_u[16 * w2 + 4 * lg + kk][lr];
        floatx4 O0 = {QS0[0] + QS1[0], QS0[1] + QS1[1], QS0[2] + QS1[2], QS0[3] + QS1[3]};
        floatx4 O1 = {0.f, 0.f, 0.f, 0.f};
        floatx4 A0[OWN], A1[OWN];
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
            A0[o] = floatx4{Sown[o][0] * cur.Ec[o].x, Sown[o][1] * cur.Ec[o].y,
                            Sown[o][2] * cur.Ec[o].z, Sown[o][3] * cur.Ec[o].w};
            A1[o] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int w2 = 0; w2 < NW; w2 += 2) {
#pragma unroll
            for (int u = 0; u < 2 && w2 + u < NW; ++u)
                nxt.Pr[w2 + u] = *reinterpret_cast<const float4 *>(bn + B::kP + B::frag(w, w2 + u, NW) + 4 * lane);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                O0 = mfma4(get4(cur.Pr[w2], kk), uk[w2][kk], O0);
#pragma unroll
                for (int o = 0; o < OWN; ++o)
                    A0[o] = mfma4(get4(cur.Kd[o][w2], kk), uk[w2][kk], A0[o]);
                if (w2 + 1 < NW) {
                    O1 = mfma4(get4(cur.Pr[w2 + 1], kk), uk[w2 + 1][kk], O1);
#pragma unroll
                    for (int o = 0; o < OWN; ++o)
                        A1[o] = mfma4(get4(cur.Kd[o][w2 + 1], kk), uk[w2 + 1][kk], A1[o]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
            const int t8 = own_tile(o);
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2)
                nxt.Kd[o][w2] = *reinterpret_cast<const float4 *>(bn + B::kKd + B::frag(t8, w2, NW) + 4 * lane);
            nxt.Ec[o] = *reinterpret_cast<const float4 *>(bn + B::kEc + 16 * t8 + 4 * lg);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t tr = (int64_t)n * C + 16 * w + 4 * lg + i;
            if (!LAST || tr < T) core[(tr * H + h) * D + j0 + lr] = scale * (O0[i] + O1[i]);
        }
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Sown[o][i] = A0[o][i] + A1[o][i];
                s_S[16 * own_tile(o) + 4 * lg + i][lr] = Sown[o][i];
            }
        }
        __syncthreads();   // B2: new state slice visible
#pragma unroll
        for (int t8 = 0; t8 < DT; ++t8)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sr[t8][i] = s_S[16 * t8 + 4 * lg + i][lr];
    };

    int n = 0;
    for (; n + 2 < NC; n += 2) {
        chunk(n, X, Y, std::false_type{});
        chunk(n + 1, Y, X, std::false_type{});
    }
    if (n + 1 < NC) {       // two chunks left
        chunk(n, X, Y, std::false_type{});
        chunk(n + 1, Y, X, std::true_type{});
    } else {                // one chunk left
        chunk(n, X, Y, std::true_type{});
    }

#pragma unroll
    for (int o = 0; o < OWN; ++o)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Sg[(int64_t)(16 * own_tile(o) + 4 * lg + i) * D + j0 + lr] = Sown[o][i];
}

// ---------------------------------------------------------------------------
// kda_chunk_fwd_split: the same pass over the split operand blocks (D and C
// multiples of 32).  Every product runs on the 16x16x32 bf16 MFMA as
// hi*hi + (hi*lo + lo*hi), the two parts in separate fp32 accumulators.
// The right operands (the state slice S and the corrected writes U) are
// split once, by the wave that produced them, and exchanged through LDS as
// ready-made bf16 operands in the pair order of the left operands (see Blk):
// for contraction block kb, lane l's eight values are its elements of fp32
// tiles 2kb and 2kb+1, so the producer of tile t writes its lane's four
// values to half t%2 of block t/2 of the same lane.  The state itself stays
// fp32 in the registers of the wave that updates it.
//
// Two waves per 16-row block of the chunk, one per role, so that each SIMD
// runs one wave of each: the chain waves carry the critical path
// S -> W S -> U -> Kd^T U -> S' and own the state tiles; the output waves
// compute O = scale (Qg S + P U) from the same LDS operands, off that path.
// Both roles pass the same two barriers per chunk (U published; S' published)
// and load their own operands of the next chunk while computing the current
// one.  The operand blocks of a segment are read from the last-level cache;
// what bounds a chunk is the CU's vector-memory data path (each workgroup
// reads the head's whole block per chunk, about 116 KiB).
// ---------------------------------------------------------------------------
// PF = true loads the operands of the next chunk while the current one is
// computed.  PF = false is the instance for launches whose walks are one
// chunk each (every sequence at most C rows): no next chunk to load ahead,
// one operand register set, so two workgroups fit per CU where the
// loading-ahead instance fits one.  Same products in the same order, so the
// same bits.
// LDS of a walk over NJ 16-column tiles: the exchanged right operands.
template <int D, int C, int NJ>
struct __align__(16) WalkLds {
    uint4 s_Sb[NJ][D / 32][2][kWave];   // S slice, right operand (hi, lo), per column tile
    uint4 s_Ub[NJ][C / 32][2][kWave];   // U, right operand (hi, lo), per column tile
};

// The walk of head h over value columns 16*jt0 .. 16*(jt0 + NJ) - 1 by the
// 2*C/16 waves whose workgroup-local thread indices are tid.  Each wave runs
// its role for all NJ column tiles, so the left operands it loads (W, Kd,
// Qg, P: the same for every column of the head) serve NJ tiles; per tile the
// products, their order and every addition are those of NJ = 1, so any NJ
// gives the same bits.
template <int D, int C, bool PF, int NJ>
__device__ __forceinline__ void walk_split(const float *__restrict__ ws, float *__restrict__ state,
                                           float *__restrict__ core, int T, int NC, int H,
                                           float scale, int h, int jt0, int tid,
                                           WalkLds<D, C, NJ> &L)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    constexpr int KD = DT / 2, KC = NW / 2;   // 32-deep blocks over D and over C
    constexpr int OWN = (DT + NW - 1) / NW;
    using B = Blk<D, C>;
    static_assert(B::kSplit, "split operand blocks need D, C multiples of 32");
    const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = r < NW;            // waves 0..NW-1 carry the state
    const int w = chain ? r : r - NW;     // 16-row block of the chunk (and state tiles w + NW o)
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;

    // publish an owned tile (or a U tile) as a right operand: 8 bytes of hi
    // and of lo in half `half` of this lane's 16-byte slots
    auto put = [&](uint4 (&dst)[2][kWave], int half, const float4 &x) {
        uint2 hi, lo;
        split4(x, hi, lo);
        reinterpret_cast<uint2 *>(&dst[0][lane])[half] = hi;
        reinterpret_cast<uint2 *>(&dst[1][lane])[half] = lo;
    };
    auto get = [&](const uint4 (&src)[2][kWave], bf16x8 &hi, bf16x8 &lo) {
        hi = __builtin_bit_cast(bf16x8, src[0][lane]);
        lo = __builtin_bit_cast(bf16x8, src[1][lane]);
    };
    auto block = [&](int n) { return ws + ((int64_t)n * H + h) * B::kSize; };
    auto ldp = [&](const float *p, bf16x8 &hi, bf16x8 &lo) {
        hi = *reinterpret_cast<const bf16x8 *>(p + 4 * lane);
        lo = *reinterpret_cast<const bf16x8 *>(p + 256 + 4 * lane);
    };

    if (chain) {
        // ---- state chain: U = U' - W S, S' = Ec * S + Kd^T U
        // (a global-space pointer: with several sequences the state address
        // comes from a pointer table, and flat accesses would be waited for
        // with the LDS counter)
        typedef __attribute__((address_space(1))) float gfloat;
        gfloat *__restrict__ Sg = (gfloat *)(state + (int64_t)h * D * D);
        auto own_tile = [&](int o) { return min(w + NW * o, DT - 1); };
        // Sown[j][o][i] = S[16*t + 4*lg + i][16*(jt0 + j) + lr], t = own_tile(o)
        float4 Sown[NJ][OWN];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int o = 0; o < OWN; ++o) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    e[i] = Sg[(int64_t)(16 * own_tile(o) + 4 * lg + i) * D + 16 * (jt0 + j) + lr];
                Sown[j][o] = make_float4(e[0], e[1], e[2], e[3]);
            }
        struct Ops {
            bf16x8 Wh[KD], Wl[KD], Kh[OWN][KC], Kl[OWN][KC];
            float4 Ec[OWN];
            float4 Up[NJ];     // U'[16w + 4lg + i][16 (jt0 + j) + lr], i = 0..3
        };
        auto load_Kd = [&](Ops &R, const float *b) {
#pragma unroll
            for (int o = 0; o < OWN; ++o) {
                const int t8 = own_tile(o);
#pragma unroll
                for (int kb = 0; kb < KC; ++kb) ldp(b + B::kKd + B::pfrag(t8, kb, KC), R.Kh[o][kb], R.Kl[o][kb]);
                R.Ec[o] = *reinterpret_cast<const float4 *>(b + B::kEc + 16 * t8 + 4 * lg);
            }
        };
        Ops X;
        [[maybe_unused]] Ops Y;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            X.Up[j] = *reinterpret_cast<const float4 *>(block(0) + B::kU + B::frag(jt0 + j, w, NW) + 4 * lane);
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) ldp(block(0) + B::kW + B::pfrag(w, kb, KD), X.Wh[kb], X.Wl[kb]);
        load_Kd(X, block(0));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int o = 0; o < OWN; ++o) {
                const int t8 = own_tile(o);
                if (DT % NW == 0 || w + NW * o < DT) put(L.s_Sb[j][t8 / 2], t8 % 2, Sown[j][o]);
            }
        __syncthreads();   // B0: S operand visible
        __builtin_amdgcn_sched_barrier(0);

        // Each phase takes the column tiles one after another (their products
        // never mix), so only one tile's right operands are live at a time;
        // the loads of the next chunk's operands go with the first tile.
        auto chunk = [&](int n, Ops &cur, Ops &nxt) {
            [[maybe_unused]] const float *bn = block(min(n + 1, NC - 1));   // the last chunk reloads itself
            if constexpr (PF) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    nxt.Up[j] = *reinterpret_cast<const float4 *>(bn + B::kU + B::frag(jt0 + j, w, NW) + 4 * lane);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bf16x8 sh[KD], sl[KD];
#pragma unroll
                for (int kb = 0; kb < KD; ++kb) get(L.s_Sb[j][kb], sh[kb], sl[kb]);
                floatx4 Wa[2], Wb[2];
                Wa[0] = floatx4{-cur.Up[j].x, -cur.Up[j].y, -cur.Up[j].z, -cur.Up[j].w};
                Wa[1] = Wb[0] = Wb[1] = floatx4{0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KD; ++kb) {
                    if constexpr (PF) {
                        if (j == 0) ldp(bn + B::kW + B::pfrag(w, kb, KD), nxt.Wh[kb], nxt.Wl[kb]);
                    }
                    Wa[kb & 1] = mfma_bf16(cur.Wh[kb], sh[kb], Wa[kb & 1]);
                    Wb[kb & 1] = mfma_bf16(cur.Wh[kb], sl[kb], Wb[kb & 1]);
                    Wb[kb & 1] = mfma_bf16(cur.Wl[kb], sh[kb], Wb[kb & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                float4 u;
                u.x = -((Wa[0][0] + Wa[1][0]) + (Wb[0][0] + Wb[1][0]));
                u.y = -((Wa[0][1] + Wa[1][1]) + (Wb[0][1] + Wb[1][1]));
                u.z = -((Wa[0][2] + Wa[1][2]) + (Wb[0][2] + Wb[1][2]));
                u.w = -((Wa[0][3] + Wa[1][3]) + (Wb[0][3] + Wb[1][3]));
                put(L.s_Ub[j][w / 2], w % 2, u);
            }
            __syncthreads();   // B1: U operand visible; every read of the S operand done
            __builtin_amdgcn_sched_barrier(0);

#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bf16x8 uh[KC], ul[KC];
#pragma unroll
                for (int kb = 0; kb < KC; ++kb) get(L.s_Ub[j][kb], uh[kb], ul[kb]);
                floatx4 Aa[OWN], Ab[OWN];
#pragma unroll
                for (int o = 0; o < OWN; ++o) {
                    Aa[o] = floatx4{Sown[j][o].x * cur.Ec[o].x, Sown[j][o].y * cur.Ec[o].y,
                                    Sown[j][o].z * cur.Ec[o].z, Sown[j][o].w * cur.Ec[o].w};
                    Ab[o] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KC; ++kb) {
#pragma unroll
                    for (int o = 0; o < OWN; ++o) {
                        Aa[o] = mfma_bf16(cur.Kh[o][kb], uh[kb], Aa[o]);
                        Ab[o] = mfma_bf16(cur.Kh[o][kb], ul[kb], Ab[o]);
                        Ab[o] = mfma_bf16(cur.Kl[o][kb], uh[kb], Ab[o]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int o = 0; o < OWN; ++o) {
                    Sown[j][o] = make_float4(Aa[o][0] + Ab[o][0], Aa[o][1] + Ab[o][1],
                                             Aa[o][2] + Ab[o][2], Aa[o][3] + Ab[o][3]);
                }
            }
            if constexpr (PF) load_Kd(nxt, bn);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int o = 0; o < OWN; ++o) {
                    const int t8 = own_tile(o);
                    if (DT % NW == 0 || w + NW * o < DT) put(L.s_Sb[j][t8 / 2], t8 % 2, Sown[j][o]);
                }
            __syncthreads();   // B2: S operand visible; every read of the U operand done
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (PF) {
            int n = 0;
            for (; n + 1 < NC; n += 2) {
                chunk(n, X, Y);
                chunk(n + 1, Y, X);
            }
            if (n < NC) chunk(n, X, Y);
        } else {
            chunk(0, X, X);   // NC == 1
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int o = 0; o < OWN; ++o) {
                const float e[4] = {Sown[j][o].x, Sown[j][o].y, Sown[j][o].z, Sown[j][o].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sg[(int64_t)(16 * own_tile(o) + 4 * lg + i) * D + 16 * (jt0 + j) + lr] = e[i];
            }
    } else {
        // ---- outputs: O = scale (Qg S + P U)
        struct Ops {
            bf16x8 Qh[KD], Ql[KD], Ph[KC], Pl[KC];
        };
        Ops X;
        [[maybe_unused]] Ops Y;
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) ldp(block(0) + B::kQ + B::pfrag(w, kb, KD), X.Qh[kb], X.Ql[kb]);
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
            if (2 * kb <= w)   // fragments wholly above the diagonal are zero (not stored)
                ldp(block(0) + B::kP + B::pfrag(w, kb, KC), X.Ph[kb], X.Pl[kb]);
        __syncthreads();   // B0
        __builtin_amdgcn_sched_barrier(0);

        auto chunk = [&](int n, Ops &cur, Ops &nxt, auto last) {
            constexpr bool LAST = decltype(last)::value;
            [[maybe_unused]] const float *bn = block(min(n + 1, NC - 1));
            floatx4 Oa[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bf16x8 sh[KD], sl[KD];
#pragma unroll
                for (int kb = 0; kb < KD; ++kb) get(L.s_Sb[j][kb], sh[kb], sl[kb]);
                floatx4 Qa[2], Qb[2];
                Qa[0] = Qa[1] = Qb[0] = Qb[1] = floatx4{0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KD; ++kb) {
                    if constexpr (PF) {
                        if (j == 0) ldp(bn + B::kQ + B::pfrag(w, kb, KD), nxt.Qh[kb], nxt.Ql[kb]);
                    }
                    Qa[kb & 1] = mfma_bf16(cur.Qh[kb], sh[kb], Qa[kb & 1]);
                    Qb[kb & 1] = mfma_bf16(cur.Qh[kb], sl[kb], Qb[kb & 1]);
                    Qb[kb & 1] = mfma_bf16(cur.Ql[kb], sh[kb], Qb[kb & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                Oa[j] = floatx4{(Qa[0][0] + Qa[1][0]) + (Qb[0][0] + Qb[1][0]),
                                (Qa[0][1] + Qa[1][1]) + (Qb[0][1] + Qb[1][1]),
                                (Qa[0][2] + Qa[1][2]) + (Qb[0][2] + Qb[1][2]),
                                (Qa[0][3] + Qa[1][3]) + (Qb[0][3] + Qb[1][3])};
            }
            __syncthreads();   // B1
            __builtin_amdgcn_sched_barrier(0);

#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bf16x8 uh[KC], ul[KC];
#pragma unroll
                for (int kb = 0; kb < KC; ++kb) get(L.s_Ub[j][kb], uh[kb], ul[kb]);
                floatx4 Ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KC; ++kb) {
                    if (2 * kb <= w) {
                        if constexpr (PF) {
                            if (j == 0) ldp(bn + B::kP + B::pfrag(w, kb, KC), nxt.Ph[kb], nxt.Pl[kb]);
                        }
                        Oa[j] = mfma_bf16(cur.Ph[kb], uh[kb], Oa[j]);
                        Ob = mfma_bf16(cur.Ph[kb], ul[kb], Ob);
                        Ob = mfma_bf16(cur.Pl[kb], uh[kb], Ob);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t tr = (int64_t)n * C + 16 * w + 4 * lg + i;
                    if (!LAST || tr < T)
                        core[(tr * H + h) * D + 16 * (jt0 + j) + lr] = scale * (Oa[j][i] + Ob[i]);
                }
            }

            __syncthreads();   // B2
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (PF) {
            int n = 0;
            for (; n + 2 < NC; n += 2) {
                chunk(n, X, Y, std::false_type{});
                chunk(n + 1, Y, X, std::false_type{});
            }
            if (n + 1 < NC) {
                chunk(n, X, Y, std::false_type{});
                chunk(n + 1, Y, X, std::true_type{});
            } else {
                chunk(n, X, Y, std::true_type{});
            }
        } else {
            chunk(0, X, X, std::true_type{});   // NC == 1
        }
    }
}

// A walk of one chunk over the whole head by the C/16 waves whose
// workgroup-local thread indices are tid: wave w takes chunk rows
// 16w .. 16w + 15 (U, O) and the state tiles w + (C/16) o (S'), for every
// value-column tile in turn.  All of its left operands (W, Qg, P of its
// rows, Kd of its state tiles, U' of its rows) are loaded at the start; the
// whole incoming state is published to LDS at once, fp32, in the pair order
// of the right operands (a one-chunk walk reads the incoming state only:
// each wave splits what it reads, and the state update reads its tiles
// there too), and U of one column tile at a time, double-buffered, so a
// column tile costs one barrier and no global load.  Per tile every
// product, its accumulator and every addition are those of walk_split, so
// the core rows and the new state are the same bits.
//   blk:   the chunk's operand block;   state: the head's D x D state
//   core:  the chunk's first row;       T: rows of the chunk that exist
//   W_LDS: W and U' are read from wl and ul, LDS in the block's layouts
//          that the workgroup's own prepare left there (and that the state
//          then overwrites), instead of from the block
template <int D, int C>
struct __align__(16) Walk1Lds {
    float4 s_Sf[D / 16][D / 32][2][kWave];  // the state (fp32) in right-operand pair order, per column tile
    uint4 s_Ub[2][C / 32][2][kWave];         // U as right operand, two column tiles in turn
};

template <int D, int C, bool W_LDS = false>
__device__ __forceinline__ void walk1_split(const float *__restrict__ blk, float *__restrict__ state,
                                            float *__restrict__ core, int T, int H, float scale,
                                            int h, int tid, Walk1Lds<D, C> &L,
                                            const float *wl = nullptr, const float *ul = nullptr)
{
    constexpr int NW = PrefCfg<D, C>::kNW, DT = PrefCfg<D, C>::kDT;
    constexpr int KD = DT / 2, KC = NW / 2, OWN = DT / NW;
    using B = Blk<D, C>;
    static_assert(B::kSplit && DT % NW == 0, "split operand blocks, whole state tiles per wave");
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    typedef __attribute__((address_space(1))) float gfloat;
    typedef __attribute__((address_space(1))) char gchar;
    // the state pointer is the same for the whole workgroup (scalar registers)
    const uint64_t sp = reinterpret_cast<uint64_t>(state);
    gfloat *__restrict__ Sg = reinterpret_cast<gfloat *>(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sp >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sp));
    // S[16 t8 + 4 lg + i][16 j + lr], as a 32-bit byte offset from that base
    auto at = [&](int t8, int i, int j) -> gfloat & {
        const uint32_t off = (uint32_t)(((16 * t8 + 4 * lg + i) * D + 16 * j + lr) * 4);
        return *reinterpret_cast<gfloat *>(reinterpret_cast<gchar *>(Sg) + off);
    };
    auto ldS = [&](int t8, int j) { return make_float4(at(t8, 0, j), at(t8, 1, j), at(t8, 2, j), at(t8, 3, j)); };
    auto own_tile = [&](int o) { return w + NW * o; };
    auto put = [&](uint4 (&dst)[2][kWave], int half, const float4 &x) {
        uint2 hi, lo;
        split4(x, hi, lo);
        reinterpret_cast<uint2 *>(&dst[0][lane])[half] = hi;
        reinterpret_cast<uint2 *>(&dst[1][lane])[half] = lo;
    };
    auto get = [&](const uint4 (&src)[2][kWave], bf16x8 &hi, bf16x8 &lo) {
        hi = __builtin_bit_cast(bf16x8, src[0][lane]);
        lo = __builtin_bit_cast(bf16x8, src[1][lane]);
    };
    auto ldp = [&](const float *p, bf16x8 &hi, bf16x8 &lo) {
        hi = *reinterpret_cast<const bf16x8 *>(p + 4 * lane);
        lo = *reinterpret_cast<const bf16x8 *>(p + 256 + 4 * lane);
    };
    auto ldU = [&](int j) {
        return *reinterpret_cast<const float4 *>((W_LDS ? ul : blk + B::kU) + B::frag(j, w, NW) + 4 * lane);
    };

    // every load of the prologue in flight at once: the incoming state of
    // this wave's tiles first, then its left operands
    float4 S0[DT][OWN];
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
        for (int o = 0; o < OWN; ++o) S0[j][o] = ldS(own_tile(o), j);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 Wh[KD], Wl[KD], Qh[KD], Ql[KD], Ph[KC], Pl[KC], Kh[OWN][KC], Kl[OWN][KC];
    float4 Ec[OWN];
#pragma unroll
    for (int kb = 0; kb < KD; ++kb) {
        ldp((W_LDS ? wl : blk + B::kW) + B::pfrag(w, kb, KD), Wh[kb], Wl[kb]);
        ldp(blk + B::kQ + B::pfrag(w, kb, KD), Qh[kb], Ql[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < KC; ++kb)
        if (2 * kb <= w)   // fragments wholly above the diagonal are zero (not stored)
            ldp(blk + B::kP + B::pfrag(w, kb, KC), Ph[kb], Pl[kb]);
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
#pragma unroll
        for (int kb = 0; kb < KC; ++kb) ldp(blk + B::kKd + B::pfrag(own_tile(o), kb, KC), Kh[o][kb], Kl[o][kb]);
        Ec[o] = *reinterpret_cast<const float4 *>(blk + B::kEc + 16 * own_tile(o) + 4 * lg);
    }
    float4 Up[DT];
    if constexpr (W_LDS) {
#pragma unroll
        for (int j = 0; j < DT; ++j) Up[j] = ldU(j);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (W_LDS) __syncthreads();   // every wave has W and U' before the state overwrites them
    // the incoming state of this wave's tiles, every column tile
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
        for (int o = 0; o < OWN; ++o) L.s_Sf[j][own_tile(o) / 2][own_tile(o) % 2][lane] = S0[j][o];
    if constexpr (!W_LDS) {
#pragma unroll
        for (int j = 0; j < DT; ++j) Up[j] = ldU(j);
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < DT; ++j) {
        const float4 up = Up[j];
        // U = U' - W S and QS = Qg S for rows 16w.., column tile j
        bf16x8 sh[KD], sl[KD];
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) split8(L.s_Sf[j][kb][0][lane], L.s_Sf[j][kb][1][lane], sh[kb], sl[kb]);
        floatx4 Wa[2], Wb[2], Qa[2], Qb[2];
        Wa[0] = floatx4{-up.x, -up.y, -up.z, -up.w};
        Wa[1] = Wb[0] = Wb[1] = floatx4{0.f, 0.f, 0.f, 0.f};
        Qa[0] = Qa[1] = Qb[0] = Qb[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) {
            Wa[kb & 1] = mfma_bf16(Wh[kb], sh[kb], Wa[kb & 1]);
            Wb[kb & 1] = mfma_bf16(Wh[kb], sl[kb], Wb[kb & 1]);
            Wb[kb & 1] = mfma_bf16(Wl[kb], sh[kb], Wb[kb & 1]);
            Qa[kb & 1] = mfma_bf16(Qh[kb], sh[kb], Qa[kb & 1]);
            Qb[kb & 1] = mfma_bf16(Qh[kb], sl[kb], Qb[kb & 1]);
            Qb[kb & 1] = mfma_bf16(Ql[kb], sh[kb], Qb[kb & 1]);
        }
        float u[4];
        floatx4 Oa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = -((Wa[0][i] + Wa[1][i]) + (Wb[0][i] + Wb[1][i]));
            Oa[i] = (Qa[0][i] + Qa[1][i]) + (Qb[0][i] + Qb[1][i]);
        }
        put(L.s_Ub[j & 1][w / 2], w % 2, make_float4(u[0], u[1], u[2], u[3]));
        __syncthreads();   // U of tile j visible; every read of U of tile j - 2 done
        bf16x8 uh[KC], ul[KC];
#pragma unroll
        for (int kb = 0; kb < KC; ++kb) get(L.s_Ub[j & 1][kb], uh[kb], ul[kb]);
        // O = scale (QS + P U)
        floatx4 Ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KC; ++kb) {
            if (2 * kb <= w) {
                Oa = mfma_bf16(Ph[kb], uh[kb], Oa);
                Ob = mfma_bf16(Ph[kb], ul[kb], Ob);
                Ob = mfma_bf16(Pl[kb], uh[kb], Ob);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * lg + i;
            if (r < T) core[((int64_t)r * H + h) * D + 16 * j + lr] = scale * (Oa[i] + Ob[i]);
        }
        // S' = Ec * S + Kd^T U for this wave's state tiles
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
            const float4 so = L.s_Sf[j][own_tile(o) / 2][own_tile(o) % 2][lane];
            floatx4 Aa = {so.x * Ec[o].x, so.y * Ec[o].y, so.z * Ec[o].z, so.w * Ec[o].w};
            floatx4 Ab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KC; ++kb) {
                Aa = mfma_bf16(Kh[o][kb], uh[kb], Aa);
                Ab = mfma_bf16(Kh[o][kb], ul[kb], Ab);
                Ab = mfma_bf16(Kl[o][kb], uh[kb], Ab);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) at(own_tile(o), i, j) = Aa[i] + Ab[i];
        }
    }
}

template <int D, int C, bool PF = true, int NJ = 1>
__global__ __launch_bounds__(2 * C / 16 * 64) __attribute__((amdgpu_waves_per_eu(PF || NJ > 1 ? 2 : 4))) void kda_chunk_fwd_split_kernel(
    const float *__restrict__ ws, float *__restrict__ state, float *__restrict__ core, int T,
    int NC, int H, float scale, const Varlen vl)
{
    using B = Blk<D, C>;
    const int h = blockIdx.x % H, jt = NJ * (blockIdx.x / H);
    if (vl.cu) {   // the blockIdx.y-th sequence of the segment: its state and chunks here
        int s;
        SeqSpan sp;
        if (!walker_span<C>(vl, blockIdx.y, s, sp)) return;   // uniform over the workgroup
        const int64_t g0 = max(sp.chunk0, (int64_t)vl.seg_lo);
        const int64_t g1 = min(sp.chunk0 + sp.nch, (int64_t)vl.seg_hi);
        if (g0 >= g1) return;
        const int c0 = (int)(g0 - sp.chunk0);   // first chunk of the sequence walked here
        state = vl.states[s];
        core += (sp.row0 + (int64_t)c0 * C) * H * D;
        ws += (g0 - vl.seg_lo) * H * B::kSize;
        NC = (int)(g1 - g0);
        T = min(sp.T - c0 * C, NC * C);
    }
    __shared__ WalkLds<D, C, NJ> L;
    walk_split<D, C, PF, NJ>(ws, state, core, T, NC, H, scale, h, jt, (int)threadIdx.x, L);
}

// The forward pass over walks of one chunk each (kda_chunk_fwd_split_kernel
// without its load-ahead register set, or whole-head walk1_split workgroups),
// launched from its own translation unit so that the kernels here keep their
// place in this file's module.
template <int D, int C>
hipError_t fwd_split_one_chunk(dim3 grid, const float *ws, float *state, float *core, int T,
                               int NC, int H, float scale, const Varlen &vl, hipStream_t stream);
// Prepare and walk of a several-sequence launch whose sequences are all at
// most one chunk, in one kernel.
template <int D, int C>
hipError_t prefill_one_chunk(const float *q, const float *k, const float *v, const float *gate,
                             const float *beta, float *core, int H, float scale, void *workspace,
                             const Varlen &vl, hipStream_t stream);

}  // namespace kda
