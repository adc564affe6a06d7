// Recurrent KDA decode: one or K tokens per sequence, state read once from HBM,
// walked in registers, written once (plus optional per-row snapshots).
//
// Operation ("Glm5NextKdaLayer" page, decode and decode_k): per head, with
// S[i][j] (i = key channel, j = value channel), each token:
//   S' = diag(exp(g)) S;  u = beta (v - S'^T k);  S = S' + k u^T;
//   o  = scale S^T q = scale (S'^T q + u (k . q)).
// The second form of o needs one reduction pass over S instead of two; it is
// the same quantity.
//
// Layout: one workgroup per (head, column slice, sequence).  The head's D x D
// fp32 state is contiguous (64 KiB at D = 128); thread t owns the float4
// column group cg = t % (DC/4) of its slice in rows rg + 16*r, so every
// load/store instruction covers whole 128-byte row pieces (128-bit accesses).
// Column sums over the key axis take a fixed tree (see RecCfg).  The same kernel serves
// single-token decode (K = 1) and K-token decode, which makes the K-token
// result bit-identical to K single-token calls: each step runs the same
// instructions on the same values, and fp32 registers hold exactly what an
// fp32 store and reload would.
//
// Write-on-accept ("Glm5NextLayer" page, LayerWriteOnAccept: verify, then
// fold the accepted rows into the state) is two more runs of the same code:
// a verify run writes the K rows' outputs and leaves the state untouched
// (write_state false), and a fold run applies the first n_accept[b] rows to
// the state and writes no output.  The state a fold leaves is therefore
// bitwise the snapshot a K-row decode would have written after that row.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_gemv.hpp"
#include "kda_launch.hpp"
#include "kda_rows.hpp"

namespace kda {

// One workgroup per (head, value-column slice, sequence).  The recurrence
// never mixes value columns (column j of S evolves with its own u_j), so a
// head's state splits into NS slices of D/NS columns with no exchange.  The
// key-axis sums are formed in an order fixed by D alone — 16 row groups each
// chain their D/16 rows (rows rg, rg + 16, ...), partner groups (2p, 2p + 1)
// are added, and the 8 pair sums are added in order p = 0..7 — so every
// slice count gives the same bits, and the launch picks the count from the
// batch size: few sequences get more, smaller workgroups.  Likewise a thread
// may carry one row group or a partner pair of them (RGT), which moves the
// pair sum from a shuffle into the thread without changing it.
template <int D, int NS, int RGT = 1>
struct RecCfg {
    static constexpr int kRG = 16;                 // row groups
    static constexpr int kRGT = RGT;               // row groups per thread (1 or 2)
    static constexpr int kDC = D / NS;             // columns per slice
    static constexpr int kCG = kDC / 4;            // float4 column groups per row
    static constexpr int kThreads = kRG / RGT * kCG;
    static constexpr int kRPT = D / kRG;           // rows per row group
    static constexpr int kPairs = kRG / 2;
    static_assert(RGT == 2 || (2 * kCG <= kWave && kWave % (2 * kCG) == 0),
                  "row-group pairs must share a wave");
    static_assert(kRPT * kRG == D && kDC * NS == D && kDC % 4 == 0, "bad tiling");
};

// State traffic is touched once per call: non-temporal 16-byte accesses
// (streaming through the caches) measured ~11 % faster than plain ones.
__device__ __forceinline__ float4 load_stream(const float *p) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_stream(float *p, const float4 &v) {
    __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4 *>(p));
}

__device__ __forceinline__ float4 fma4(float a, const float4 &b, const float4 &c) {
    return make_float4(__builtin_fmaf(a, b.x, c.x), __builtin_fmaf(a, b.y, c.y),
                       __builtin_fmaf(a, b.z, c.z), __builtin_fmaf(a, b.w, c.w));
}

// The key-axis partial sums of one row (exchanged through LDS).
template <int D, int NS, int RGT>
struct __align__(16) RecRed {
    float4 s_red[RecCfg<D, NS, RGT>::kPairs][2][RecCfg<D, NS, RGT>::kCG];
    float s_kq[RecCfg<D, NS, RGT>::kPairs];
};

// The workgroup's LDS: one row's q, k, v and decay factors e = exp(g), and the
// key-axis partial sums.
template <int D, int NS, int RGT>
struct __align__(16) RecLds {
    float s_q[D], s_k[D], s_v[D], s_e[D];
    RecRed<D, NS, RGT> red;
};

// One row of the recurrence over this workgroup's slice (value columns c0 ..
// c0 + D/NS - 1), with the row's q, k, v and e (D values each, in LDS):
// decays S, forms u = beta (v - S'^T k) and o = scale (S'^T q + u (k . q)),
// and adds k u^T to S.  Thread row 0 owns whole columns and stores o: to
// core_row (the row's first value column of this slice) and o_lds (the same
// columns), each when given; and u to u_row (same columns) when given.
// Passes one barrier (the key-axis sums go through R); the caller passes
// another before R or the row's operands are rewritten.
template <int D, int NS, int RGT>
__device__ __forceinline__ void rec_row(float4 (&S)[RGT][D / 16], const float *s_q,
                                        const float *s_k, const float *s_v, const float *s_e,
                                        RecRed<D, NS, RGT> &R, float bt, float scale, int c0,
                                        int tid, float *core_row, float *o_lds,
                                        float *u_row = nullptr)
{
    using Cfg = RecCfg<D, NS, RGT>;
    constexpr int CG = Cfg::kCG, RG = Cfg::kRG, RPT = Cfg::kRPT, NP = Cfg::kPairs;
    const int cg = tid % CG;
    const int tr = tid / CG;                        // thread row index
    // row group of this thread's j-th set of rows: tr, or 2 tr + j
    auto rgof = [&](int j) { return RGT == 1 ? tr : 2 * tr + j; };

    // decay, then per row group the partial column sums of S'^T k and
    // S'^T q over its rows, and the matching partial of k . q
    float4 pkj[RGT], pqj[RGT];
    float kqj[RGT];
#pragma unroll
    for (int j = 0; j < RGT; ++j) {
        pkj[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        pqj[j] = pkj[j];
        kqj[j] = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rgof(j) + RG * r;
            const float e = s_e[i], ki = s_k[i], qi = s_q[i];
            S[j][r] = make_float4(S[j][r].x * e, S[j][r].y * e, S[j][r].z * e, S[j][r].w * e);
            pkj[j] = fma4(ki, S[j][r], pkj[j]);
            pqj[j] = fma4(qi, S[j][r], pqj[j]);
            kqj[j] = __builtin_fmaf(ki, qi, kqj[j]);
        }
    }
    // add partner row groups (2p, 2p + 1): in the thread, or CG lanes
    // apart in one wave; then the 8 pair sums in order through LDS
    float4 pk = pkj[0], pq = pqj[0];
    float kq = kqj[0];
    if constexpr (RGT == 2) {
        pk = make_float4(pk.x + pkj[1].x, pk.y + pkj[1].y, pk.z + pkj[1].z, pk.w + pkj[1].w);
        pq = make_float4(pq.x + pqj[1].x, pq.y + pqj[1].y, pq.z + pqj[1].z, pq.w + pqj[1].w);
        kq += kqj[1];
    } else {
        pk.x += __shfl_xor(pk.x, CG); pk.y += __shfl_xor(pk.y, CG);
        pk.z += __shfl_xor(pk.z, CG); pk.w += __shfl_xor(pk.w, CG);
        pq.x += __shfl_xor(pq.x, CG); pq.y += __shfl_xor(pq.y, CG);
        pq.z += __shfl_xor(pq.z, CG); pq.w += __shfl_xor(pq.w, CG);
        kq += __shfl_xor(kq, CG);
    }
    const int pr = RGT == 2 ? tr : tr >> 1;   // pair index
    if (RGT == 2 || (tr & 1) == 0) {
        R.s_red[pr][0][cg] = pk;
        R.s_red[pr][1][cg] = pq;
        if (cg == 0) R.s_kq[pr] = kq;
    }
    __syncthreads();
    pk = R.s_red[0][0][cg];
    pq = R.s_red[0][1][cg];
    kq = R.s_kq[0];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
        const float4 a = R.s_red[p][0][cg], c = R.s_red[p][1][cg];
        pk = make_float4(pk.x + a.x, pk.y + a.y, pk.z + a.z, pk.w + a.w);
        pq = make_float4(pq.x + c.x, pq.y + c.y, pq.z + c.z, pq.w + c.w);
        kq += R.s_kq[p];
    }
    const float4 v4 = reinterpret_cast<const float4 *>(s_v + c0)[cg];
    const float4 u = make_float4(bt * (v4.x - pk.x), bt * (v4.y - pk.y),
                                 bt * (v4.z - pk.z), bt * (v4.w - pk.w));
    if ((core_row != nullptr || o_lds != nullptr) && tr == 0) {
        const float4 o = make_float4(scale * __builtin_fmaf(u.x, kq, pq.x),
                                     scale * __builtin_fmaf(u.y, kq, pq.y),
                                     scale * __builtin_fmaf(u.z, kq, pq.z),
                                     scale * __builtin_fmaf(u.w, kq, pq.w));
        if (core_row != nullptr) reinterpret_cast<float4 *>(core_row)[cg] = o;
        if (o_lds != nullptr) reinterpret_cast<float4 *>(o_lds)[cg] = o;
    }
    if (u_row != nullptr && tr == 0) reinterpret_cast<float4 *>(u_row)[cg] = u;
#pragma unroll
    for (int j = 0; j < RGT; ++j)
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            S[j][r] = fma4(s_k[rgof(j) + RG * r], u, S[j][r]);
}

template <int D, int NS, int RGT>
__global__ __launch_bounds__((RecCfg<D, NS, RGT>::kThreads)) void kda_recurrent_kernel(
    const uint16_t *__restrict__ qkv, int64_t ldqkv, const float *__restrict__ gate,
    const float *__restrict__ beta, float *const *__restrict__ state,
    float *const *__restrict__ snap, float *__restrict__ core, int K, int H, float scale,
    bool write_state, const int32_t *__restrict__ n_accept, int32_t *__restrict__ status,
    float *const *__restrict__ wy)
{
    using Cfg = RecCfg<D, NS, RGT>;
    constexpr int CG = Cfg::kCG, RG = Cfg::kRG, RPT = Cfg::kRPT;

    const int h = blockIdx.x / NS;
    const int c0 = (blockIdx.x % NS) * Cfg::kDC;   // first value column of this slice
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int tr = tid / CG;                        // thread row index
    const int qkvw = H * D;
    // row group of this thread's j-th set of rows: tr, or 2 tr + j
    auto rgof = [&](int j) { return RGT == 1 ? tr : 2 * tr + j; };

    __shared__ RecLds<D, NS, RGT> L;

    // rows walked: all K, or the accepted ones when folding (none: nothing to
    // do); a count outside [0, K] is clamped and reported (one thread per
    // sequence)
    const int na = n_accept ? n_accept[b] : K;
    if (status != nullptr && (na < 0 || na > K) && blockIdx.x == 0 && tid == 0)
        atomicOr(status, kReportAcceptClamped);
    const int rows = min(max(na, 0), K);
    if (rows == 0) return;   // uniform over the workgroup

    float *__restrict__ Sg = state[b] + (size_t)h * D * D + c0;
    float4 S[RGT][RPT];
#pragma unroll
    for (int j = 0; j < RGT; ++j)
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            S[j][r] = load_stream(Sg + (size_t)(rgof(j) + RG * r) * D + 4 * cg);

    for (int t = 0; t < rows; ++t) {
        const size_t row = (size_t)b * K + t;
        const uint16_t *__restrict__ qrow = qkv + row * ldqkv + (size_t)h * D;
        for (int i = tid; i < D; i += Cfg::kThreads) {
            L.s_q[i] = bf16_to_f32(qrow[i]);
            L.s_k[i] = bf16_to_f32(qrow[qkvw + i]);
            L.s_v[i] = bf16_to_f32(qrow[2 * qkvw + i]);
            L.s_e[i] = exp2_fast(gate[(row * H + h) * D + i] * kLog2e);
        }
        const float bt = beta[row * H + h];
        __syncthreads();

        rec_row<D, NS, RGT>(S, L.s_q, L.s_k, L.s_v, L.s_e, L.red, bt, scale, c0, tid,
                            core != nullptr ? core + (row * H + h) * D + c0 : nullptr, nullptr,
                            wy != nullptr ? wy[b] + ((size_t)h * K + t) * D + c0 : nullptr);

        if (snap != nullptr && t + 1 < K) {
            float *__restrict__ Sn = snap[(size_t)b * (K - 1) + t] + (size_t)h * D * D + c0;
#pragma unroll
            for (int j = 0; j < RGT; ++j)
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    store_stream(Sn + (size_t)(rgof(j) + RG * r) * D + 4 * cg, S[j][r]);
        }
        __syncthreads();  // LDS is rewritten by the next row
    }

    if (write_state) {
#pragma unroll
        for (int j = 0; j < RGT; ++j)
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                store_stream(Sg + (size_t)(rgof(j) + RG * r) * D + 4 * cg, S[j][r]);
    }
}

// Entry b of a device table of device pointers, read on the vector-memory
// path (a buffer load) instead of the scalar one, and kept in vector
// registers: the read then counts among the wave's vector loads, so the
// loads issued after it that need no table overlap its latency, and only the
// loads through the pointer wait for it.
template <typename T>
__device__ __forceinline__ T *table_entry(T *const *table, int b)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T **>(table), (short)0, (b + 1) * (int)sizeof(T *), 0x00020000);
    const uint2 p = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  r, (unsigned)b * sizeof(T *), 0, 0));
    return reinterpret_cast<T *>((uint64_t)p.x | ((uint64_t)p.y << 32));
}

// load_stream through a pointer known to address device memory (a global
// access rather than a flat one, which the LDS wait counter would also track)
typedef __attribute__((address_space(1))) floatx4 gfloatx4;
__device__ __forceinline__ float4 gload_stream(const float *p) {
    const floatx4 v = __builtin_nontemporal_load((const gfloatx4 *)p);
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void gstore_stream(float *p, const float4 &v) {
    __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, (gfloatx4 *)p);
}

// The block decode's per-head stages, one workgroup per (head h, sequence b)
// over the whole head (see launch_kda_mixer).  Every global operand is
// loaded first — the pointer-table entries of the sequence (state, conv
// window, u rows, snapshots), then what needs no table (gate weights, conv
// taps and pre-conv rows, fa and ga rows, the gate constants, beta), then the
// carried conv rows and last the state, which only the recurrence waits for.
// Every load is issued whatever the thread's item (indices clamped to ones
// that exist, unused values dropped), so that the compiler can count the
// loads in flight exactly and wait for each group alone: a load issued
// under a branch makes it wait for everything issued before.  Then:
//   1. conv + SiLU + L2 of all K rows at once, a thread per (row, section q,
//      k or v, 8 channels), the head's D/8 threads of a section adjacent and
//      aligned so the L2 sum takes conv_silu_l2's shuffle tree; rows to LDS;
//   2. wave w forms column tile w of the head in the f_b product and in the
//      g_b product as dense_gemv_bf16_batchm forms them (kda_gemv.hpp; with
//      R <= 128 each contraction quarter is one step: quarter q takes step
//      q), the A operand (fa or ga rows) from LDS; then a thread per (row,
//      column) rounds them: g_raw with the log-decay gate of its bf16 value
//      (as the f_b product's epilogue forms it, kept in LDS as exp(gate)),
//      out_gate;
//   3. the recurrence row by row (one barrier a row: the key-axis sums of
//      consecutive rows use two buffers), outputs kept in LDS;
//   4. the gated RMSNorm of all K rows at once (the head's D/8 threads of a
//      row adjacent and aligned, gated_rmsnorm's shuffle tree), and, when
//      the states are written, the conv window moved past the K rows.
// Each stage runs the per-row code of its own kernel on the same values, so
// every buffer gets the bits those launches write.
template <int D>
struct MixerCfg {
    using Rec = RecCfg<D, 1, 1>;
    static constexpr int kThreads = Rec::kThreads;
    static constexpr int kWaves = kThreads / kWave;
    static constexpr int kSL = D / 8;                  // threads per section of a row
    static constexpr int kCL = 3 * kSL;                // conv threads per row
    static constexpr int kTiles = D / kGemvColTile;    // column tiles per product
    static constexpr int kLR = kMixerMaxRank + 8;      // LDS row stride of fa, ga (elements)
    static_assert(kThreads % kWave == 0 && kWave % kSL == 0, "sections must not straddle waves");
    static_assert(kTiles == kWaves, "one column tile of each product per wave");
};

// A warm-up workgroup (MixerArgs::warm_w): workgroup j of nw, dispatched as
// number base + j, reads one word of every 128-byte line of the tiles t = x
// (mod 8), x its XCD, nw / 8 workgroups sharing each XCD's tiles.  It first
// sleeps warm_sleeps x 2048 cycles (about the mixer's load phase), so the
// mixer's own loads go ahead.
template <int NT>
__device__ __forceinline__ void mixer_warm(const MixerArgs &a, int j, int nw, int base, int tid)
{
    const int per = nw / 8;
    if (j >= 8 * per) return;
    const int x = (base + j) & 7;
    const int64_t tb = a.warm_tile_bytes, tiles = (a.warm_bytes + tb - 1) / tb;
    const int64_t lines_per_tile = tb / 128;
    // this workgroup's tiles: x + 8 (j / 8) + 8 per r, r = 0, 1, ...
    const int64_t t0 = x + 8 * (j / 8), dt = 8 * (int64_t)per;
    const int64_t mine = t0 < tiles ? (tiles - 1 - t0) / dt + 1 : 0;
    const int64_t total = mine * lines_per_tile;
    const char *w = reinterpret_cast<const char *>(a.warm_w);
    for (int i = 0; i < a.warm_sleeps; ++i) __builtin_amdgcn_s_sleep(32);
    uint32_t acc = 0;
#pragma unroll 4
    for (int64_t i = tid; i < total; i += NT) {
        const int64_t off = (t0 + dt * (i / lines_per_tile)) * tb + 128 * (i % lines_per_tile);
        if (off < a.warm_bytes) acc ^= *reinterpret_cast<const uint32_t *>(w + off);
    }
    asm volatile("" ::"v"(acc));   // the words are read, their values unused
}

template <int D, int KS>
__global__ __launch_bounds__((MixerCfg<D>::kThreads)) void kda_mixer_kernel(const MixerArgs a)
{
    if ((int)blockIdx.y >= a.B) {   // a warm-up workgroup
        mixer_warm<MixerCfg<D>::kThreads>(a, (int)(blockIdx.x + gridDim.x * (blockIdx.y - a.B)),
                                          (int)(gridDim.x * (gridDim.y - a.B)),
                                          a.H * a.B, (int)threadIdx.x);
        return;
    }
    using Cfg = MixerCfg<D>;
    using Rec = typename Cfg::Rec;
    constexpr int NT = Cfg::kThreads, SL = Cfg::kSL, CL = Cfg::kCL, LR = Cfg::kLR;
    constexpr int CG = Rec::kCG, RG = Rec::kRG, RPT = Rec::kRPT;
    const int h = blockIdx.x, b = blockIdx.y, K = a.K, H = a.H, R = a.R;
    const int tid = threadIdx.x;
    const int cg = tid % CG, tr = tid / CG;
    const int wave = tid / kWave, lane = tid % kWave;
    const int lr = lane & 15, kg = lane >> 4;
    const int64_t qkvw = (int64_t)H * D, cd = 3 * qkvw, row0 = (int64_t)b * K;
    const int nsteps = R >> 5;   // 1 .. 4

    __shared__ __align__(16) float s_x[kMixerMaxRows][3][D];   // conv output rows: q, k, v
    __shared__ __align__(16) float s_e[kMixerMaxRows][D];      // exp(gate)
    __shared__ __align__(16) float s_o[kMixerMaxRows][D];      // recurrence outputs
    __shared__ __align__(16) uint16_t s_og[kMixerMaxRows][D];  // out_gate
    __shared__ __align__(16) uint16_t s_lr[2][kMixerMaxRows * LR];   // fa, ga rows
    __shared__ float s_g[kMixerMaxRows][2 * D];                 // gate products, fp32
    __shared__ __align__(16) float s_dtb[D];
    __shared__ float s_beta[kMixerMaxRows], s_rate;
    __shared__ float *s_snp[kMixerMaxRows];       // state snapshot after each row but the last
    __shared__ uint16_t *s_csnp[kMixerMaxRows];   // conv snapshot after each row but the last
    __shared__ RecRed<D, 1, 1> s_red[2];

    // --- loads: the pointer-table entries (snapshots of row min(tid, K-2),
    // staged in LDS for every thread) ---
    float *const Sb = table_entry(a.state, b);
    const uint16_t *const cst = table_entry(a.conv_state, b);
    float *const wyb = a.wy != nullptr ? table_entry(a.wy, b) : nullptr;
    const int snap0 = b * (K - 1) + min(tid, max(K - 2, 0));
    float *const snp = a.snap != nullptr && K > 1 ? table_entry(a.snap, snap0) : nullptr;
    uint16_t *const csnp = a.conv_snap != nullptr && K > 1 ? table_entry(a.conv_snap, snap0) : nullptr;

    // gate weights: column tile `wave` of each product, this lane's row, step
    // q, in the MFMA operand's layout
    uintx4 wf[kGemvQuarters], wg[kGemvQuarters];
    {
        const int64_t n = (int64_t)h * D + kGemvColTile * wave + lr;
#pragma unroll
        for (int q = 0; q < kGemvQuarters; ++q) {
            const int64_t o = n * R + 32 * min(q, nsteps - 1) + 8 * kg;
            wf[q] = *reinterpret_cast<const uintx4 *>(a.f_b + o);
            wg[q] = *reinterpret_cast<const uintx4 *>(a.g_b + o);
        }
    }

    // conv items: i = (row t, section, 8 channels), row-major; the window of
    // row t is entries t .. t + 3 of [carried rows 1 .. 3; rows 0 .. K-1]
    const int nitems = K * CL;
    auto item = [&](int i, int &t, int &section, int64_t &c) {
        t = i / CL;
        section = (i % CL) / SL;
        c = section * qkvw + (int64_t)h * D + 8 * (i % SL);
    };
    auto load_x = [&](int i, uint4 (&taps)[kConvKC], uint4 (&xw)[kConvKC]) {
        int t, section;
        int64_t c;
        item(i, t, section, c);
        conv_taps_load(a.conv_w, c, taps);
#pragma unroll
        for (int jj = 0; jj < kConvKC; ++jj) {
            const int e = max(t + jj, kConvKC - 1);
            xw[jj] = *reinterpret_cast<const uint4 *>(a.x + (row0 + e - (kConvKC - 1)) * a.ldx + c);
        }
    };
    auto load_carried = [&](int i, uint4 (&cw)[kConvKC - 1]) {
        int t, section;
        int64_t c;
        item(i, t, section, c);
#pragma unroll
        for (int jj = 0; jj + 1 < kConvKC; ++jj)
            cw[jj] = gload16(cst + (int64_t)(min(t + jj, kConvKC - 2) + 1) * cd + c);
    };
    const int i0 = min(tid, nitems - 1);
    uint4 taps[kConvKC], xw[kConvKC], cw[kConvKC - 1];
    load_x(i0, taps, xw);

    // fa and ga rows (one 16-byte piece a thread when that covers them), the
    // gate constants, beta
    constexpr int kLrAll = 2 * kMixerMaxRows * kMixerMaxRank / 8;   // pieces at most
    const int nlr = 2 * K * (R / 8);
    auto lr_piece = [&](int i) {
        const int which = i / (K * (R / 8)), e = i % (K * (R / 8));
        return (which == 0 ? a.fa : a.ga) + row0 * R + 8 * e;
    };
    auto lr_store = [&](int i, const uint4 &v) {
        const int which = i / (K * (R / 8)), e = i % (K * (R / 8));
        *reinterpret_cast<uint4 *>(&s_lr[which][(e / (R / 8)) * LR + 8 * (e % (R / 8))]) = v;
    };
    // With KS > 1 the front left f_a, g_a and b_proj as KS chunk sums each
    // (launch_lowrank_finish's layout): this thread's piece of 8 columns and
    // beta's b_proj column come as their chunk sums, added here in chunk
    // order (split_sum), and fa, ga, b_raw and beta are written here.
    const int64_t Mrows = (int64_t)a.B * K;
    uint4 lrv = make_uint4(0u, 0u, 0u, 0u);
    float4 lp[KS][2];
    float bp[KS], btv = 0.f;
    if constexpr (KS == 1) {
        if constexpr (kLrAll <= NT) lrv = *reinterpret_cast<const uint4 *>(lr_piece(min(tid, nlr - 1)));
        btv = a.beta[(row0 + min(tid, K - 1)) * H + h];
    } else {
        if constexpr (kLrAll <= NT) {
            const int i = min(tid, nlr - 1);
            const int which = i / (K * (R / 8)), e = i % (K * (R / 8));
            const float *pw = a.lr_part + ((int64_t)which * KS * Mrows + row0 + e / (R / 8)) * R +
                              8 * (e % (R / 8));
#pragma unroll
            for (int c = 0; c < KS; ++c) {
                lp[c][0] = *reinterpret_cast<const float4 *>(pw + (int64_t)c * Mrows * R);
                lp[c][1] = *reinterpret_cast<const float4 *>(pw + (int64_t)c * Mrows * R + 4);
            }
        }
        const float *pb = a.lr_part + 2 * KS * Mrows * R + (row0 + min(tid, K - 1)) * H + h;
#pragma unroll
        for (int c = 0; c < KS; ++c) bp[c] = pb[(int64_t)c * Mrows * H];
    }
    const float4 dtv = *reinterpret_cast<const float4 *>(a.dt_bias + (int64_t)h * D + 4 * (tid % (D / 4)));
    const float alog = a.a_log[h];
    const uint4 nw = *reinterpret_cast<const uint4 *>(a.norm_w + 8 * (tid % SL));

    // through the tables: the carried conv rows, then the state
    load_carried(i0, cw);
    float *__restrict__ Sg = Sb + (size_t)h * D * D;
    float4 S[1][RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[0][r] = gload_stream(Sg + (size_t)(tr + RG * r) * D + 4 * cg);

    // small operands to LDS
    if constexpr (KS == 1) {
        if constexpr (kLrAll <= NT) {
            if (tid < nlr) lr_store(tid, lrv);
        } else {
            for (int i = tid; i < nlr; i += NT) lr_store(i, *reinterpret_cast<const uint4 *>(lr_piece(i)));
        }
        if (tid < K) s_beta[tid] = btv;
    } else {
        // a piece: 8 columns of row ml of fa or ga, rounded as the front's
        // epilogue would have rounded them (sequence b's rows written by head 0)
        auto finish_piece = [&](int i, const float (&f)[8]) {
            const int which = i / (K * (R / 8)), e = i % (K * (R / 8));
            const uint4 v = pack8(f);
            lr_store(i, v);
            if (h == 0)
                *reinterpret_cast<uint4 *>((which == 0 ? a.fa : a.ga) + row0 * R + 8 * e) = v;
        };
        if constexpr (kLrAll <= NT) {
            if (tid < nlr) {
                float f[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    f[jj] = get4(lp[0][jj / 4], jj % 4);
#pragma unroll
                    for (int c = 1; c < KS; ++c) f[jj] = f[jj] + get4(lp[c][jj / 4], jj % 4);
                }
                finish_piece(tid, f);
            }
        } else {
            for (int i = tid; i < nlr; i += NT) {
                const int which = i / (K * (R / 8)), e = i % (K * (R / 8));
                const float *pw = a.lr_part + (int64_t)which * KS * Mrows * R;
                float f[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    f[jj] = split_sum(pw, KS, Mrows, row0 + e / (R / 8), R, 8 * (e % (R / 8)) + jj);
                finish_piece(i, f);
            }
        }
        if (tid < K) {
            float v = bp[0];
#pragma unroll
            for (int c = 1; c < KS; ++c) v = v + bp[c];
            const uint32_t u = f32_to_bf16(v);
            const float bt = sigmoid_fast(bf16_to_f32(u));
            a.b_raw[(row0 + tid) * H + h] = (uint16_t)u;
            a.beta[(row0 + tid) * H + h] = bt;
            s_beta[tid] = bt;
        }
    }
    if (tid < D / 4) reinterpret_cast<float4 *>(s_dtb)[tid] = dtv;
    if (tid == 0) s_rate = decay_rate(alog);
    if (tid + 1 < K) {
        s_snp[tid] = snp;
        s_csnp[tid] = csnp;
    }
    __syncthreads();

    // --- 1. conv of every row (whole sections per pass: NT % SL == 0) ---
    auto conv_item = [&](int i, const uint4 (&tp)[kConvKC], const uint4 (&xr)[kConvKC],
                         const uint4 (&cr)[kConvKC - 1]) {
        int t, section;
        int64_t c;
        item(i, t, section, c);
        uint4 win[kConvKC];
#pragma unroll
        for (int jj = 0; jj < kConvKC; ++jj)
            win[jj] = jj + 1 < kConvKC && t + jj < kConvKC - 1 ? cr[min(jj, kConvKC - 2)] : xr[jj];
        float wt[8][kConvKC];
        conv_taps_unpack(tp, wt);
        const uint4 packed = conv_row<SL>(win, wt, section < 2, a.eps_l2);
        *reinterpret_cast<uint4 *>(a.y + (row0 + t) * a.ldy + c) = packed;
        if (a.conv_snap != nullptr && t + 1 < K) {
            uint16_t *dst = s_csnp[t];
#pragma unroll
            for (int jj = 0; jj < kConvKC; ++jj) gstore16(dst + (int64_t)jj * cd + c, win[jj]);
        }
        float f[8];
        unpack8(packed, f);
        float *dst = &s_x[t][section][8 * (i % SL)];
        reinterpret_cast<float4 *>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
        reinterpret_cast<float4 *>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
    };
    if (tid < nitems) conv_item(tid, taps, xw, cw);
    for (int i = NT + tid; i < nitems; i += NT) {   // more items than threads
        load_x(i, taps, xw);
        load_carried(i, cw);
        conv_item(i, taps, xw, cw);
    }

    // --- 2. the gate products (rows past K of the A operand are left zero:
    // a row only meets its own output row), quarters added in order ---
    {
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        uintx4 xf[kGemvQuarters] = {}, xg[kGemvQuarters] = {};
        if (lr < K) {
#pragma unroll
            for (int q = 0; q < kGemvQuarters; ++q) {
                const int o = lr * LR + 32 * min(q, nsteps - 1) + 8 * kg;
                xf[q] = *reinterpret_cast<const uintx4 *>(&s_lr[0][o]);
                xg[q] = *reinterpret_cast<const uintx4 *>(&s_lr[1][o]);
            }
        }
        floatx4 pf[kGemvQuarters], pg[kGemvQuarters];
#pragma unroll
        for (int q = 0; q < kGemvQuarters; ++q) {
            pf[q] = mfma_bf16(__builtin_bit_cast(bf16x8, xf[q]), __builtin_bit_cast(bf16x8, wf[q]), zero);
            pg[q] = mfma_bf16(__builtin_bit_cast(bf16x8, xg[q]), __builtin_bit_cast(bf16x8, wg[q]), zero);
        }
        floatx4 tf = pf[0], tg = pg[0];   // quarters past the last step add zeros
#pragma unroll
        for (int q = 1; q < kGemvQuarters; ++q) {
            tf = tf + (q < nsteps ? pf[q] : zero);
            tg = tg + (q < nsteps ? pg[q] : zero);
        }
        // rows 4 kg + i, column lr of the tile
        const int col = kGemvColTile * wave + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * kg + i < K) {
                s_g[4 * kg + i][col] = tf[i];
                s_g[4 * kg + i][D + col] = tg[i];
            }
    }
    __syncthreads();
    for (int i = tid; i < 2 * K * D; i += NT) {
        const int ml = i / (2 * D), col = i % (2 * D);
        const uint32_t u = f32_to_bf16(s_g[ml][col]);
        if (col < D) {
            const int64_t o = (row0 + ml) * qkvw + (int64_t)h * D + col;
            const float gv = log_decay(bf16_to_f32(u), s_dtb[col], s_rate);
            a.g_raw[o] = (uint16_t)u;
            a.gate[o] = gv;
            s_e[ml][col] = exp2_fast(gv * kLog2e);
        } else {
            a.out_gate[(row0 + ml) * qkvw + (int64_t)h * D + col - D] = (uint16_t)u;
            s_og[ml][col - D] = (uint16_t)u;
        }
    }
    __syncthreads();

    // --- 3. the recurrence ---
    for (int t = 0; t < K; ++t) {
        const int64_t row = row0 + t;
        rec_row<D, 1, 1>(S, s_x[t][0], s_x[t][1], s_x[t][2], s_e[t], s_red[t & 1], s_beta[t],
                         a.scale, 0, tid, a.core + (row * H + h) * D, s_o[t],
                         wyb != nullptr ? wyb + ((size_t)h * K + t) * D : nullptr);
        if (a.snap != nullptr && t + 1 < K) {
            float *__restrict__ Sn = s_snp[t] + (size_t)h * D * D;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                gstore_stream(Sn + (size_t)(tr + RG * r) * D + 4 * cg, S[0][r]);
        }
    }
    if (a.write_state) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) gstore_stream(Sg + (size_t)(tr + RG * r) * D + 4 * cg, S[0][r]);
    }
    __syncthreads();   // every output row in LDS

    // --- 4. the gated RMSNorm of every row (whole rows per pass) ---
    for (int i = tid; i < K * SL; i += NT) {
        const int t = i / SL, l = i % SL;
        const float4 lo = reinterpret_cast<const float4 *>(s_o[t])[2 * l];
        const float4 hi = reinterpret_cast<const float4 *>(s_o[t])[2 * l + 1];
        const float xv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const int64_t o0 = (row0 + t) * qkvw + (int64_t)h * D + 8 * l;
        *reinterpret_cast<uint4 *>(a.out + o0) = gated_norm8<D>(
            xv, *reinterpret_cast<const uint4 *>(&s_og[t][8 * l]), nw, a.eps_rms);
    }
    // the conv window after the K rows: entries K-1 .. K+2 of [carried rows
    // 1 .. 3; rows 0 .. K-1], each thread's 8 channels read whole before any
    // is written (every read of the old window above is behind a barrier)
    if (a.write_state) {
        uint16_t *st = const_cast<uint16_t *>(cst);
        for (int i = tid; i < CL; i += NT) {
            const int64_t c = (i / SL) * qkvw + (int64_t)h * D + 8 * (i % SL);
            uint4 win[kConvKC];
#pragma unroll
            for (int jj = 0; jj < kConvKC; ++jj) {
                const int e = K - 1 + jj;
                win[jj] = e < kConvKC - 1 ? gload16(st + (int64_t)(e + 1) * cd + c)
                                          : *reinterpret_cast<const uint4 *>(
                                                a.x + (row0 + e - (kConvKC - 1)) * a.ldx + c);
            }
#pragma unroll
            for (int jj = 0; jj < kConvKC; ++jj) gstore16(st + (int64_t)jj * cd + c, win[jj]);
        }
    }
}

// Compute units of the current device (cached per device).
static int device_cus()
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

hipError_t launch_kda_mixer(const MixerArgs &a0, int B, int head_dim, hipStream_t stream)
{
    if (a0.ks != 1 && a0.ks != kLowRankSplit) return hipErrorInvalidValue;
    MixerArgs a = a0;
    a.B = B;
    // warm-up workgroups: whole rows of H on the CUs the (head, sequence)
    // workgroups leave free (one workgroup fills a CU's LDS), when they are
    // enough to read at most 256 KiB each within the fused kernel's time
    // (measured with 32 heads and a 32 MiB o_proj: 1.3, 1.1, 0.4 and 0.5 us
    // gained at 1, 2, 3 and 4 sequences; at 6, 512 KiB each, 0.9 us lost)
    int rows = 0;
    if (a.warm_w != nullptr && a.warm_bytes > 0 && a.warm_tile_bytes >= 128) {
        const int64_t free_cus = (int64_t)device_cus() - (int64_t)a.H * B;
        if (free_cus > 0) {
            rows = (int)(free_cus / a.H);
            const int64_t used = (int64_t)rows * a.H / 8 * 8;   // workgroups that read
            if (used == 0 || a.warm_bytes > used * (256 << 10)) rows = 0;
        }
    }
    const dim3 grid(a.H, B + rows);
    if (head_dim == 128) {
        if (a.ks == 1)
            hipLaunchKernelGGL((kda_mixer_kernel<128, 1>), grid, dim3(MixerCfg<128>::kThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((kda_mixer_kernel<128, kLowRankSplit>), grid,
                               dim3(MixerCfg<128>::kThreads), 0, stream, a);
    } else {
        if (a.ks == 1)
            hipLaunchKernelGGL((kda_mixer_kernel<16, 1>), grid, dim3(MixerCfg<16>::kThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((kda_mixer_kernel<16, kLowRankSplit>), grid,
                               dim3(MixerCfg<16>::kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D, int NS, int RGT = 1>
static hipError_t recurrent_ns(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                               const float *beta, float *const *state, float *const *snap,
                               float *core, int B, int K, int heads, float scale,
                               bool write_state, const int32_t *n_accept, int32_t *status,
                               hipStream_t stream, float *const *wy = nullptr)
{
    hipLaunchKernelGGL((kda_recurrent_kernel<D, NS, RGT>), dim3(heads * NS, B),
                       dim3(RecCfg<D, NS, RGT>::kThreads), 0, stream, qkv, ldqkv, gate, beta,
                       state, snap, core, K, heads, scale, write_state, n_accept, status, wy);
    return hipGetLastError();
}

// Slices per head: one per CU's worth of (sequence, head) pairs is enough for
// large batches; few pairs get 4 (or 2) slices each.  Every choice gives the
// same bits.
template <int D>
static hipError_t recurrent_t(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                              const float *beta, float *const *state, float *const *snap,
                              float *core, int B, int K, int heads, float scale, bool write_state,
                              const int32_t *n_accept, int32_t *status, hipStream_t stream,
                              float *const *wy = nullptr)
{
    const int64_t pairs = (int64_t)B * heads;
    if constexpr (D >= 128) {
        if (pairs <= 128)
            return recurrent_ns<D, 4>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads, scale,
                                      write_state, n_accept, status, stream, wy);
        if (pairs <= 256)
            return recurrent_ns<D, 2>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads, scale,
                                      write_state, n_accept, status, stream, wy);
    }
    // whole heads: the write-on-accept verify (state read only) and fold run
    // two row groups per thread (256 threads, more state in flight per CU);
    // decode and decode_k keep one (512 threads), measured faster for them
    if constexpr (D >= 128)
        if (!write_state || n_accept)
            return recurrent_ns<D, 1, 2>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads,
                                         scale, write_state, n_accept, status, stream, wy);
    return recurrent_ns<D, 1>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads, scale,
                              write_state, n_accept, status, stream, wy);
}

hipError_t launch_kda_recurrent(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                const float *beta, float *const *state, float *const *snap,
                                float *core, int B, int K, int heads, int head_dim,
                                float scale, hipStream_t stream)
{
    return head_dim == 128
               ? recurrent_t<128>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads, scale,
                                  true, nullptr, nullptr, stream)
               : recurrent_t<16>(qkv, ldqkv, gate, beta, state, snap, core, B, K, heads, scale,
                                 true, nullptr, nullptr, stream);
}

hipError_t launch_kda_verify(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                             const float *beta, float *const *state, float *core, int B, int K,
                             int heads, int head_dim, float scale, hipStream_t stream)
{
    return head_dim == 128
               ? recurrent_t<128>(qkv, ldqkv, gate, beta, state, nullptr, core, B, K, heads,
                                  scale, false, nullptr, nullptr, stream)
               : recurrent_t<16>(qkv, ldqkv, gate, beta, state, nullptr, core, B, K, heads,
                                 scale, false, nullptr, nullptr, stream);
}

hipError_t launch_kda_verify_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                const float *beta, float *const *state, float *const *wy,
                                float *core, int B, int K, int heads, int head_dim, float scale,
                                hipStream_t stream)
{
    return head_dim == 128
               ? recurrent_t<128>(qkv, ldqkv, gate, beta, state, nullptr, core, B, K, heads,
                                  scale, false, nullptr, nullptr, stream, wy)
               : recurrent_t<16>(qkv, ldqkv, gate, beta, state, nullptr, core, B, K, heads,
                                 scale, false, nullptr, nullptr, stream, wy);
}

// Table-form fold ("Glm5NextLayer" page, LayerWriteOnAccept: gdn_fold_accepted
// over the verify's WY tables).  Unrolling the recurrence over the first n
// rows of a sequence,
//   S_n = diag(e^{g_{n-1}}) .. diag(e^{g_0}) S_0
//         + sum_{s<n} diag(e^{g_{n-1}}) .. diag(e^{g_{s+1}}) k_s u_s^T,
// so with the verify's u rows (the table) the accepted rows fold into the
// state in one pass: per key channel i, with the decays summed from the last
// row down (sigma_s = g_{s+1} + .. + g_{n-1}, sigma_{-1} the whole sum),
//   S[i][j] = e^{sigma_{-1}[i]} S_0[i][j], then for s = n-1 .. 0:
//   S[i][j] += (e^{sigma_s[i]} k_s[i]) u_s[j]        (one fma, in that order).
// One workgroup per (head, value-column slice, sequence), the decode's
// thread layout; the accepted rows go through LDS in blocks of kFoldRows.
constexpr int kFoldRows = 16;

template <int D, int NS>
__global__ __launch_bounds__((RecCfg<D, NS, 1>::kThreads)) void kda_fold_wy_kernel(
    const uint16_t *__restrict__ qkv, int64_t ldqkv, const float *__restrict__ gate,
    float *const *__restrict__ state, float *const *__restrict__ wy,
    const int32_t *__restrict__ n_accept, int K, int H, int32_t *__restrict__ status)
{
    using Cfg = RecCfg<D, NS, 1>;
    constexpr int CG = Cfg::kCG, RG = Cfg::kRG, RPT = Cfg::kRPT, NT = Cfg::kThreads;
    static_assert(NT >= D, "one thread per key channel for the decay sums");
    const int h = blockIdx.x / NS;
    const int c0 = (blockIdx.x % NS) * Cfg::kDC;
    const int b = blockIdx.y;
    const int tid = threadIdx.x, cg = tid % CG, tr = tid / CG;
    const int na = n_accept[b];
    if (status != nullptr && (na < 0 || na > K) && blockIdx.x == 0 && tid == 0)
        atomicOr(status, kReportAcceptClamped);
    const int n = min(max(na, 0), K);
    if (n == 0) return;   // uniform over the workgroup

    __shared__ float s_a[kFoldRows][D];          // e^{sigma_s} k_s, per key channel
    __shared__ float s_e[D];                     // e^{sigma_{-1}}
    __shared__ float4 s_u[kFoldRows][CG];        // u_s, this slice's columns
    const int64_t qkvw = (int64_t)H * D;
    const float *__restrict__ u_tab = wy[b] + (size_t)h * K * D + c0;

    if (tid < D) {   // the whole decay sum, from the last accepted row down
        float sg = 0.f;
        for (int s = n - 1; s >= 0; --s) sg += gate[(((size_t)b * K + s) * H + h) * D + tid];
        s_e[tid] = exp2_fast(sg * kLog2e);
    }
    float *__restrict__ Sg = state[b] + (size_t)h * D * D + c0;
    float4 S[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = load_stream(Sg + (size_t)(tr + RG * r) * D + 4 * cg);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float e = s_e[tr + RG * r];
        S[r] = make_float4(S[r].x * e, S[r].y * e, S[r].z * e, S[r].w * e);
    }

    float sig = 0.f;   // sigma_s of the row being tabulated (channel tid)
    for (int s1 = n; s1 > 0; s1 -= kFoldRows) {
        const int s0 = max(0, s1 - kFoldRows);
        __syncthreads();   // the previous block's table reads are done
        if (tid < D) {
            for (int s = s1 - 1; s >= s0; --s) {
                const size_t row = (size_t)b * K + s;
                const float k = bf16_to_f32(qkv[row * ldqkv + qkvw + (int64_t)h * D + tid]);
                s_a[s - s0][tid] = exp2_fast(sig * kLog2e) * k;
                sig += gate[(row * H + h) * D + tid];
            }
        }
        for (int idx = tid; idx < (s1 - s0) * CG; idx += NT) {
            const int s = s0 + idx / CG, c = idx % CG;
            s_u[s - s0][c] = reinterpret_cast<const float4 *>(u_tab + (size_t)s * D)[c];
        }
        __syncthreads();
        for (int s = s1 - 1; s >= s0; --s) {
            const float4 u = s_u[s - s0][cg];
#pragma unroll
            for (int r = 0; r < RPT; ++r) S[r] = fma4(s_a[s - s0][tr + RG * r], u, S[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) store_stream(Sg + (size_t)(tr + RG * r) * D + 4 * cg, S[r]);
}

template <int D>
static hipError_t fold_wy_t(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                            float *const *state, float *const *wy, const int32_t *n_accept, int B,
                            int K, int heads, int32_t *status, hipStream_t stream)
{
    const int64_t pairs = (int64_t)B * heads;
    auto go = [&](auto ns) {
        constexpr int NS = decltype(ns)::value;
        hipLaunchKernelGGL((kda_fold_wy_kernel<D, NS>), dim3(heads * NS, B),
                           dim3(RecCfg<D, NS, 1>::kThreads), 0, stream, qkv, ldqkv, gate, state,
                           wy, n_accept, K, heads, status);
        return hipGetLastError();
    };
    if constexpr (D >= 128) {
        if (pairs <= 128) return go(std::integral_constant<int, 4>{});
        if (pairs <= 256) return go(std::integral_constant<int, 2>{});
    }
    return go(std::integral_constant<int, 1>{});
}

hipError_t launch_kda_fold_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                              float *const *state, float *const *wy, const int32_t *n_accept,
                              int B, int K, int heads, int head_dim, int32_t *status,
                              hipStream_t stream)
{
    return head_dim == 128
               ? fold_wy_t<128>(qkv, ldqkv, gate, state, wy, n_accept, B, K, heads, status, stream)
               : fold_wy_t<16>(qkv, ldqkv, gate, state, wy, n_accept, B, K, heads, status, stream);
}

hipError_t launch_kda_fold(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                           const float *beta, float *const *state, const int32_t *n_accept,
                           int B, int K, int heads, int head_dim, int32_t *status,
                           hipStream_t stream)
{
    return head_dim == 128
               ? recurrent_t<128>(qkv, ldqkv, gate, beta, state, nullptr, nullptr, B, K, heads,
                                  1.f, true, n_accept, status, stream)
               : recurrent_t<16>(qkv, ldqkv, gate, beta, state, nullptr, nullptr, B, K, heads,
                                 1.f, true, n_accept, status, stream);
}

}  // namespace kda
