/*
 * KDA oracle: plain token-serial fp64 reference of the Kimi-Delta-Attention
 * core and its fused stages.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU product path
 * never links, loads or calls it, and this library shares no code, header,
 * table or helper with the GPU path.
 *
 * Every array is dense, row-major, fp64, owned by the caller.  Values that the
 * documented buffer contract stores in BF16 are rounded with orc_bf16() (round
 * to nearest, ties to even) at exactly those points and nowhere else.
 *
 * Sources (the four API pages of the documented engine):
 *   "Glm5NextKdaWorkspace" page: fields conv_out, q_f32, gate, beta, core,
 *       g_raw, out_gate, o_norm_out (the buffer contract).
 *   "Glm5NextKdaLayer" page: methods decode, decode_k, prefill,
 *       prefill_with_pad_fill.
 *   "Glm5NextKdaWeights" page: fields conv, dt_bias, a_log, o_norm.
 * The pages name the operations but print no formula; each function states
 * the reading it implements.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Round x to the nearest bfloat16 value (8 significant bits, fp32 exponent
 * range, subnormals kept, ties to even, overflow to +-inf) and return that
 * value as a double.  NaN stays NaN. */
double orc_bf16(double x);

/* orc_bf16 applied to each of n values. */
void orc_bf16_array(int64_t n, const double *x, double *out);

/* One projection with torch Linear weights ("Glm5NextKdaWeights" page):
 *   x [T][in], w [out][in]  ->  y [T][out] = bf16(x w^T), fp64 sums. */
void orc_linear(int T, int in, int out, const double *x, const double *w, double *y);

/* Short causal depthwise conv + SiLU + per-head L2 on the q and k sections,
 * for ONE sequence ("Glm5NextKdaWorkspace" page, field conv_out;
 * "Glm5NextKdaWeights" page, field conv).
 *   x      [rows][conv_dim]   pre-conv q|k|v rows
 *   w      [conv_dim][kc]     tap kc-1 multiplies the current row
 *   state  [kc][conv_dim]     in/out: the last kc pre-conv rows, newest last
 *   snaps  [rows-1][kc][conv_dim] or NULL: the window after row t
 *   y      [rows][conv_dim]   bf16-rounded outputs
 * conv_dim = 3*heads*head_dim. */
void orc_conv_silu_l2(int rows, int heads, int head_dim, int kc, double eps_l2,
                      const double *x, const double *w, double *state,
                      double *snaps, double *y);

/* Bounded per-channel log-decay and write strength ("Glm5NextKdaWorkspace"
 * page, fields gate and beta; "Glm5NextKdaWeights" page, fields a_log and
 * dt_bias).
 *   g_raw [T][heads*head_dim], b_raw [T][heads] or NULL
 *   a_log [heads] (per head), dt_bias [heads*head_dim] (per channel)
 *   gate  [T][heads][head_dim], beta [T][heads] (untouched if b_raw is NULL) */
void orc_kda_gate(int T, int heads, int head_dim, const double *g_raw,
                  const double *b_raw, const double *a_log,
                  const double *dt_bias, double *gate, double *beta);

/* Token-serial KDA recurrence for ONE sequence, heads [h0, h1) only
 * ("Glm5NextKdaLayer" page, decode / decode_k / prefill).
 *   q,k,v,g [T][heads][D], beta [T][heads]
 *   S       [heads][D][D] in/out, S[h][i][j]: i = key channel, j = value
 *   core    [T][heads][D]
 *   snaps   [T-1][heads][D][D] or NULL: the state after row t, t < T-1 */
void orc_kda_recurrence(int T, int heads, int D, int h0, int h1,
                        const double *q, const double *k, const double *v,
                        const double *g, const double *beta, double scale,
                        double *S, double *core, double *snaps);

/* Sigmoid-gated RMSNorm per (token, head) ("Glm5NextKdaWorkspace" page,
 * field o_norm_out; "Glm5NextKdaWeights" page, field o_norm).
 *   core [T][heads][D], out_gate [T][heads*D], w [D], out [T][heads*D]
 *   (bf16-rounded). */
void orc_gated_rmsnorm(int T, int heads, int D, double eps, const double *core,
                       const double *out_gate, const double *w, double *out);

#ifdef __cplusplus
}
#endif
#endif
