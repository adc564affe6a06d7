/*
 * KDA oracle: plain token-serial fp64 reference.  TEST INFRASTRUCTURE ONLY
 * (see kda_oracle.h): the GPU product path never calls it.
 *
 * Written for a reader who checks it against the pages by eye: one loop per
 * step of the definition, no blocking, fusion or reordering, fp64 throughout,
 * BF16 rounding only where the buffer contract stores BF16.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* BF16 rounding.  bfloat16 = fp32's sign and 8-bit exponent with 7 stored   */
/* mantissa bits, i.e. 8 significant bits.  Normal numbers are rounded to    */
/* 8 significant bits; below the smallest normal (2^-126) the spacing is     */
/* fixed at 2^-133.  nearbyint() rounds ties to even in the default mode.    */
/* ------------------------------------------------------------------------ */
double orc_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    const double ax = fabs(x);
    double r;
    if (ax < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(ax, 133)), -133);
    } else {
        int e;
        const double m = frexp(ax, &e); /* ax = m * 2^e, 0.5 <= m < 1 */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
    /* largest finite bfloat16 is (2 - 2^-7) * 2^127 = 255 * 2^120 */
    if (r > ldexp(255.0, 120))
        r = INFINITY;
    return copysign(r, x);
}

void orc_bf16_array(int64_t n, const double *x, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* One projection ("Glm5NextKdaWeights" page: weights in torch Linear        */
/* layout [out, in], BF16): y = x W^T, i.e. y[t][o] = sum_i x[t][i] w[o][i],  */
/* summed in fp64 in index order, then rounded to bf16, since every          */
/* projection output is a BF16 buffer ("Glm5NextKdaWorkspace" page: fields   */
/* qkv_parts, g_raw, out_gate, final_out).                                   */
/* ------------------------------------------------------------------------ */
void orc_linear(int T, int in, int out, const double *x, const double *w, double *y)
{
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < out; ++o) {
            double acc = 0.0;
            for (int i = 0; i < in; ++i)
                acc += x[(size_t)t * in + i] * w[(size_t)o * in + i];
            y[(size_t)t * out + o] = orc_bf16(acc);
        }
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x); above 20 the correction log1p(e^-x) < 2.1e-9
 * relative is dropped, the usual threshold of this activation. */
static double softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }

/* ------------------------------------------------------------------------ */
/* Short causal depthwise conv + SiLU + q/k L2.                               */
/* Reading: the conv weight is a depthwise Conv1d kernel [conv_dim, kc]       */
/* ("Glm5NextKdaWeights" page, field conv); tap j multiplies the input        */
/* kc-1-j rows back, so tap kc-1 meets the current row; no bias.  The state   */
/* is the window of the last kc pre-conv rows, newest last: each row first    */
/* enters the window, then the output is the tap-weighted sum over it.        */
/* SiLU on every channel; then each head of the q and k sections is divided   */
/* by sqrt(sum of squares + eps_l2); v is not normalised ("Glm5NextKdaLayer"  */
/* page, decode: q/k leave the conv already normalised).  One BF16 rounding   */
/* of the final value ("Glm5NextKdaWorkspace" page, field conv_out).          */
/* ------------------------------------------------------------------------ */
void orc_conv_silu_l2(int rows, int heads, int head_dim, int kc, double eps_l2,
                      const double *x, const double *w, double *state,
                      double *snaps, double *y)
{
    const int qkv = heads * head_dim;
    const int conv_dim = 3 * qkv;
    double *s = (double *)malloc(sizeof(double) * (size_t)conv_dim);

    for (int t = 0; t < rows; ++t) {
        /* 1. slide the window: drop the oldest row, append row t */
        for (int j = 0; j + 1 < kc; ++j)
            for (int c = 0; c < conv_dim; ++c)
                state[(size_t)j * conv_dim + c] = state[(size_t)(j + 1) * conv_dim + c];
        for (int c = 0; c < conv_dim; ++c)
            state[(size_t)(kc - 1) * conv_dim + c] = x[(size_t)t * conv_dim + c];

        /* 2. depthwise conv over the window, then SiLU */
        for (int c = 0; c < conv_dim; ++c) {
            double pre = 0.0;
            for (int j = 0; j < kc; ++j)
                pre += w[(size_t)c * kc + j] * state[(size_t)j * conv_dim + c];
            s[c] = pre * sigmoid(pre);
        }

        /* 3. L2 per head over the q section (heads 0..H-1) and the k section
         *    (heads H..2H-1); the v section is left as is */
        for (int blk = 0; blk < 2 * heads; ++blk) {
            double ss = 0.0;
            for (int d = 0; d < head_dim; ++d)
                ss += s[blk * head_dim + d] * s[blk * head_dim + d];
            const double inv = 1.0 / sqrt(ss + eps_l2);
            for (int d = 0; d < head_dim; ++d)
                s[blk * head_dim + d] *= inv;
        }

        /* 4. store as BF16 */
        for (int c = 0; c < conv_dim; ++c)
            y[(size_t)t * conv_dim + c] = orc_bf16(s[c]);

        /* 5. snapshot of the window after row t, for t < rows-1 */
        if (snaps && t < rows - 1)
            memcpy(snaps + (size_t)t * kc * conv_dim, state,
                   sizeof(double) * (size_t)kc * conv_dim);
    }
    free(s);
}

/* ------------------------------------------------------------------------ */
/* kda_gate and beta.                                                         */
/* gate[t,h,d] = -exp(a_log[h]) * softplus(g_raw[t, h*D+d] + dt_bias[h*D+d])  */
/* a_log is per head, dt_bias per channel ("Glm5NextKdaWeights" page, fields  */
/* a_log and dt_bias).  The decay factor exp(gate) lies in (0, 1]: the        */
/* log-decay is bounded above by zero.  beta = sigmoid(b_raw)                 */
/* ("Glm5NextKdaWorkspace" page, field beta).                                 */
/* ------------------------------------------------------------------------ */
void orc_kda_gate(int T, int heads, int head_dim, const double *g_raw,
                  const double *b_raw, const double *a_log,
                  const double *dt_bias, double *gate, double *beta)
{
    const int qkv = heads * head_dim;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < heads; ++h) {
            const double A = exp(a_log[h]);
            for (int d = 0; d < head_dim; ++d) {
                const int c = h * head_dim + d;
                gate[((size_t)t * heads + h) * head_dim + d] =
                    -A * softplus(g_raw[(size_t)t * qkv + c] + dt_bias[c]);
            }
            if (b_raw)
                beta[(size_t)t * heads + h] = sigmoid(b_raw[(size_t)t * heads + h]);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The KDA recurrence, one token at a time.  Per head, with S[i][j] (i = key  */
/* channel, j = value channel), for each token t:                             */
/*   1. decay:   S[i][:] *= exp(g_t[i])          (per-channel, key axis)      */
/*   2. predict: p[j] = sum_i S[i][j] k_t[i]                                  */
/*   3. error:   u[j] = beta_t (v_t[j] - p[j])                                */
/*   4. write:   S[i][j] += k_t[i] u[j]                                       */
/*   5. read:    o_t[j] = scale * sum_i S[i][j] q_t[i]                        */
/* q and k are used as given, never re-normalised ("Glm5NextKdaLayer" page,   */
/* decode).  Prefill is this recurrence from the carried state              */
/* ("Glm5NextKdaLayer" page, prefill); decode_k is it over K rows with a copy */
/* of the state after every row but the last (decode_k).                     */
/* ------------------------------------------------------------------------ */
void orc_kda_recurrence(int T, int heads, int D, int h0, int h1,
                        const double *q, const double *k, const double *v,
                        const double *g, const double *beta, double scale,
                        double *S, double *core, double *snaps)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)D);
    double *u = (double *)malloc(sizeof(double) * (size_t)D);

    for (int t = 0; t < T; ++t) {
        for (int h = h0; h < h1; ++h) {
            double *Sh = S + (size_t)h * D * D;
            const size_t row = ((size_t)t * heads + h) * D;
            const double *qt = q + row, *kt = k + row, *vt = v + row, *gt = g + row;
            const double bt = beta[(size_t)t * heads + h];

            for (int i = 0; i < D; ++i) {                    /* 1 */
                const double a = exp(gt[i]);
                for (int j = 0; j < D; ++j)
                    Sh[(size_t)i * D + j] *= a;
            }
            for (int j = 0; j < D; ++j) {                    /* 2 */
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += Sh[(size_t)i * D + j] * kt[i];
                p[j] = acc;
            }
            for (int j = 0; j < D; ++j)                      /* 3 */
                u[j] = bt * (vt[j] - p[j]);
            for (int i = 0; i < D; ++i)                      /* 4 */
                for (int j = 0; j < D; ++j)
                    Sh[(size_t)i * D + j] += kt[i] * u[j];
            for (int j = 0; j < D; ++j) {                    /* 5 */
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += Sh[(size_t)i * D + j] * qt[i];
                core[row + j] = scale * acc;
            }
            if (snaps && t < T - 1)
                memcpy(snaps + ((size_t)t * heads + h) * D * D, Sh,
                       sizeof(double) * (size_t)D * D);
        }
    }
    free(p);
    free(u);
}

/* ------------------------------------------------------------------------ */
/* Sigmoid-gated RMSNorm per (token, head): normalise by the root mean square */
/* over the head's D channels, multiply by the o_norm weight, then by the     */
/* sigmoid of the low-rank output gate; store BF16 ("Glm5NextKdaWorkspace"    */
/* page, fields out_gate and o_norm_out; "Glm5NextKdaWeights" page, o_norm).  */
/* ------------------------------------------------------------------------ */
void orc_gated_rmsnorm(int T, int heads, int D, double eps, const double *core,
                       const double *out_gate, const double *w, double *out)
{
    const int qkv = heads * D;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < heads; ++h) {
            const double *x = core + ((size_t)t * heads + h) * D;
            double ms = 0.0;
            for (int d = 0; d < D; ++d)
                ms += x[d] * x[d];
            ms /= D;
            const double r = 1.0 / sqrt(ms + eps);
            for (int d = 0; d < D; ++d) {
                const size_t c = (size_t)t * qkv + (size_t)h * D + d;
                out[c] = orc_bf16(x[d] * r * w[d] * sigmoid(out_gate[c]));
            }
        }
    }
}
