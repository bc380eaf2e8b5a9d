/*
 * oracle.c -- plain, slow CPU reference for one pre-norm decoder block,
 * forward and backward, and for causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library; the two meet only through the seeded
 * input generator.
 *
 * Everything is evaluated straight from the definitions in double precision:
 * inputs arrive as doubles (fp32 / bf16 values widened exactly), every sum is
 * accumulated in double in a fixed sequential order, and nothing is blocked,
 * fused or reordered beyond what the definitions state.  OpenMP only splits
 * independent outputs across threads, so results do not depend on the thread
 * count.
 *
 * Sources (page title, section):
 *   "nanoeuler — CUDA kernels": rmsnorm_cpu_fwd / rmsnorm_cpu_bwd,
 *       matmul_cpu / matmul_backward_cpu, rope_cpu (the inverse rotation for
 *       the backward), attention_cpu_fwd / attention_cpu_bwd (causal GQA,
 *       kv head = h / (NH/NKV), scale 1/sqrt(hs)), swiglu_cpu_fwd/bwd,
 *       residual_add_kernel, the flash_attn_* declarations (packed qkv in,
 *       out + lse out; dqkv from qkv, out, dout, lse).
 *   "microgpt.cu": rmsnorm without gamma, relu_forward/backward_kernel,
 *       forward_position (pre-norm block with ReLU MLP), attention_backward
 *       (dS = P * (dP - sum P dP)).
 *   "nx_f32_qwen2_train_gate.nx source": build_rope / rope_node (NeoX
 *       half-split rotation, theta_i = base^(-2i/D)), rmsnorm_gamma, QKV bias
 *       added before RoPE, SwiGLU MLP.
 *   llm.c train_gpt2.c (embedded in the rummy 2.2.0 package-diff page):
 *       layernorm_forward / layernorm_backward, matmul_forward / backward with
 *       bias, gelu_forward / gelu_backward (tanh approximation), residual.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>

/* Thread teams only for loops with enough work: small calls (the unit
 * tests' finite differences) would otherwise be dominated by team start-up.
 * Every output is still computed by one thread in a fixed order, so the
 * results do not depend on this choice. */
#define ORC_PARALLEL(work) ((work) >= 65536.0)
#endif

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* norms                                                                      */
/* ------------------------------------------------------------------------ */

/* RMSNorm (nanoeuler rmsnorm_cpu_fwd; microgpt rmsnorm without gamma):
 *   r = (mean_i x_i^2 + eps)^(-1/2),  y_i = x_i * r * gamma_i.
 * LayerNorm (llm.c layernorm_forward):
 *   mu = mean_i x_i, var = mean_i (x_i - mu)^2 (biased),
 *   r = (var + eps)^(-1/2),  y_i = (x_i - mu) * r * w_i + b_i.
 * Writes rstd[r] and (LayerNorm) mean[r]. */
void orc_norm_forward(int mode, const double *x, const double *g, const double *b,
                      double eps, long R, int C, double *out, double *rstd, double *mean)
{
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * C))
    for (long r = 0; r < R; r++) {
        const double *xr = x + r * C;
        double mu = 0.0;
        if (mode == ORC_NORM_LAYER) {
            for (int i = 0; i < C; i++) mu += xr[i];
            mu /= C;
        }
        double ss = 0.0;
        for (int i = 0; i < C; i++) {
            double d = xr[i] - mu;
            ss += d * d;
        }
        double rs = 1.0 / sqrt(ss / C + eps);
        for (int i = 0; i < C; i++) {
            double n = (xr[i] - mu) * rs;
            if (mode != ORC_NORM_RMS_NOGAMMA) n *= g[i];
            if (mode == ORC_NORM_LAYER) n += b[i];
            out[r * C + i] = n;
        }
        rstd[r] = rs;
        if (mean) mean[r] = mu;
    }
}

/* Backward of the norms; dx, dg, db are ACCUMULATED (+=), as the pages do
 * (nanoeuler rmsnorm_cpu_bwd, llm.c layernorm_backward).  Both norms are
 * n = xhat g (+ b) with xhat = (x - mu) r, r = (var + eps)^(-1/2): for RMS,
 * mu = 0 and var = mean(x^2); for LayerNorm, mu = mean(x) and var the biased
 * variance.  With dxhat = g dy (g = 1 without gamma), the chain rule through
 * r (and mu) gives
 *   RMS:        dx_i += r (dxhat_i - xhat_i mean_j(dxhat_j xhat_j))
 *   LayerNorm:  dx_i += r (dxhat_i - mean_j(dxhat_j) - xhat_i mean_j(dxhat_j xhat_j))
 * (d r / d x_j = -r^3 (x_j - mu) / C; for LayerNorm d mu / d x_j = 1/C adds the
 * mean(dxhat) term), and dg_i += sum over rows of dy_i xhat_i, db_i += sum dy_i. */
void orc_norm_backward(int mode, const double *dy, const double *x, const double *g,
                       const double *rstd, const double *mean, long R, int C,
                       double *dx, double *dg, double *db)
{
    const int layer = mode == ORC_NORM_LAYER, has_g = mode != ORC_NORM_RMS_NOGAMMA;
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * C))
    for (long r = 0; r < R; r++) {
        const double *xr = x + r * C, *dyr = dy + r * C;
        double *dxr = dx + r * C;
        const double rs = rstd[r], mu = layer ? mean[r] : 0.0;
        double m_dxh = 0.0, m_dxh_xh = 0.0;    /* mean(dxhat), mean(dxhat xhat) */
        for (int i = 0; i < C; i++) {
            double xh = (xr[i] - mu) * rs;
            double dxh = (has_g ? g[i] : 1.0) * dyr[i];
            m_dxh += dxh;
            m_dxh_xh += dxh * xh;
        }
        m_dxh /= C;
        m_dxh_xh /= C;
        if (!layer) m_dxh = 0.0;    /* RMS: no mean is subtracted */
        for (int i = 0; i < C; i++) {
            double xh = (xr[i] - mu) * rs;
            double dxh = (has_g ? g[i] : 1.0) * dyr[i];
            dxr[i] += rs * (dxh - m_dxh - xh * m_dxh_xh);
        }
    }
    if (mode == ORC_NORM_RMS_NOGAMMA) return;
    /* parameter gradients: one thread per column, rows summed in order */
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * C))
    for (int i = 0; i < C; i++) {
        double sg = 0.0, sb = 0.0;
        for (long r = 0; r < R; r++) {
            double xh = (x[r * C + i] - (mode == ORC_NORM_LAYER ? mean[r] : 0.0)) * rstd[r];
            sg += dy[r * C + i] * xh;
            sb += dy[r * C + i];
        }
        dg[i] += sg;
        if (mode == ORC_NORM_LAYER) db[i] += sb;
    }
}

/* ------------------------------------------------------------------------ */
/* linear layers (weights row-major [out, in])                               */
/* ------------------------------------------------------------------------ */

/* Loop structure of the linear layers: every output is one sum over its
 * contraction index, taken in increasing order, accumulated in double.  For
 * memory locality only (no change to any sum), blocks of ORC_RB rows or
 * outputs advance together through one pass over the shared operand, and the
 * forward reads a transposed copy of w, so that the innermost loop runs over
 * contiguous outputs. */
#define ORC_RB 8
#define ORC_KT 256

/* out[r,o] = sum_i inp[r,i] w[o,i] (+ bias[o])   (nanoeuler matmul_cpu; llm.c
 * matmul_forward).  Each output's sum runs over i in order. */
void orc_linear_forward(const double *inp, const double *w, const double *bias,
                        long R, int K, int N, double *out)
{
    double *wt = (double *)malloc(sizeof(double) * (size_t)K * N);   /* wt[i][o] = w[o][i] */
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)K * N))
    for (int i = 0; i < K; i++)
        for (int o = 0; o < N; o++) wt[(size_t)i * N + o] = w[(size_t)o * K + i];
    const long nblk = (R + ORC_RB - 1) / ORC_RB;
    #pragma omp parallel if(ORC_PARALLEL((double)R * K * N))
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)ORC_RB * N);
        #pragma omp for schedule(static)
        for (long blk = 0; blk < nblk; blk++) {
            const long r0 = blk * ORC_RB;
            const int nr = (int)(R - r0 < ORC_RB ? R - r0 : ORC_RB);
            for (long e = 0; e < (long)nr * N; e++) acc[e] = 0.0;
            for (int i = 0; i < K; i++) {
                const double *wi = wt + (size_t)i * N;
                for (int rr = 0; rr < nr; rr++) {
                    const double xi = inp[(r0 + rr) * K + i];
                    double *a = acc + (size_t)rr * N;
                    for (int o = 0; o < N; o++) a[o] += xi * wi[o];
                }
            }
            for (int rr = 0; rr < nr; rr++)
                for (int o = 0; o < N; o++)
                    out[(r0 + rr) * N + o] = acc[(size_t)rr * N + o] + (bias ? bias[o] : 0.0);
        }
        free(acc);
    }
    free(wt);
}

/* dinp[r,i] += sum_o dout[r,o] w[o,i];  dw[o,i] += sum_r dout[r,o] inp[r,i];
 * dbias[o] += sum_r dout[r,o]   (nanoeuler matmul_backward_cpu; llm.c
 * matmul_backward).  Any of dinp, dw, dbias may be NULL.  Each sum runs over
 * o (dinp) or r (dw, dbias) in order. */
void orc_linear_backward(const double *dout, const double *inp, const double *w,
                         long R, int K, int N, double *dinp, double *dw, double *dbias)
{
    if (dinp) {
        const long nblk = (R + ORC_RB - 1) / ORC_RB;
        #pragma omp parallel if(ORC_PARALLEL((double)R * K * N))
        {
            double *acc = (double *)malloc(sizeof(double) * (size_t)ORC_RB * K);
            #pragma omp for schedule(static)
            for (long blk = 0; blk < nblk; blk++) {
                const long r0 = blk * ORC_RB;
                const int nr = (int)(R - r0 < ORC_RB ? R - r0 : ORC_RB);
                for (long e = 0; e < (long)nr * K; e++) acc[e] = 0.0;
                for (int o = 0; o < N; o++) {
                    const double *wr = w + (size_t)o * K;
                    for (int rr = 0; rr < nr; rr++) {
                        const double d = dout[(r0 + rr) * N + o];
                        double *a = acc + (size_t)rr * K;
                        for (int i = 0; i < K; i++) a[i] += d * wr[i];
                    }
                }
                for (int rr = 0; rr < nr; rr++)
                    for (int i = 0; i < K; i++) dinp[(r0 + rr) * K + i] += acc[(size_t)rr * K + i];
            }
            free(acc);
        }
    }
    if (dbias) {
        #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * N))
        for (int o = 0; o < N; o++) {
            double sb = 0.0;
            for (long r = 0; r < R; r++) sb += dout[r * N + o];
            dbias[o] += sb;
        }
    }
    if (dw) {
        /* tiles of ORC_RB outputs x ORC_KT input columns (the accumulator tile
         * stays in the first-level cache) */
        const int nob = (N + ORC_RB - 1) / ORC_RB, nkt = (K + ORC_KT - 1) / ORC_KT;
        #pragma omp parallel for schedule(static) collapse(2) if(ORC_PARALLEL((double)R * K * N))
        for (int blk = 0; blk < nob; blk++)
            for (int kt = 0; kt < nkt; kt++) {
                const int o0 = blk * ORC_RB, i0 = kt * ORC_KT;
                const int no = N - o0 < ORC_RB ? N - o0 : ORC_RB;
                const int ni = K - i0 < ORC_KT ? K - i0 : ORC_KT;
                double acc[ORC_RB * ORC_KT];
                for (int e = 0; e < no * ORC_KT; e++) acc[e] = 0.0;
                for (long r = 0; r < R; r++) {
                    const double *xr = inp + r * K + i0;
                    for (int oo = 0; oo < no; oo++) {
                        const double d = dout[r * N + o0 + oo];
                        double *a = acc + oo * ORC_KT;
                        for (int i = 0; i < ni; i++) a[i] += d * xr[i];
                    }
                }
                for (int oo = 0; oo < no; oo++)
                    for (int i = 0; i < ni; i++) dw[(size_t)(o0 + oo) * K + i0 + i] += acc[oo * ORC_KT + i];
            }
    }
}

/* ------------------------------------------------------------------------ */
/* NeoX rotary embedding                                                      */
/* ------------------------------------------------------------------------ */

/* NeoX half-split RoPE (nx_f32_qwen2_train_gate build_rope / rope_node):
 * pairs (i, i + hd/2), theta_i = base^(-2i/hd), angle = t * theta_i with t the
 * position inside the sequence.
 *   forward: x' = x cos - y sin,  y' = y cos + x sin
 *   inverse (the transposed rotation, used for the backward as nanoeuler's
 *   rope_cpu does with inverse=1): x' = x cos + y sin,  y' = -x sin + y cos.
 * Applied in place to `nheads` heads of width hd starting at column `off` of
 * rows of width `stride`. */
void orc_rope(double *buf, int B, int T, int stride, int off, int nheads, int hd,
              double base, int inverse)
{
    int half = hd / 2;
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)B * T * nheads * hd))
    for (long bt = 0; bt < (long)B * T; bt++) {
        int t = (int)(bt % T);
        for (int h = 0; h < nheads; h++) {
            double *v = buf + bt * stride + off + (long)h * hd;
            for (int i = 0; i < half; i++) {
                double theta = pow(base, -2.0 * i / hd);
                double ang = t * theta;
                double c = cos(ang), s = sin(ang);
                double x = v[i], y = v[i + half];
                if (!inverse) {
                    v[i] = x * c - y * s;
                    v[i + half] = y * c + x * s;
                } else {
                    v[i] = x * c + y * s;
                    v[i + half] = -x * s + y * c;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* causal grouped-query attention                                             */
/* ------------------------------------------------------------------------ */
/* qkv row (b,t) = [q heads (NH*hd) | k heads (NKV*hd) | v heads (NKV*hd)];
 * query head h reads kv head h / (NH/NKV); scale = 1/sqrt(hd) applied to
 * q.k; key j is visible to query t iff j <= t (nanoeuler attention_cpu_fwd). */

static void scores_row(const double *qkv, int b, int t, int h, int T, int C, int NH, int NKV,
                       double *s)
{
    int hd = C / NH, QKV = C + 2 * NKV * hd, kh = h / (NH / NKV);
    double scale = 1.0 / sqrt((double)hd);
    const double *q = qkv + ((long)b * T + t) * QKV + (long)h * hd;
    for (int j = 0; j <= t; j++) {
        const double *k = qkv + ((long)b * T + j) * QKV + C + (long)kh * hd;
        double acc = 0.0;
        for (int d = 0; d < hd; d++) acc += q[d] * k[d];
        s[j] = acc * scale;
    }
}

/* Row-wise form: for each (b, h, t) the scores s_j (j <= t), m = max_j s_j,
 * l = sum_j exp(s_j - m), P_j = exp(s_j - m) / l, o = sum_j P_j v_j and the
 * natural-log logsumexp lse = m + ln l.  out [B,T,C] with head h at columns
 * h*hd; lse [B][NH][T].  No T x T buffer. */
void orc_attn_forward(const double *qkv, int B, int T, int C, int NH, int NKV,
                      double *out, double *lse)
{
    int hd = C / NH, QKV = C + 2 * NKV * hd, kh_div = NH / NKV;
    #pragma omp parallel if(ORC_PARALLEL((double)B * NH * T * T * hd))
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        #pragma omp for schedule(dynamic, 1) collapse(2)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < NH; h++) {
                int kh = h / kh_div;
                for (int t = 0; t < T; t++) {
                    scores_row(qkv, b, t, h, T, C, NH, NKV, s);
                    double m = s[0];
                    for (int j = 1; j <= t; j++) if (s[j] > m) m = s[j];
                    double l = 0.0;
                    for (int j = 0; j <= t; j++) l += exp(s[j] - m);
                    double *o = out + ((long)b * T + t) * C + (long)h * hd;
                    for (int d = 0; d < hd; d++) o[d] = 0.0;
                    for (int j = 0; j <= t; j++) {
                        double p = exp(s[j] - m) / l;
                        const double *v = qkv + ((long)b * T + j) * QKV + C + (long)NKV * hd + (long)kh * hd;
                        for (int d = 0; d < hd; d++) o[d] += p * v[d];
                    }
                    if (lse) lse[((long)b * NH + h) * T + t] = m + log(l);
                }
            }
        free(s);
    }
}

/* Row-wise backward, from qkv and dout only (the probabilities are rebuilt from
 * the scores): dP_j = dO . v_j, D = sum_j P_j dP_j, dS_j = P_j (dP_j - D)
 * (the softmax Jacobian, microgpt attention_backward), then
 *   dq_t = scale sum_j dS_j k_j,  dk_j += scale dS_j q_t,  dv_j += P_j dO_t,
 * with dk/dv summed over the NH/NKV query heads that share kv head kh.
 * dqkv is OVERWRITTEN. */
void orc_attn_backward(const double *qkv, const double *dout, int B, int T, int C, int NH,
                       int NKV, double *dqkv)
{
    int hd = C / NH, QKV = C + 2 * NKV * hd, grp = NH / NKV;
    double scale = 1.0 / sqrt((double)hd);
    memset(dqkv, 0, sizeof(double) * (size_t)B * T * QKV);
    #pragma omp parallel if(ORC_PARALLEL((double)B * NH * T * T * hd))
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double *p = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        /* one thread owns (b, kh): it writes dk/dv of that kv head and dq of
         * the group's query heads */
        #pragma omp for schedule(dynamic, 1) collapse(2)
        for (int b = 0; b < B; b++)
            for (int kh = 0; kh < NKV; kh++)
                for (int h = kh * grp; h < (kh + 1) * grp; h++)
                    for (int t = 0; t < T; t++) {
                        scores_row(qkv, b, t, h, T, C, NH, NKV, s);
                        double m = s[0];
                        for (int j = 1; j <= t; j++) if (s[j] > m) m = s[j];
                        double l = 0.0;
                        for (int j = 0; j <= t; j++) l += exp(s[j] - m);
                        const double *dO = dout + ((long)b * T + t) * C + (long)h * hd;
                        const double *q = qkv + ((long)b * T + t) * QKV + (long)h * hd;
                        double D = 0.0;
                        for (int j = 0; j <= t; j++) {
                            p[j] = exp(s[j] - m) / l;
                            const double *v = qkv + ((long)b * T + j) * QKV + C + (long)NKV * hd + (long)kh * hd;
                            double acc = 0.0;
                            for (int d = 0; d < hd; d++) acc += dO[d] * v[d];
                            dp[j] = acc;
                            D += p[j] * dp[j];
                        }
                        double *dq = dqkv + ((long)b * T + t) * QKV + (long)h * hd;
                        for (int j = 0; j <= t; j++) {
                            double ds = p[j] * (dp[j] - D);
                            long row = ((long)b * T + j) * QKV;
                            const double *k = qkv + row + C + (long)kh * hd;
                            double *dk = dqkv + row + C + (long)kh * hd;
                            double *dv = dqkv + row + C + (long)NKV * hd + (long)kh * hd;
                            for (int d = 0; d < hd; d++) {
                                dq[d] += scale * ds * k[d];
                                dk[d] += scale * ds * q[d];
                                dv[d] += p[j] * dO[d];
                            }
                        }
                    }
        free(s);
        free(p);
        free(dp);
    }
}

/* Materialised form for brute-force cross-checks on tiny T (nanoeuler
 * attention_cpu_fwd / attention_cpu_bwd): explicit preatt and att [B,NH,T,T]
 * with zeros above the diagonal, and a backward through the full softmax
 * Jacobian dpre_j = sum_k a_k (delta_jk - a_j) datt_k.  att must hold
 * B*NH*T*T doubles; dqkv is OVERWRITTEN. */
void orc_attn_forward_materialized(const double *qkv, int B, int T, int C, int NH, int NKV,
                                   double *out, double *att)
{
    int hd = C / NH, QKV = C + 2 * NKV * hd, grp = NH / NKV;
    double scale = 1.0 / sqrt((double)hd);
    double *pre = (double *)malloc(sizeof(double) * (size_t)B * NH * T * T);
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                int kh = h / grp;
                long base = (((long)b * NH + h) * T + t) * T;
                const double *q = qkv + ((long)b * T + t) * QKV + (long)h * hd;
                for (int j = 0; j < T; j++) {
                    if (j > t) { pre[base + j] = 0.0; continue; }
                    const double *k = qkv + ((long)b * T + j) * QKV + C + (long)kh * hd;
                    double acc = 0.0;
                    for (int d = 0; d < hd; d++) acc += q[d] * k[d];
                    pre[base + j] = acc * scale;
                }
                double m = -INFINITY;
                for (int j = 0; j <= t; j++) if (pre[base + j] > m) m = pre[base + j];
                double sum = 0.0;
                for (int j = 0; j <= t; j++) sum += exp(pre[base + j] - m);
                for (int j = 0; j < T; j++) att[base + j] = (j <= t) ? exp(pre[base + j] - m) / sum : 0.0;
                double *o = out + ((long)b * T + t) * C + (long)h * hd;
                for (int d = 0; d < hd; d++) {
                    double acc = 0.0;
                    for (int j = 0; j < T; j++) {
                        const double *v = qkv + ((long)b * T + j) * QKV + C + (long)NKV * hd + (long)kh * hd;
                        acc += att[base + j] * v[d];
                    }
                    o[d] = acc;
                }
            }
    free(pre);
}

void orc_attn_backward_materialized(const double *qkv, const double *att, const double *dout,
                                    int B, int T, int C, int NH, int NKV, double *dqkv)
{
    int hd = C / NH, QKV = C + 2 * NKV * hd, grp = NH / NKV;
    double scale = 1.0 / sqrt((double)hd);
    double *datt = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double *dpre = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    memset(dqkv, 0, sizeof(double) * (size_t)B * T * QKV);
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                int kh = h / grp;
                const double *a = att + (((long)b * NH + h) * T + t) * T;
                const double *dO = dout + ((long)b * T + t) * C + (long)h * hd;
                for (int j = 0; j < T; j++) {
                    const double *v = qkv + ((long)b * T + j) * QKV + C + (long)NKV * hd + (long)kh * hd;
                    double *dv = dqkv + ((long)b * T + j) * QKV + C + (long)NKV * hd + (long)kh * hd;
                    double acc = 0.0;
                    for (int d = 0; d < hd; d++) {
                        acc += dO[d] * v[d];
                        dv[d] += a[j] * dO[d];
                    }
                    datt[j] = acc;
                }
                for (int j = 0; j < T; j++) {
                    double acc = 0.0;
                    for (int k = 0; k < T; k++) acc += a[k] * ((j == k ? 1.0 : 0.0) - a[j]) * datt[k];
                    dpre[j] = acc;
                }
                const double *q = qkv + ((long)b * T + t) * QKV + (long)h * hd;
                double *dq = dqkv + ((long)b * T + t) * QKV + (long)h * hd;
                for (int j = 0; j <= t; j++) {
                    const double *k = qkv + ((long)b * T + j) * QKV + C + (long)kh * hd;
                    double *dk = dqkv + ((long)b * T + j) * QKV + C + (long)kh * hd;
                    for (int d = 0; d < hd; d++) {
                        dq[d] += dpre[j] * scale * k[d];
                        dk[d] += dpre[j] * scale * q[d];
                    }
                }
            }
    free(datt);
    free(dpre);
}

/* Attention restricted to the last R query rows of ONE sequence (same
 * definition as orc_attn_forward / orc_attn_backward, evaluated on a subset):
 *   q_tail [R][NH*hd]  queries of positions T-R .. T-1
 *   k, v   [T][NKV*hd] keys / values of all positions
 *   dout_tail [R][NH*hd]
 * Outputs o_tail [R][NH*hd], lse_tail [NH][R], dq_tail [R][NH*hd], and
 * dk_tail / dv_tail [R][NKV*hd] for key positions T-R .. T-1.  Causality makes
 * the tail's dk / dv exact: only queries t >= j see key j, and all of them are
 * in the tail. */
void orc_attn_tail(const double *q_tail, const double *k, const double *v, const double *dout_tail,
                   int T, int R, int NH, int NKV, int hd, double *o_tail, double *lse_tail,
                   double *dq_tail, double *dk_tail, double *dv_tail)
{
    int grp = NH / NKV, C = NH * hd, KV = NKV * hd, t0 = T - R;
    double scale = 1.0 / sqrt((double)hd);
    memset(dk_tail, 0, sizeof(double) * (size_t)R * KV);
    memset(dv_tail, 0, sizeof(double) * (size_t)R * KV);
    #pragma omp parallel if(ORC_PARALLEL((double)R * T * NH * hd))
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        double *p = (double *)malloc(sizeof(double) * (size_t)T);
        double *dp = (double *)malloc(sizeof(double) * (size_t)T);
        #pragma omp for schedule(dynamic, 1)
        for (int kh = 0; kh < NKV; kh++)
            for (int h = kh * grp; h < (kh + 1) * grp; h++)
                for (int r = 0; r < R; r++) {
                    int t = t0 + r;
                    const double *q = q_tail + (long)r * C + (long)h * hd;
                    const double *dO = dout_tail + (long)r * C + (long)h * hd;
                    for (int j = 0; j <= t; j++) {
                        const double *kj = k + (long)j * KV + (long)kh * hd;
                        double acc = 0.0;
                        for (int d = 0; d < hd; d++) acc += q[d] * kj[d];
                        s[j] = acc * scale;
                    }
                    double m = s[0];
                    for (int j = 1; j <= t; j++) if (s[j] > m) m = s[j];
                    double l = 0.0;
                    for (int j = 0; j <= t; j++) l += exp(s[j] - m);
                    double *o = o_tail + (long)r * C + (long)h * hd;
                    for (int d = 0; d < hd; d++) o[d] = 0.0;
                    double D = 0.0;
                    for (int j = 0; j <= t; j++) {
                        p[j] = exp(s[j] - m) / l;
                        const double *vj = v + (long)j * KV + (long)kh * hd;
                        double acc = 0.0;
                        for (int d = 0; d < hd; d++) {
                            o[d] += p[j] * vj[d];
                            acc += dO[d] * vj[d];
                        }
                        dp[j] = acc;
                        D += p[j] * dp[j];
                    }
                    lse_tail[(long)h * R + r] = m + log(l);
                    double *dq = dq_tail + (long)r * C + (long)h * hd;
                    for (int d = 0; d < hd; d++) dq[d] = 0.0;
                    for (int j = 0; j <= t; j++) {
                        double ds = p[j] * (dp[j] - D);
                        const double *kj = k + (long)j * KV + (long)kh * hd;
                        for (int d = 0; d < hd; d++) dq[d] += scale * ds * kj[d];
                        if (j >= t0) {
                            double *dk = dk_tail + (long)(j - t0) * KV + (long)kh * hd;
                            double *dv = dv_tail + (long)(j - t0) * KV + (long)kh * hd;
                            for (int d = 0; d < hd; d++) {
                                dk[d] += scale * ds * q[d];
                                dv[d] += p[j] * dO[d];
                            }
                        }
                    }
                }
        free(s);
        free(p);
        free(dp);
    }
}

/* Decode attention ("microgpt.cu": attention_forward_kernel as called from
 * forward_position, where the keys / values of every position so far sit in
 * a per-layer cache and the query of the newest position reads cache rows
 * 0 .. pos_id).  One query per sequence against the first lens[b] rows of
 * its cache:
 *   q [B][NH*hd];  k_cache, v_cache [B][Tmax][NKV*hd] (row t holds kv head
 *   kh at columns kh*hd, as the microgpt cache rows hold all heads of one
 *   position);  s_j = q_h . k_j / sqrt(hd) for j < lens[b] with kh =
 *   h / (NH/NKV);  out [B][NH*hd] = sum_j softmax(s)_j v_j;  lse [B][NH] =
 *   m + ln sum_j exp(s_j - m).
 * An empty cache (lens[b] = 0) gives out = 0 and lse = -inf (an empty sum).
 * Rows at or beyond lens[b] are never read. */
void orc_attn_decode(const double *q, const double *kc, const double *vc, const int *lens, int B,
                     int NH, int NKV, int hd, int Tmax, double *out, double *lse)
{
    int grp = NH / NKV, KV = NKV * hd;
    double scale = 1.0 / sqrt((double)hd);
    #pragma omp parallel if(ORC_PARALLEL((double)B * NH * Tmax * hd))
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
        #pragma omp for schedule(dynamic, 1) collapse(2)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < NH; h++) {
                int kh = h / grp, n = lens[b];
                const double *qh = q + ((long)b * NH + h) * hd;
                const double *kb = kc + (long)b * Tmax * KV + (long)kh * hd;
                const double *vb = vc + (long)b * Tmax * KV + (long)kh * hd;
                double *o = out + ((long)b * NH + h) * hd;
                for (int d = 0; d < hd; d++) o[d] = 0.0;
                if (n <= 0) {
                    lse[(long)b * NH + h] = -INFINITY;
                    continue;
                }
                for (int j = 0; j < n; j++) {
                    double acc = 0.0;
                    for (int d = 0; d < hd; d++) acc += qh[d] * kb[(long)j * KV + d];
                    s[j] = acc * scale;
                }
                double m = s[0];
                for (int j = 1; j < n; j++) if (s[j] > m) m = s[j];
                double l = 0.0;
                for (int j = 0; j < n; j++) l += exp(s[j] - m);
                for (int j = 0; j < n; j++) {
                    double p = exp(s[j] - m) / l;
                    for (int d = 0; d < hd; d++) o[d] += p * vb[(long)j * KV + d];
                }
                lse[(long)b * NH + h] = m + log(l);
            }
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* MLP activations                                                            */
/* ------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static const double GELU_K = 0.7978845608028654; /* sqrt(2/pi) */
static const double GELU_C = 0.044715;

/* up holds [gate | up] (2H columns) for SwiGLU, f (H columns) otherwise.
 *   SwiGLU (nanoeuler swiglu_cpu_fwd): h = g sigma(g) u
 *   ReLU (microgpt relu_forward_kernel): h = f if f > 0 else 0
 *   GELU (llm.c gelu_forward): h = f/2 (1 + tanh(sqrt(2/pi)(f + 0.044715 f^3))) */
void orc_act_forward(int mlp, const double *up, long R, int H, double *h)
{
    int W = (mlp == ORC_MLP_SWIGLU) ? 2 * H : H;
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * H))
    for (long r = 0; r < R; r++)
        for (int j = 0; j < H; j++) {
            double f = up[r * W + j], y;
            if (mlp == ORC_MLP_SWIGLU) y = f * sigmoid(f) * up[r * W + H + j];
            else if (mlp == ORC_MLP_RELU) y = f > 0.0 ? f : 0.0;
            else y = 0.5 * f * (1.0 + tanh(GELU_K * (f + GELU_C * f * f * f)));
            h[r * H + j] = y;
        }
}

/* dup is OVERWRITTEN.
 *   SwiGLU (nanoeuler swiglu_cpu_bwd): dg = dh u sigma(g)(1 + g(1 - sigma(g))), du = dh g sigma(g)
 *   ReLU (microgpt relu_backward_kernel): df = dh if f > 0 else 0 (zero at f = 0)
 *   GELU (llm.c gelu_backward): df = dh [ (1 + tanh u)/2 + f/2 sech^2(u) sqrt(2/pi)(1 + 3 0.044715 f^2) ],
 *        u = sqrt(2/pi)(f + 0.044715 f^3) */
void orc_act_backward(int mlp, const double *dh, const double *up, long R, int H, double *dup)
{
    int W = (mlp == ORC_MLP_SWIGLU) ? 2 * H : H;
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * H))
    for (long r = 0; r < R; r++)
        for (int j = 0; j < H; j++) {
            double d = dh[r * H + j], f = up[r * W + j];
            if (mlp == ORC_MLP_SWIGLU) {
                double u = up[r * W + H + j], sg = sigmoid(f);
                dup[r * W + j] = d * u * sg * (1.0 + f * (1.0 - sg));
                dup[r * W + H + j] = d * f * sg;
            } else if (mlp == ORC_MLP_RELU) {
                dup[r * W + j] = f > 0.0 ? d : 0.0;
            } else {
                double u = GELU_K * (f + GELU_C * f * f * f);
                double th = tanh(u), sech2 = 1.0 - th * th;
                dup[r * W + j] = d * (0.5 * (1.0 + th) + 0.5 * f * sech2 * GELU_K * (1.0 + 3.0 * GELU_C * f * f));
            }
        }
}

/* ------------------------------------------------------------------------ */
/* the block                                                                  */
/* ------------------------------------------------------------------------ */

static void *xcalloc(size_t n) { return calloc(n ? n : 1, sizeof(double)); }

/* Pre-norm block forward:
 *   n1 = Norm1(x);  qkv = n1 Wqkv^T + bqkv;  RoPE(q, k) (after the bias);
 *   o, lse = attention(qkv);  x2 = x + o Wo^T + bo;  n2 = Norm2(x2);
 *   up = n2 Wup^T + bup;  h = act(up);  y = x2 + h Wdown^T + bdown.
 * Every intermediate is written to `sv` (caller-allocated, see orc_saved). */
void orc_block_forward(const orc_cfg *c, const orc_weights *w, const double *x, double *y,
                       orc_saved *sv)
{
    long BT = (long)c->B * c->T;
    int C = c->C, hd = C / c->NH, QKV = C + 2 * c->NKV * hd, H = c->H;
    int W = (c->mlp == ORC_MLP_SWIGLU) ? 2 * H : H;
    orc_norm_forward(c->norm, x, w->g1, w->b1, c->eps, BT, C, sv->n1, sv->r1, sv->mu1);
    orc_linear_forward(sv->n1, w->wqkv, c->qkv_bias ? w->bqkv : NULL, BT, C, QKV, sv->qkv);
    if (c->rope == ORC_ROPE_NEOX) {
        orc_rope(sv->qkv, c->B, c->T, QKV, 0, c->NH, hd, c->rope_base, 0);
        orc_rope(sv->qkv, c->B, c->T, QKV, C, c->NKV, hd, c->rope_base, 0);
    }
    orc_attn_forward(sv->qkv, c->B, c->T, C, c->NH, c->NKV, sv->o, sv->lse);
    orc_linear_forward(sv->o, w->wo, c->o_bias ? w->bo : NULL, BT, C, C, sv->x2);
    for (long i = 0; i < BT * C; i++) sv->x2[i] += x[i];
    orc_norm_forward(c->norm, sv->x2, w->g2, w->b2, c->eps, BT, C, sv->n2, sv->r2, sv->mu2);
    orc_linear_forward(sv->n2, w->w_up, c->mlp_bias ? w->b_up : NULL, BT, C, W, sv->up);
    orc_act_forward(c->mlp, sv->up, BT, H, sv->h);
    orc_linear_forward(sv->h, w->w_down, c->mlp_bias ? w->b_down : NULL, BT, H, C, y);
    for (long i = 0; i < BT * C; i++) y[i] += sv->x2[i];
}

/* Block backward from dy = dL/dy; dx is OVERWRITTEN, every parameter gradient
 * in `gr` is ACCUMULATED (+=); NULL gradient pointers are skipped.
 *   dh = dy Wdown (dWdown, dbdown);  dup = act'(dh);  dn2 = dup Wup (dWup, dbup);
 *   dx2 = dy + Norm2^T(dn2) (dg2, db2);  do = dx2 Wo (dWo, dbo);
 *   dqkv = attention^T(do);  inverse RoPE on dq, dk;  dn1 = dqkv Wqkv (dWqkv, dbqkv);
 *   dx = dx2 + Norm1^T(dn1) (dg1, db1). */
void orc_block_backward(const orc_cfg *c, const orc_weights *w, const double *x,
                        const orc_saved *sv, const double *dy, double *dx, orc_grads *gr)
{
    long BT = (long)c->B * c->T;
    int C = c->C, hd = C / c->NH, QKV = C + 2 * c->NKV * hd, H = c->H;
    int W = (c->mlp == ORC_MLP_SWIGLU) ? 2 * H : H;
    double *dh = (double *)xcalloc((size_t)BT * H);
    double *dup = (double *)xcalloc((size_t)BT * W);
    double *dn2 = (double *)xcalloc((size_t)BT * C);
    double *dx2 = (double *)xcalloc((size_t)BT * C);
    double *dO = (double *)xcalloc((size_t)BT * C);
    double *dqkv = (double *)xcalloc((size_t)BT * QKV);
    double *dn1 = (double *)xcalloc((size_t)BT * C);

    orc_linear_backward(dy, sv->h, w->w_down, BT, H, C, dh, gr->w_down,
                        c->mlp_bias ? gr->b_down : NULL);
    orc_act_backward(c->mlp, dh, sv->up, BT, H, dup);
    orc_linear_backward(dup, sv->n2, w->w_up, BT, C, W, dn2, gr->w_up,
                        c->mlp_bias ? gr->b_up : NULL);
    memcpy(dx2, dy, sizeof(double) * (size_t)BT * C);
    orc_norm_backward(c->norm, dn2, sv->x2, w->g2, sv->r2, sv->mu2, BT, C, dx2, gr->g2, gr->b2);
    orc_linear_backward(dx2, sv->o, w->wo, BT, C, C, dO, gr->wo, c->o_bias ? gr->bo : NULL);
    orc_attn_backward(sv->qkv, dO, c->B, c->T, C, c->NH, c->NKV, dqkv);
    if (c->rope == ORC_ROPE_NEOX) {
        orc_rope(dqkv, c->B, c->T, QKV, 0, c->NH, hd, c->rope_base, 1);
        orc_rope(dqkv, c->B, c->T, QKV, C, c->NKV, hd, c->rope_base, 1);
    }
    orc_linear_backward(dqkv, sv->n1, w->wqkv, BT, C, QKV, dn1, gr->wqkv,
                        c->qkv_bias ? gr->bqkv : NULL);
    memcpy(dx, dx2, sizeof(double) * (size_t)BT * C);
    orc_norm_backward(c->norm, dn1, x, w->g1, sv->r1, sv->mu1, BT, C, dx, gr->g1, gr->b1);

    free(dh); free(dup); free(dn2); free(dx2); free(dO); free(dqkv); free(dn1);
}

/* ------------------------------------------------------------------------ */
/* model harness: embedding, softmax cross-entropy                            */
/* ------------------------------------------------------------------------ */

/* Token (+ position) embedding (llm.c encoder_forward; microgpt
 * forward_position adds wte and wpe rows; nanoeuler encoder_forward_kernel
 * has no position table):  x[b,t,i] = wte[ids[b,t], i] (+ wpe[t, i]).
 * wpe may be NULL. */
void orc_embed_forward(const int *ids, const double *wte, const double *wpe, int B, int T, int C,
                       double *x)
{
    for (long bt = 0; bt < (long)B * T; bt++) {
        int t = (int)(bt % T);
        const double *e = wte + (size_t)ids[bt] * C;
        for (int i = 0; i < C; i++)
            x[bt * C + i] = e[i] + (wpe ? wpe[(size_t)t * C + i] : 0.0);
    }
}

/* Embedding backward (llm.c encoder_backward; nanoeuler encoder_backward_cpu):
 *   dwte[ids[b,t], i] += dx[b,t,i];  dwpe[t, i] += dx[b,t,i].
 * Positions are added in order b, t for every element (threads split the
 * columns i), so repeated ids sum in a fixed order.  dwpe may be NULL. */
void orc_embed_backward(const int *ids, const double *dx, int B, int T, int C, double *dwte,
                        double *dwpe)
{
    long BT = (long)B * T;
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)BT * C))
    for (int i = 0; i < C; i++) {
        for (long bt = 0; bt < BT; bt++) {
            double d = dx[bt * C + i];
            dwte[(size_t)ids[bt] * C + i] += d;
            if (dwpe) dwpe[(size_t)(bt % T) * C + i] += d;
        }
    }
}

/* Softmax cross-entropy of R rows of V logits (nanoeuler softmax_ce_cpu with
 * one head; llm.c crossentropy_forward / crossentropy_softmax_backward):
 *   lse_r = m_r + log sum_v exp(l_rv - m_r),  m_r = max_v l_rv
 *   loss_r = lse_r - l_r,target_r
 *   dlogits_rv = scale * (exp(l_rv - lse_r) - [v == target_r])
 * A row whose target is negative (a masked position) has loss_r = 0 and a
 * zero gradient row.  Returns scale * sum_r loss_r.  row_loss may be NULL. */
double orc_softmax_ce(const double *logits, const int *targets, long R, int V, double scale,
                      double *dlogits, double *row_loss)
{
    double total = 0.0;
    double *rl = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    #pragma omp parallel for schedule(static) if(ORC_PARALLEL((double)R * V))
    for (long r = 0; r < R; r++) {
        const double *l = logits + (size_t)r * V;
        double *dl = dlogits ? dlogits + (size_t)r * V : NULL;
        int tg = targets[r];
        if (tg < 0) {
            rl[r] = 0.0;
            if (dl) for (int v = 0; v < V; v++) dl[v] = 0.0;
            continue;
        }
        double m = l[0];
        for (int v = 1; v < V; v++) if (l[v] > m) m = l[v];
        double s = 0.0;
        for (int v = 0; v < V; v++) s += exp(l[v] - m);
        double lse = m + log(s);
        rl[r] = lse - l[tg];
        if (dl) for (int v = 0; v < V; v++) dl[v] = scale * (exp(l[v] - lse) - (v == tg ? 1.0 : 0.0));
    }
    for (long r = 0; r < R; r++) {
        total += rl[r];
        if (row_loss) row_loss[r] = rl[r];
    }
    free(rl);
    return scale * total;
}

/* ------------------------------------------------------------------------ */
/* optimizer                                                                  */
/* ------------------------------------------------------------------------ */

/* One AdamW step at step number t >= 1 ("nanoeuler — CUDA kernels"
 * adamw_cpu; llm.c gpt2_update; microgpt adam_update_param without decay).
 * The moments are exponential moving averages of g and g^2, each moved a
 * fraction (1 - beta) of the way toward the new value; dividing by
 * 1 - beta^t removes the bias of their zero start; the decay is decoupled
 * (it shrinks the parameter by lr*wd, independently of the moments):
 *   m' = m + (1 - b1)(g - m),   v' = v + (1 - b2)(g^2 - v)
 *   p' = (1 - lr wd) p - lr (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps)
 * In place on p, m, v. */
void orc_adamw(double *p, const double *g, double *m, double *v, long n, double lr, double b1,
               double b2, double eps, double wd, int t)
{
    const double bias1 = 1.0 - pow(b1, t), bias2 = 1.0 - pow(b2, t);
    const double shrink = 1.0 - lr * wd;
    for (long i = 0; i < n; i++) {
        const double gi = g[i];
        m[i] += (1.0 - b1) * (gi - m[i]);
        v[i] += (1.0 - b2) * (gi * gi - v[i]);
        const double step = (m[i] / bias1) / (sqrt(v[i] / bias2) + eps);
        p[i] = shrink * p[i] - lr * step;
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
