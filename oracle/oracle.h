/*
 * oracle.h -- declarations of the CPU reference (test infrastructure only).
 * All tensors are row-major double arrays; shapes as in oracle.c.
 */
#ifndef DTB_ORACLE_H
#define DTB_ORACLE_H

#define ORC_NORM_RMS 0
#define ORC_NORM_RMS_NOGAMMA 1
#define ORC_NORM_LAYER 2

#define ORC_MLP_SWIGLU 0
#define ORC_MLP_RELU 1
#define ORC_MLP_GELU 2

#define ORC_ROPE_NONE 0
#define ORC_ROPE_NEOX 1

typedef struct {
    int B, T, C, NH, NKV, H;
    int norm, mlp, rope;
    double rope_base, eps;
    int qkv_bias, o_bias, mlp_bias;
} orc_cfg;

/* g1/b1: norm1 gamma/beta [C]; wqkv [QKV,C]; bqkv [QKV]; wo [C,C]; bo [C];
 * g2/b2 [C]; w_up [2H,C] (gate rows then up rows) or [H,C]; b_up; w_down [C,H]; b_down [C] */
typedef struct {
    const double *g1, *b1, *wqkv, *bqkv, *wo, *bo, *g2, *b2, *w_up, *b_up, *w_down, *b_down;
} orc_weights;

typedef struct {
    double *g1, *b1, *wqkv, *bqkv, *wo, *bo, *g2, *b2, *w_up, *b_up, *w_down, *b_down;
} orc_grads;

/* intermediates of the forward: n1 [BT,C], r1/mu1 [BT], qkv [BT,QKV] (after
 * RoPE), o [BT,C], lse [B,NH,T], x2 [BT,C], n2 [BT,C], r2/mu2 [BT],
 * up [BT,2H or H] (pre-activation), h [BT,H] */
typedef struct {
    double *n1, *r1, *mu1, *qkv, *o, *lse, *x2, *n2, *r2, *mu2, *up, *h;
} orc_saved;

void orc_norm_forward(int mode, const double *x, const double *g, const double *b,
                      double eps, long R, int C, double *out, double *rstd, double *mean);
void orc_norm_backward(int mode, const double *dy, const double *x, const double *g,
                       const double *rstd, const double *mean, long R, int C,
                       double *dx, double *dg, double *db);
void orc_linear_forward(const double *inp, const double *w, const double *bias,
                        long R, int K, int N, double *out);
void orc_linear_backward(const double *dout, const double *inp, const double *w,
                         long R, int K, int N, double *dinp, double *dw, double *dbias);
void orc_rope(double *buf, int B, int T, int stride, int off, int nheads, int hd,
              double base, int inverse);
void orc_attn_forward(const double *qkv, int B, int T, int C, int NH, int NKV,
                      double *out, double *lse);
void orc_attn_backward(const double *qkv, const double *dout, int B, int T, int C, int NH,
                       int NKV, double *dqkv);
void orc_attn_forward_materialized(const double *qkv, int B, int T, int C, int NH, int NKV,
                                   double *out, double *att);
void orc_attn_backward_materialized(const double *qkv, const double *att, const double *dout,
                                    int B, int T, int C, int NH, int NKV, double *dqkv);
void orc_attn_tail(const double *q_tail, const double *k, const double *v, const double *dout_tail,
                   int T, int R, int NH, int NKV, int hd, double *o_tail, double *lse_tail,
                   double *dq_tail, double *dk_tail, double *dv_tail);
void orc_attn_decode(const double *q, const double *kc, const double *vc, const int *lens, int B,
                     int NH, int NKV, int hd, int Tmax, double *out, double *lse);
void orc_act_forward(int mlp, const double *up, long R, int H, double *h);
void orc_act_backward(int mlp, const double *dh, const double *up, long R, int H, double *dup);
void orc_block_forward(const orc_cfg *c, const orc_weights *w, const double *x, double *y,
                       orc_saved *sv);
void orc_block_backward(const orc_cfg *c, const orc_weights *w, const double *x,
                        const orc_saved *sv, const double *dy, double *dx, orc_grads *gr);
void orc_embed_forward(const int *ids, const double *wte, const double *wpe, int B, int T, int C,
                       double *x);
void orc_embed_backward(const int *ids, const double *dx, int B, int T, int C, double *dwte,
                        double *dwpe);
double orc_softmax_ce(const double *logits, const int *targets, long R, int V, double scale,
                      double *dlogits, double *row_loss);
void orc_adamw(double *p, const double *g, double *m, double *v, long n, double lr, double b1,
               double b2, double eps, double wd, int t);
int orc_num_threads(void);
void orc_set_num_threads(int n);

#endif
