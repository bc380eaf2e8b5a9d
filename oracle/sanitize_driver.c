/*
 * sanitize_driver.c -- calls every function of the oracle on small seeded
 * inputs, for a build of oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure; built and run by
 * tests/test_oracle_sanitize.py with gcc, on the host only).  Every block
 * configuration (three norms x three activations x RoPE on/off x biases
 * on/off), the attention forms (row-wise, materialised, tail rows, decode
 * with empty and full caches), the harness steps and AdamW.  Buffers are
 * sized exactly, so any read or write past them is reported.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;

static double urand(void) {   /* xorshift64*, uniform in [-1, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

static double *arr(size_t n) {   /* exactly n doubles, filled */
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; i++) p[i] = 0.5 * urand();
    return p;
}

static double *zeros(size_t n) { return (double *)calloc(n ? n : 1, sizeof(double)); }

static void block_case(int norm, int mlp, int rope, int bias) {
    orc_cfg c = {2, 5, 8, 2, 1, 12, norm, mlp, rope, 1e4, 1e-5, bias, bias, bias};
    const int hd = c.C / c.NH, QKV = c.C + 2 * c.NKV * hd, W = mlp == ORC_MLP_SWIGLU ? 2 * c.H : c.H;
    const long BT = (long)c.B * c.T;
    double *g1 = arr(c.C), *b1 = arr(c.C), *wqkv = arr((size_t)QKV * c.C), *bqkv = arr(QKV), *wo = arr(c.C * c.C),
           *bo = arr(c.C), *g2 = arr(c.C), *b2 = arr(c.C), *wup = arr((size_t)W * c.C), *bup = arr(W),
           *wdn = arr((size_t)c.C * c.H), *bdn = arr(c.C);
    orc_weights w = {g1, b1, wqkv, bqkv, wo, bo, g2, b2, wup, bup, wdn, bdn};
    orc_saved sv = {zeros(BT * c.C), zeros(BT), zeros(BT), zeros(BT * QKV), zeros(BT * c.C),
                    zeros((size_t)c.B * c.NH * c.T), zeros(BT * c.C), zeros(BT * c.C), zeros(BT), zeros(BT),
                    zeros(BT * W), zeros(BT * c.H)};
    orc_grads gr = {zeros(c.C), zeros(c.C), zeros((size_t)QKV * c.C), zeros(QKV), zeros(c.C * c.C), zeros(c.C),
                    zeros(c.C), zeros(c.C), zeros((size_t)W * c.C), zeros(W), zeros((size_t)c.C * c.H),
                    zeros(c.C)};
    double *x = arr(BT * c.C), *y = zeros(BT * c.C), *dy = arr(BT * c.C), *dx = zeros(BT * c.C);
    orc_block_forward(&c, &w, x, y, &sv);
    orc_block_backward(&c, &w, x, &sv, dy, dx, &gr);
    double *all[] = {g1, b1, wqkv, bqkv, wo, bo, g2, b2, wup, bup, wdn, bdn, sv.n1, sv.r1, sv.mu1, sv.qkv,
                     sv.o, sv.lse, sv.x2, sv.n2, sv.r2, sv.mu2, sv.up, sv.h, gr.g1, gr.b1, gr.wqkv, gr.bqkv,
                     gr.wo, gr.bo, gr.g2, gr.b2, gr.w_up, gr.b_up, gr.w_down, gr.b_down, x, y, dy, dx};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; i++) free(all[i]);
}

static void attention_cases(void) {
    const int B = 2, T = 7, NH = 4, NKV = 2, hd = 4, C = NH * hd, QKV = C + 2 * NKV * hd;
    double *qkv = arr((size_t)B * T * QKV), *dout = arr((size_t)B * T * C);
    double *o = zeros((size_t)B * T * C), *lse = zeros((size_t)B * NH * T), *dqkv = zeros((size_t)B * T * QKV);
    double *att = zeros((size_t)B * NH * T * T), *dqkv2 = zeros((size_t)B * T * QKV);
    orc_attn_forward(qkv, B, T, C, NH, NKV, o, lse);
    orc_attn_backward(qkv, dout, B, T, C, NH, NKV, dqkv);
    orc_attn_forward_materialized(qkv, B, T, C, NH, NKV, o, att);
    orc_attn_backward_materialized(qkv, att, dout, B, T, C, NH, NKV, dqkv2);
    /* the last R rows of one sequence against all of its keys */
    const int R = 3, KV = NKV * hd;
    double *qt = arr((size_t)R * C), *k = arr((size_t)T * KV), *v = arr((size_t)T * KV), *dot = arr((size_t)R * C);
    double *ot = zeros((size_t)R * C), *lt = zeros((size_t)NH * R), *dqt = zeros((size_t)R * C),
           *dkt = zeros((size_t)R * KV), *dvt = zeros((size_t)R * KV);
    orc_attn_tail(qt, k, v, dot, T, R, NH, NKV, hd, ot, lt, dqt, dkt, dvt);
    /* decode: an empty cache, a partly filled one and a full one */
    const int DB = 3, Tmax = 9;
    int lens[3] = {0, 4, 9};
    double *q = arr((size_t)DB * C), *kc = arr((size_t)DB * Tmax * KV), *vc = arr((size_t)DB * Tmax * KV);
    double *dout1 = zeros((size_t)DB * C), *dl = zeros((size_t)DB * NH);
    orc_attn_decode(q, kc, vc, lens, DB, NH, NKV, hd, Tmax, dout1, dl);
    /* RoPE forward and inverse on the q and k heads of the packed rows */
    orc_rope(qkv, B, T, QKV, 0, NH, hd, 1e4, 0);
    orc_rope(qkv, B, T, QKV, C, NKV, hd, 1e4, 1);
    double *all[] = {qkv, dout, o, lse, dqkv, att, dqkv2, qt, k, v, dot, ot, lt, dqt, dkt, dvt, q, kc, vc, dout1, dl};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; i++) free(all[i]);
}

static void harness_cases(void) {
    const int B = 2, T = 5, C = 8, V = 11;
    int ids[10] = {0, 3, 10, 3, 7, 1, 1, 9, 4, 0};
    int tgt[10] = {3, 10, 3, -1, 2, 1, 9, 4, 0, 5};   /* one masked target */
    double *wte = arr((size_t)V * C), *wpe = arr((size_t)T * C), *x = zeros((size_t)B * T * C);
    double *dwte = zeros((size_t)V * C), *dwpe = zeros((size_t)T * C), *dx = arr((size_t)B * T * C);
    orc_embed_forward(ids, wte, wpe, B, T, C, x);
    orc_embed_backward(ids, dx, B, T, C, dwte, dwpe);
    double *lg = arr((size_t)B * T * V), *dl = zeros((size_t)B * T * V), *rl = zeros((size_t)B * T);
    (void)orc_softmax_ce(lg, tgt, (long)B * T, V, 0.1, dl, rl);
    const long n = 37;
    double *p = arr(n), *g = arr(n), *m = zeros(n), *v = zeros(n);
    for (int t = 1; t <= 3; t++) orc_adamw(p, g, m, v, n, 1e-3, 0.9, 0.95, 1e-8, 0.1, t);
    double *y = zeros((size_t)B * T * C), *rs = zeros((size_t)B * T), *mu = zeros((size_t)B * T);
    double *gg = arr(C), *bb = arr(C), *dg = zeros(C), *db = zeros(C), *dxx = zeros((size_t)B * T * C);
    for (int mode = 0; mode < 3; mode++) {
        orc_norm_forward(mode, x, gg, bb, 1e-5, (long)B * T, C, y, rs, mu);
        orc_norm_backward(mode, dx, x, gg, rs, mu, (long)B * T, C, dxx, dg, db);
    }
    double *h = zeros((size_t)B * T * C), *dup = zeros((size_t)B * T * 2 * C), *up = arr((size_t)B * T * 2 * C);
    for (int mlp = 0; mlp < 3; mlp++) {
        orc_act_forward(mlp, up, (long)B * T, C, h);
        orc_act_backward(mlp, dx, up, (long)B * T, C, dup);
    }
    double *lw = arr((size_t)6 * C), *lb = arr(6), *lo = zeros((size_t)B * T * 6), *ldi = zeros((size_t)B * T * C),
           *ldw = zeros((size_t)6 * C), *ldb = zeros(6);
    orc_linear_forward(x, lw, lb, (long)B * T, C, 6, lo);
    orc_linear_backward(lo, x, lw, (long)B * T, C, 6, ldi, ldw, ldb);
    double *all[] = {wte, wpe, x, dwte, dwpe, dx, lg, dl, rl, p, g, m, v, y, rs, mu, gg, bb, dg, db, dxx, h,
                     dup, up, lw, lb, lo, ldi, ldw, ldb};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; i++) free(all[i]);
}

int main(void) {
    int n = 0;
    for (int norm = 0; norm < 3; norm++)
        for (int mlp = 0; mlp < 3; mlp++)
            for (int rope = 0; rope < 2; rope++)
                for (int bias = 0; bias < 2; bias++) {
                    block_case(norm, mlp, rope, bias);
                    n++;
                }
    attention_cases();
    harness_cases();
    printf("oracle sanitizer driver: %d block configurations, attention, harness and optimizer done\n", n);
    return 0;
}
