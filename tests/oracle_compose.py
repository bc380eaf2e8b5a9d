"""Compositions of the oracle's per-op functions used by the full-size tests
(test helper; no test functions here)."""
import numpy as np


def block_tail_reference(orc, cfg, w, x, dy, R):
    """Forward output and input gradient of the last R rows of ONE sequence
    (x, dy: [T, C]), composed from the oracle's per-op functions."""
    T, C, NH, NKV, H = cfg.T, cfg.C, cfg.NH, cfg.NKV, cfg.H
    hd = C // NH
    KV = NKV * hd
    t0 = T - R
    g1, b1, g2, b2 = w.get("g1"), w.get("b1"), w.get("g2"), w.get("b2")
    n1, r1, mu1 = orc.norm_forward(cfg.norm, x, g1, b1, cfg.eps)
    wq, wk, wv = w["wqkv"][:C], w["wqkv"][C:C + KV], w["wqkv"][C + KV:]
    bq = bk = bv = None
    if cfg.qkv_bias:
        bq, bk, bv = w["bqkv"][:C], w["bqkv"][C:C + KV], w["bqkv"][C + KV:]
    k = orc.linear_forward(n1, wk, bk)
    v = orc.linear_forward(n1, wv, bv)
    q_full = np.zeros((T, C))
    q_full[t0:] = orc.linear_forward(n1[t0:], wq, bq)
    if cfg.rope == "neox":
        k = orc.rope(k, 1, T, KV, 0, NKV, hd, cfg.rope_base)
        q_full = orc.rope(q_full, 1, T, C, 0, NH, hd, cfg.rope_base)
    qt = q_full[t0:]
    zeros = np.zeros((R, C))
    o_t, lse_t, _, _, _ = orc.attn_tail(qt, k, v, zeros, T, R, NH, NKV, hd)
    xt = x[t0:].astype(np.float64)
    x2 = xt + orc.linear_forward(o_t, w["wo"], w.get("bo"))
    n2, r2, mu2 = orc.norm_forward(cfg.norm, x2, g2, b2, cfg.eps)
    up = orc.linear_forward(n2, w["w_up"], w.get("b_up"))
    h = orc.act_forward(cfg.mlp, up, H)
    y = x2 + orc.linear_forward(h, w["w_down"], w.get("b_down"))
    # backward of the tail rows
    dyt = dy[t0:].astype(np.float64)
    dh, _, _ = orc.linear_backward(dyt, h, w["w_down"])
    dup = orc.act_backward(cfg.mlp, dh, up, H)
    dn2, _, _ = orc.linear_backward(dup, n2, w["w_up"])
    dn, _, _ = orc.norm_backward(cfg.norm, dn2, x2, g2, r2, mu2)
    dx2 = dyt + dn
    dO, _, _ = orc.linear_backward(dx2, o_t, w["wo"])
    _, _, dq, dk, dv = orc.attn_tail(qt, k, v, dO, T, R, NH, NKV, hd)
    if cfg.rope == "neox":
        dqf = np.zeros((T, C))
        dqf[t0:] = dq
        dkf = np.zeros((T, KV))
        dkf[t0:] = dk
        dq = orc.rope(dqf, 1, T, C, 0, NH, hd, cfg.rope_base, inverse=True)[t0:]
        dk = orc.rope(dkf, 1, T, KV, 0, NKV, hd, cfg.rope_base, inverse=True)[t0:]
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dn1, _, _ = orc.linear_backward(dqkv, n1[t0:], w["wqkv"])
    dn, _, _ = orc.norm_backward(cfg.norm, dn1, x[t0:], g1, r1[t0:], mu1[t0:])
    return y, dx2 + dn, lse_t
