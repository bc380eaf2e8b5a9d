"""Pins of the CPU oracle's per-op functions to things other than itself:
library routines (numpy / torch float64), closed forms, invariants, brute
force and central finite differences.  CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

rng = np.random.default_rng(1234)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def T64(a):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)


# ---------------------------------------------------------------- linear --
def test_linear_forward_matches_matmul(orc):
    x = rng.standard_normal((7, 13))
    w = rng.standard_normal((5, 13))
    b = rng.standard_normal(5)
    assert rel(orc.linear_forward(x, w, b), x @ w.T + b) < 1e-14
    assert rel(orc.linear_forward(x, w), x @ w.T) < 1e-14


def test_linear_backward_matches_matmul(orc):
    x = rng.standard_normal((9, 6))
    w = rng.standard_normal((4, 6))
    dy = rng.standard_normal((9, 4))
    dinp, dw, db = orc.linear_backward(dy, x, w)
    assert rel(dinp, dy @ w) < 1e-14
    assert rel(dw, dy.T @ x) < 1e-14
    # bias gradient two ways: column sum, and the gradient of sum(dy * (x w^T + b)) in b
    assert rel(db, dy.sum(0)) < 1e-14
    bt = torch.zeros(4, dtype=torch.float64, requires_grad=True)
    (T64(dy) * (T64(x) @ T64(w).T + bt)).sum().backward()
    assert rel(db, bt.grad.numpy()) < 1e-14


# ----------------------------------------------------------------- norms --
@pytest.mark.parametrize("mode", ["rms", "rms_nogamma", "layer"])
def test_norm_forward_matches_torch(orc, mode):
    C = 24
    x = rng.standard_normal((11, C)) * 3 + (0.5 if mode == "layer" else 0)
    g = 1 + 0.2 * rng.standard_normal(C)
    b = 0.1 * rng.standard_normal(C)
    eps = 1e-5
    out, rstd, mean = orc.norm_forward(mode, x, g if mode != "rms_nogamma" else None,
                                       b if mode == "layer" else None, eps)
    if mode == "layer":
        ref = F.layer_norm(T64(x), (C,), T64(g), T64(b), eps)
    else:
        ref = F.rms_norm(T64(x), (C,), T64(g) if mode == "rms" else None, eps)
    assert rel(out, ref.numpy()) < 1e-13


def test_rms_invariant(orc):
    C, eps = 32, 1e-5
    x = rng.standard_normal((5, C)) * 0.01   # small, so eps matters
    g = 1 + 0.3 * rng.standard_normal(C)
    out, rstd, _ = orc.norm_forward("rms", x, g, None, eps)
    ms = (x ** 2).mean(1)
    assert rel(((out / g) ** 2).mean(1), ms / (ms + eps)) < 1e-12
    assert rel(rstd, 1 / np.sqrt(ms + eps)) < 1e-14


def test_layernorm_invariants(orc):
    C, eps = 40, 1e-5
    x = rng.standard_normal((6, C)) * 0.02 + 3.0
    out, rstd, mean = orc.norm_forward("layer", x, np.ones(C), np.zeros(C), eps)
    var = x.var(1)
    assert np.abs(out.mean(1)).max() < 1e-12
    assert rel(out.var(1), var / (var + eps)) < 1e-10
    assert rel(mean, x.mean(1)) < 1e-14


@pytest.mark.parametrize("mode", ["rms", "rms_nogamma", "layer"])
def test_norm_backward_matches_autograd(orc, mode):
    C, R, eps = 20, 9, 1e-5
    x = rng.standard_normal((R, C))
    g = 1 + 0.2 * rng.standard_normal(C)
    b = 0.1 * rng.standard_normal(C)
    dy = rng.standard_normal((R, C))
    out, rstd, mean = orc.norm_forward(mode, x, g, b, eps)
    dx, dg, db = orc.norm_backward(mode, dy, x, g, rstd, mean)
    xt = T64(x).requires_grad_()
    gt = T64(g).requires_grad_()
    bt = T64(b).requires_grad_()
    if mode == "layer":
        y = F.layer_norm(xt, (C,), gt, bt, eps)
    else:
        y = F.rms_norm(xt, (C,), gt if mode == "rms" else None, eps)
    (y * T64(dy)).sum().backward()
    assert rel(dx, xt.grad.numpy()) < 1e-12
    if mode != "rms_nogamma":
        assert rel(dg, gt.grad.numpy()) < 1e-12
    if mode == "layer":
        assert rel(db, bt.grad.numpy()) < 1e-12
        assert np.abs(dx.sum(1)).max() < 1e-12 * np.abs(dx).max() * C


def test_norm_backward_accumulates(orc):
    """dx, dgamma are += (the caller's residual gradient rides along)."""
    import oracle
    C, R = 8, 3
    x = rng.standard_normal((R, C))
    g = rng.standard_normal(C)
    dy = rng.standard_normal((R, C))
    _, rstd, mean = orc.norm_forward("rms", x, g)
    dx0, dg0, _ = orc.norm_backward("rms", dy, x, g, rstd, mean)
    dx = np.full((R, C), 2.5)
    dg = np.full(C, -1.0)
    db = np.zeros(C)
    lib = oracle.lib()
    import ctypes
    lib.orc_norm_backward(0, oracle._p(oracle._d(dy)), oracle._p(oracle._d(x)), oracle._p(oracle._d(g)),
                          oracle._p(oracle._d(rstd)), oracle._p(oracle._d(mean)), ctypes.c_long(R), C,
                          oracle._p(dx), oracle._p(dg), oracle._p(db))
    assert rel(dx, dx0 + 2.5) < 1e-14 and rel(dg, dg0 - 1.0) < 1e-14


# ------------------------------------------------------------------ rope --
def _rope_inputs(B=2, T=9, NH=3, NKV=1, hd=8):
    C = NH * hd
    QKV = C + 2 * NKV * hd
    return rng.standard_normal((B * T, QKV)), B, T, C, NH, NKV, hd, QKV


def test_rope_complex_form(orc):
    """NeoX pairs (i, i+hd/2) rotate like the complex number x_i + i x_{i+hd/2}
    multiplied by exp(i t theta_i), theta_i = base^(-2i/hd)."""
    buf, B, T, C, NH, NKV, hd, QKV = _rope_inputs()
    base = 1e4
    out = orc.rope(buf, B, T, QKV, 0, NH, hd, base)
    half = hd // 2
    theta = base ** (-2.0 * np.arange(half) / hd)
    t = np.tile(np.arange(T), B)[:, None]
    for h in range(NH):
        z = buf[:, h * hd:h * hd + half] + 1j * buf[:, h * hd + half:(h + 1) * hd]
        zr = z * np.exp(1j * t * theta[None, :])
        assert rel(out[:, h * hd:h * hd + half], zr.real) < 1e-13
        assert rel(out[:, h * hd + half:(h + 1) * hd], zr.imag) < 1e-13
    # columns outside the rotated heads are untouched
    assert np.array_equal(out[:, NH * hd:], buf[:, NH * hd:])


def test_rope_properties(orc):
    buf, B, T, C, NH, NKV, hd, QKV = _rope_inputs()
    base = 1e6
    out = orc.rope(buf, B, T, QKV, C, NKV, hd, base)       # k heads only
    half = hd // 2
    # t = 0 rows are unchanged
    for b in range(B):
        assert np.allclose(out[b * T], buf[b * T], rtol=0, atol=0)
    # each pair keeps its norm
    k0, k1 = buf[:, C:C + half], buf[:, C + half:C + hd]
    r0, r1 = out[:, C:C + half], out[:, C + half:C + hd]
    assert rel(r0 ** 2 + r1 ** 2, k0 ** 2 + k1 ** 2) < 1e-13
    # inverse o forward = identity
    back = orc.rope(out, B, T, QKV, C, NKV, hd, base, inverse=True)
    assert rel(back, buf) < 1e-13
    # relative position: (R_t q).(R_s k) depends only on t - s
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    Tn = 12
    qb = np.zeros((Tn, hd)); qb[:] = q
    kb = np.zeros((Tn, hd)); kb[:] = k
    rq = orc.rope(qb, 1, Tn, hd, 0, 1, hd, base)
    rk = orc.rope(kb, 1, Tn, hd, 0, 1, hd, base)
    d1 = rq[7] @ rk[3]
    d2 = rq[9] @ rk[5]
    d3 = rq[4] @ rk[0]
    assert abs(d1 - d2) < 1e-12 and abs(d1 - d3) < 1e-12


def test_rope_transposed_is_gradient(orc):
    """The inverse rotation is the gradient of the forward rotation."""
    buf, B, T, C, NH, NKV, hd, QKV = _rope_inputs(B=1, T=5, NH=1, NKV=1, hd=4)
    g = rng.standard_normal(buf.shape)
    base = 1e4
    back = orc.rope(g, B, T, QKV, 0, NH, hd, base, inverse=True)
    eps = 1e-6
    for idx in [(0, 0), (3, 1), (4, 3), (2, 2)]:
        p = buf.copy(); p[idx] += eps
        m = buf.copy(); m[idx] -= eps
        fd = ((orc.rope(p, B, T, QKV, 0, NH, hd, base) - orc.rope(m, B, T, QKV, 0, NH, hd, base)) * g).sum() / (2 * eps)
        assert abs(fd - back[idx]) < 1e-8


# ------------------------------------------------------------- attention --
def _qkv(B, T, NH, NKV, hd, scale=1.0):
    C = NH * hd
    QKV = C + 2 * NKV * hd
    return rng.standard_normal((B, T, QKV)) * scale, C


def _torch_attn(qkv, B, T, C, NH, NKV):
    hd = C // NH
    q = qkv[..., :C].reshape(B, T, NH, hd).permute(0, 2, 1, 3)
    k = qkv[..., C:C + NKV * hd].reshape(B, T, NKV, hd).permute(0, 2, 1, 3)
    v = qkv[..., C + NKV * hd:].reshape(B, T, NKV, hd).permute(0, 2, 1, 3)
    k = k.repeat_interleave(NH // NKV, dim=1)
    v = v.repeat_interleave(NH // NKV, dim=1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    return o.permute(0, 2, 1, 3).reshape(B, T, C)


@pytest.mark.parametrize("B,T,NH,NKV,hd", [(2, 7, 4, 2, 4), (1, 1, 2, 1, 8), (1, 13, 3, 3, 6), (2, 5, 4, 1, 16)])
def test_attention_forward_vs_torch_and_bruteforce(orc, B, T, NH, NKV, hd):
    qkv, C = _qkv(B, T, NH, NKV, hd)
    out, lse = orc.attn_forward(qkv, B, T, C, NH, NKV)
    ref = _torch_attn(T64(qkv), B, T, C, NH, NKV).numpy()
    assert rel(out, ref) < 1e-12
    outm, att = orc.attn_forward_materialized(qkv, B, T, C, NH, NKV)
    assert rel(out, outm) < 1e-13
    # softmax rows sum to one and vanish above the diagonal
    assert np.abs(att.sum(-1) - 1).max() < 1e-12
    assert np.abs(np.triu(att, 1)).max() == 0.0
    # lse: sum_j exp(s_j - lse) = 1, with the scaled scores rebuilt by numpy
    q = qkv[..., :C].reshape(B, T, NH, hd)
    k = qkv[..., C:C + NKV * hd].reshape(B, T, NKV, hd)
    for b in range(B):
        for h in range(NH):
            s = q[b, :, h] @ k[b, :, h // (NH // NKV)].T / np.sqrt(hd)
            s = np.where(np.tril(np.ones((T, T))) > 0, s, -np.inf)
            assert np.abs(np.exp(s - lse[b, h][:, None]).sum(1) - 1).max() < 1e-12


def test_attention_special_cases(orc):
    B, T, NH, NKV, hd = 1, 6, 2, 1, 4
    qkv, C = _qkv(B, T, NH, NKV, hd)
    # T = 1: out = v
    out1, lse1 = orc.attn_forward(qkv[:, :1], B, 1, C, NH, NKV)
    v0 = qkv[0, 0, C + NKV * hd:]
    assert rel(out1[0, 0, :hd], v0) < 1e-15 and rel(out1[0, 0, hd:], v0) < 1e-15
    # all keys equal: out_t = mean(v_0..v_t)
    q2 = qkv.copy()
    q2[..., C:C + NKV * hd] = q2[:, :1, C:C + NKV * hd]
    out2, _ = orc.attn_forward(q2, B, T, C, NH, NKV)
    v = q2[0, :, C + NKV * hd:]
    cm = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    assert rel(out2[0, :, :hd], cm) < 1e-13
    # GQA == MHA with each kv head repeated
    qkv3, C3 = _qkv(2, 5, 4, 2, 4)
    o_g, l_g = orc.attn_forward(qkv3, 2, 5, C3, 4, 2)
    k = qkv3[..., C3:C3 + 8].reshape(2, 5, 2, 4).repeat(2, axis=2).reshape(2, 5, 16)
    v = qkv3[..., C3 + 8:].reshape(2, 5, 2, 4).repeat(2, axis=2).reshape(2, 5, 16)
    mha = np.concatenate([qkv3[..., :C3], k, v], -1)
    o_m, l_m = orc.attn_forward(mha, 2, 5, C3, 4, 4)
    assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)


def test_attention_causality(orc):
    B, T, NH, NKV, hd = 1, 8, 2, 1, 4
    qkv, C = _qkv(B, T, NH, NKV, hd)
    dout = rng.standard_normal((B, T, C))
    out, lse = orc.attn_forward(qkv, B, T, C, NH, NKV)
    j = 5
    p = qkv.copy()
    p[0, j:, C:] += rng.standard_normal(p[0, j:, C:].shape)   # change k, v at rows >= j
    out2, lse2 = orc.attn_forward(p, B, T, C, NH, NKV)
    assert np.array_equal(out[0, :j], out2[0, :j]) and np.array_equal(lse[..., :j], lse2[..., :j])
    # dO at rows t < j does not reach dk_j, dv_j
    d1 = orc.attn_backward(qkv, dout, B, T, C, NH, NKV)
    d2o = dout.copy()
    d2o[0, :j] += rng.standard_normal(d2o[0, :j].shape)
    d2 = orc.attn_backward(qkv, d2o, B, T, C, NH, NKV)
    assert np.array_equal(d1[0, j:, C:], d2[0, j:, C:])


@pytest.mark.parametrize("B,T,NH,NKV,hd", [(2, 6, 4, 2, 4), (1, 8, 2, 2, 8), (1, 5, 4, 1, 4)])
def test_attention_backward_vs_autograd_and_bruteforce(orc, B, T, NH, NKV, hd):
    qkv, C = _qkv(B, T, NH, NKV, hd)
    dout = rng.standard_normal((B, T, C))
    dqkv = orc.attn_backward(qkv, dout, B, T, C, NH, NKV)
    qt = T64(qkv).requires_grad_()
    (_torch_attn(qt, B, T, C, NH, NKV) * T64(dout)).sum().backward()
    assert rel(dqkv, qt.grad.numpy()) < 1e-11
    _, att = orc.attn_forward_materialized(qkv, B, T, C, NH, NKV)
    dm = orc.attn_backward_materialized(qkv, att, dout, B, T, C, NH, NKV)
    assert rel(dqkv, dm) < 1e-12


def test_attention_backward_finite_difference(orc):
    B, T, NH, NKV, hd = 1, 4, 2, 1, 4
    qkv, C = _qkv(B, T, NH, NKV, hd)
    dout = rng.standard_normal((B, T, C))
    dqkv = orc.attn_backward(qkv, dout, B, T, C, NH, NKV)
    h = 1e-6
    for idx in np.ndindex(qkv.shape):
        p = qkv.copy(); p[idx] += h
        m = qkv.copy(); m[idx] -= h
        fd = ((orc.attn_forward(p, B, T, C, NH, NKV)[0] - orc.attn_forward(m, B, T, C, NH, NKV)[0]) * dout).sum() / (2 * h)
        assert abs(fd - dqkv[idx]) <= 1e-7 * (1 + abs(fd))


def test_attention_backward_global_sums(orc):
    """sum_j dS_tj = 0 for every query row, hence sum over keys of dk is 0, and
    sum over keys of dv equals the sum of dO over the group's query rows."""
    B, T, NH, NKV, hd = 2, 9, 4, 2, 4
    qkv, C = _qkv(B, T, NH, NKV, hd)
    dout = rng.standard_normal((B, T, C))
    d = orc.attn_backward(qkv, dout, B, T, C, NH, NKV)
    dk = d[..., C:C + NKV * hd].reshape(B, T, NKV, hd)
    dv = d[..., C + NKV * hd:].reshape(B, T, NKV, hd)
    assert np.abs(dk.sum(1)).max() < 1e-12 * np.abs(dk).max() * T
    dO = dout.reshape(B, T, NKV, NH // NKV, hd).sum(3)
    assert rel(dv.sum(1), dO.sum(1)) < 1e-13


# ------------------------------------------------------------ activations --
@pytest.mark.parametrize("mlp", ["swiglu", "relu", "gelu_tanh"])
def test_activations_vs_torch(orc, mlp):
    H, R = 10, 6
    W = 2 * H if mlp == "swiglu" else H
    up = rng.standard_normal((R, W)) * 2
    dh = rng.standard_normal((R, H))
    h = orc.act_forward(mlp, up, H)
    dup = orc.act_backward(mlp, dh, up, H)
    ut = T64(up).requires_grad_()
    if mlp == "swiglu":
        ref = F.silu(ut[:, :H]) * ut[:, H:]
    elif mlp == "relu":
        ref = F.relu(ut)
    else:
        ref = F.gelu(ut, approximate="tanh")
    (ref * T64(dh)).sum().backward()
    assert rel(h, ref.detach().numpy()) < 1e-14
    assert rel(dup, ut.grad.numpy()) < 1e-13


def test_activation_special_values(orc):
    z = np.zeros((1, 2))
    assert orc.act_forward("swiglu", np.array([[0.0, 5.0]]), 1)[0, 0] == 0.0
    assert orc.act_forward("gelu_tanh", z[:, :1], 1)[0, 0] == 0.0
    assert orc.act_backward("gelu_tanh", np.ones((1, 1)), z[:, :1], 1)[0, 0] == 0.5
    assert orc.act_backward("relu", np.ones((1, 1)), z[:, :1], 1)[0, 0] == 0.0
    assert orc.act_forward("relu", np.array([[-1e-300]]), 1)[0, 0] == 0.0
    # gelu tanh closed form at x = 1: 0.5 (1 + tanh(sqrt(2/pi) 1.044715))
    v = orc.act_forward("gelu_tanh", np.array([[1.0]]), 1)[0, 0]
    assert abs(v - 0.5 * (1 + np.tanh(np.sqrt(2 / np.pi) * 1.044715))) < 1e-16


def test_attention_tail_equals_full(orc):
    """The tail evaluator is the same definition on a subset: it must agree
    with the full row-wise forward/backward on every tail row."""
    B, T, NH, NKV, hd, R = 1, 23, 4, 2, 8, 7
    qkv, C = _qkv(B, T, NH, NKV, hd)
    dout = rng.standard_normal((B, T, C))
    o, lse = orc.attn_forward(qkv, B, T, C, NH, NKV)
    d = orc.attn_backward(qkv, dout, B, T, C, NH, NKV)
    KV = NKV * hd
    ot, lt, dqt, dkt, dvt = orc.attn_tail(qkv[0, T - R:, :C], qkv[0, :, C:C + KV], qkv[0, :, C + KV:],
                                         dout[0, T - R:], T, R, NH, NKV, hd)
    assert rel(ot, o[0, T - R:]) < 1e-13 and rel(lt, lse[0, :, T - R:]) < 1e-13
    assert rel(dqt, d[0, T - R:, :C]) < 1e-12
    assert rel(dkt, d[0, T - R:, C:C + KV]) < 1e-12 and rel(dvt, d[0, T - R:, C + KV:]) < 1e-12
