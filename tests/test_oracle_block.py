"""Pins of the oracle's whole-block forward and backward.

1. An independent float64 composition from torch library routines (linear,
   rms_norm / layer_norm, scaled_dot_product_attention, silu / relu / gelu)
   with a rotate-half NeoX RoPE, differentiated by torch autograd.
2. Central finite differences of the oracle's own forward (h = 1e-5, fp64)
   against its hand-written backward, for every parameter tensor and the
   input, over every norm / MLP / RoPE / bias combination (the nx trainer's
   gradcheck protocol, made exhaustive and in double).
CPU only."""
import itertools
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

rng = np.random.default_rng(99)


def rel(a, b):
    return np.abs(np.asarray(a) - np.asarray(b)).max() / max(np.abs(np.asarray(b)).max(), 1e-300)


def make_cfg(norm, mlp, rope, bias, B=2, T=5, C=8, NH=2, NKV=1, H=12):
    return SimpleNamespace(B=B, T=T, C=C, NH=NH, NKV=NKV, H=H, norm=norm, mlp=mlp, rope=rope,
                           rope_base=1e4 if rope == "neox" else 0.0, eps=1e-5,
                           qkv_bias=bias, o_bias=bias, mlp_bias=bias)


def make_weights(c, scale=0.4):
    hd = c.C // c.NH
    QKV = c.C + 2 * c.NKV * hd
    W = 2 * c.H if c.mlp == "swiglu" else c.H
    w = {"wqkv": rng.standard_normal((QKV, c.C)) * scale, "wo": rng.standard_normal((c.C, c.C)) * scale,
         "w_up": rng.standard_normal((W, c.C)) * scale, "w_down": rng.standard_normal((c.C, c.H)) * scale}
    if c.norm != "rms_nogamma":
        w["g1"] = 1 + 0.3 * rng.standard_normal(c.C)
        w["g2"] = 1 + 0.3 * rng.standard_normal(c.C)
    if c.norm == "layer":
        w["b1"] = 0.2 * rng.standard_normal(c.C)
        w["b2"] = 0.2 * rng.standard_normal(c.C)
    if c.qkv_bias:
        w["bqkv"] = 0.2 * rng.standard_normal(QKV)
    if c.o_bias:
        w["bo"] = 0.2 * rng.standard_normal(c.C)
    if c.mlp_bias:
        w["b_up"] = 0.2 * rng.standard_normal(W)
        w["b_down"] = 0.2 * rng.standard_normal(c.C)
    return w


def torch_block(c, w, x):
    """Independent float64 block: pre-norm attention + MLP with residuals."""
    B, T, C, NH, NKV = c.B, c.T, c.C, c.NH, c.NKV
    hd = C // NH

    def norm(v, g, b):
        if c.norm == "layer":
            return F.layer_norm(v, (C,), g, b, c.eps)
        return F.rms_norm(v, (C,), g if c.norm == "rms" else None, c.eps)

    def rope(v, nh):       # v [B, T, nh*hd]; rotate_half form
        if c.rope != "neox":
            return v
        half = hd // 2
        inv = c.rope_base ** (-torch.arange(0, half, dtype=torch.float64) * 2 / hd)
        ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
        cos = torch.cat([ang.cos(), ang.cos()], -1)
        sin = torch.cat([ang.sin(), ang.sin()], -1)
        v = v.reshape(B, T, nh, hd)
        rot = torch.cat([-v[..., half:], v[..., :half]], -1)
        return (v * cos[None, :, None, :] + rot * sin[None, :, None, :]).reshape(B, T, nh * hd)

    n1 = norm(x, w.get("g1"), w.get("b1"))
    qkv = F.linear(n1, w["wqkv"], w.get("bqkv"))
    q = rope(qkv[..., :C], NH)
    k = rope(qkv[..., C:C + NKV * hd], NKV)
    v = qkv[..., C + NKV * hd:]
    qh = q.reshape(B, T, NH, hd).transpose(1, 2)
    kh = k.reshape(B, T, NKV, hd).transpose(1, 2).repeat_interleave(NH // NKV, 1)
    vh = v.reshape(B, T, NKV, hd).transpose(1, 2).repeat_interleave(NH // NKV, 1)
    o = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True).transpose(1, 2).reshape(B, T, C)
    x2 = x + F.linear(o, w["wo"], w.get("bo"))
    n2 = norm(x2, w.get("g2"), w.get("b2"))
    up = F.linear(n2, w["w_up"], w.get("b_up"))
    if c.mlp == "swiglu":
        h = F.silu(up[..., :c.H]) * up[..., c.H:]
    elif c.mlp == "relu":
        h = F.relu(up)
    else:
        h = F.gelu(up, approximate="tanh")
    return x2 + F.linear(h, w["w_down"], w.get("b_down"))


COMBOS = list(itertools.product(["rms", "rms_nogamma", "layer"], ["swiglu", "relu", "gelu_tanh"],
                                ["none", "neox"], [False, True]))


@pytest.mark.parametrize("norm,mlp,rope,bias", COMBOS)
def test_block_vs_torch_autograd(orc, norm, mlp, rope, bias):
    c = make_cfg(norm, mlp, rope, bias, B=2, T=7, C=16, NH=4, NKV=2, H=20)
    w = make_weights(c)
    x = rng.standard_normal((c.B, c.T, c.C))
    dy = rng.standard_normal((c.B, c.T, c.C))
    y, sv = orc.block_forward(c, w, x)
    dx, g = orc.block_backward(c, w, x, sv, dy)
    wt = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    xt = torch.tensor(x, requires_grad=True)
    yt = torch_block(c, wt, xt)
    (yt * torch.tensor(dy)).sum().backward()
    assert rel(y, yt.detach().numpy()) < 1e-12
    assert rel(dx, xt.grad.numpy()) < 1e-11
    for k in w:
        assert rel(g[k], wt[k].grad.numpy()) < 1e-11, k


@pytest.mark.parametrize("norm,mlp,rope,bias", COMBOS)
def test_block_finite_difference(orc, norm, mlp, rope, bias):
    c = make_cfg(norm, mlp, rope, bias)
    w = make_weights(c)
    x = rng.standard_normal((c.B, c.T, c.C))
    R = rng.standard_normal((c.B, c.T, c.C))
    _, sv = orc.block_forward(c, w, x)
    dx, g = orc.block_backward(c, w, x, sv, R)

    def loss(ww, xx):
        return float((orc.block_forward(c, ww, xx)[0] * R).sum())

    h = 1e-5
    full = (norm, mlp, rope, bias) in {("rms", "swiglu", "neox", True), ("layer", "gelu_tanh", "none", True),
                                       ("rms_nogamma", "relu", "none", False)}
    for name in list(w) + ["x"]:
        base = x if name == "x" else w[name]
        idxs = list(np.ndindex(base.shape))
        if not full and len(idxs) > 12:
            sel = rng.choice(len(idxs), 12, replace=False)
            idxs = [idxs[i] for i in sel]
        ana = dx if name == "x" else g[name]
        for idx in idxs:
            p = base.copy(); p[idx] += h
            m = base.copy(); m[idx] -= h
            if name == "x":
                fd = (loss(w, p) - loss(w, m)) / (2 * h)
            else:
                fd = (loss({**w, name: p}, x) - loss({**w, name: m}, x)) / (2 * h)
            assert abs(fd - ana[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, ana[idx])


def test_block_stack_chains_layers(orc):
    """A two-layer stack equals two single blocks chained by hand, and its dx
    equals the finite difference of the stacked loss."""
    c = make_cfg("rms", "swiglu", "neox", True)
    ws = [make_weights(c), make_weights(c)]
    x = rng.standard_normal((c.B, c.T, c.C))
    R = rng.standard_normal((c.B, c.T, c.C))
    y, dx, grads, _ = orc.block_stack(c, ws, x, R)
    y1, _ = orc.block_forward(c, ws[0], x)
    y2, _ = orc.block_forward(c, ws[1], y1)
    assert np.array_equal(y, y2)
    h = 1e-5
    for idx in [(0, 0, 0), (1, 4, 7), (0, 2, 3)]:
        p = x.copy(); p[idx] += h
        m = x.copy(); m[idx] -= h
        fd = ((orc.block_stack(c, ws, p, R)[0] - orc.block_stack(c, ws, m, R)[0]) * R).sum() / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * (1 + abs(fd))


def test_planted_mistakes_are_caught(orc):
    """Sanity of the pins themselves: a sign flip in a gradient, a wrong bias
    or a transposed weight all break agreement with the torch composition."""
    c = make_cfg("layer", "gelu_tanh", "none", True, B=1, T=4, C=8, NH=2, NKV=2, H=8)
    w = make_weights(c)
    x = rng.standard_normal((c.B, c.T, c.C))
    y, _ = orc.block_forward(c, w, x)
    wt = {k: torch.tensor(v) for k, v in w.items()}
    yt = torch_block(c, wt, torch.tensor(x)).numpy()
    assert rel(y, yt) < 1e-12
    bad = dict(w, wo=w["wo"].T.copy())
    assert rel(orc.block_forward(c, bad, x)[0], yt) > 1e-3
    bad = dict(w, b2=-w["b2"])
    assert rel(orc.block_forward(c, bad, x)[0], yt) > 1e-3


@pytest.mark.parametrize("norm,mlp,rope,bias", [("rms", "swiglu", "neox", False), ("layer", "gelu_tanh", "none", True),
                                                ("rms_nogamma", "relu", "none", False)])
def test_block_tail_composition_matches_full_block(orc, norm, mlp, rope, bias):
    """The per-op composition used for the full-size sampled checks (last R rows
    of one sequence) equals the whole-block oracle on those rows."""
    from oracle_compose import block_tail_reference
    c = make_cfg(norm, mlp, rope, bias, B=1, T=19, C=16, NH=4, NKV=2, H=24)
    w = make_weights(c)
    x = rng.standard_normal((1, c.T, c.C))
    dy = rng.standard_normal((1, c.T, c.C))
    y, sv = orc.block_forward(c, w, x)
    dx, _ = orc.block_backward(c, w, x, sv, dy)
    R = 6
    ry, rdx, rl = block_tail_reference(orc, c, w, x[0], dy[0], R)
    assert rel(ry, y[0, c.T - R:]) < 1e-12
    assert rel(rdx, dx[0, c.T - R:]) < 1e-12
    assert rel(rl, sv.lse[0][:, c.T - R:]) < 1e-12
