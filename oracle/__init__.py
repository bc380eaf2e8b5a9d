"""CPU oracle for the decoder block (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's cpu_baseline leg may import
this package.  It wraps liboracle.so (plain C, fp64, built from oracle.c with
gcc) through ctypes.  It never imports the HIP package: configurations are
passed as plain attributes (duck typing) and arrays as numpy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from types import SimpleNamespace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

NORM = {"rms": 0, "rms_nogamma": 1, "layer": 2}
MLP = {"swiglu": 0, "relu": 1, "gelu_tanh": 2}
ROPE = {"none": 0, "neox": 1}

_DP = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "C", "NH", "NKV", "H", "norm", "mlp", "rope")] + [
        ("rope_base", ctypes.c_double), ("eps", ctypes.c_double),
        ("qkv_bias", ctypes.c_int), ("o_bias", ctypes.c_int), ("mlp_bias", ctypes.c_int)]


_WNAMES = ("g1", "b1", "wqkv", "bqkv", "wo", "bo", "g2", "b2", "w_up", "b_up", "w_down", "b_down")
_SNAMES = ("n1", "r1", "mu1", "qkv", "o", "lse", "x2", "n2", "r2", "mu2", "up", "h")


class _W(ctypes.Structure):
    _fields_ = [(n, _DP) for n in _WNAMES]


class _S(ctypes.Structure):
    _fields_ = [(n, _DP) for n in _SNAMES]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = ctypes.CDLL(_SO)
        _lib.orc_num_threads.restype = ctypes.c_int
    return _lib


def _d(a):
    """Contiguous float64 copy/view of a."""
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return _DP()
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_DP)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------------------
# per-op wrappers
# ---------------------------------------------------------------------------
def norm_forward(mode: str, x, g=None, b=None, eps=1e-5):
    x = _d(x)
    C = x.shape[-1]
    R = x.size // C
    out = np.empty_like(x)
    rstd = np.empty(R)
    mean = np.empty(R)
    lib().orc_norm_forward(NORM[mode], _p(x), _p(None if g is None else _d(g)),
                           _p(None if b is None else _d(b)), ctypes.c_double(eps),
                           ctypes.c_long(R), C, _p(out), _p(rstd), _p(mean))
    return out, rstd, mean


def norm_backward(mode: str, dy, x, g, rstd, mean):
    dy, x = _d(dy), _d(x)
    C = x.shape[-1]
    R = x.size // C
    dx = np.zeros_like(x)
    dg = np.zeros(C)
    db = np.zeros(C)
    lib().orc_norm_backward(NORM[mode], _p(dy), _p(x), _p(None if g is None else _d(g)),
                            _p(_d(rstd)), _p(_d(mean)), ctypes.c_long(R), C,
                            _p(dx), _p(dg), _p(db))
    return dx, dg, db


def linear_forward(inp, w, bias=None):
    inp, w = _d(inp), _d(w)
    N, K = w.shape
    R = inp.size // K
    out = np.empty(inp.shape[:-1] + (N,))
    lib().orc_linear_forward(_p(inp), _p(w), _p(None if bias is None else _d(bias)),
                             ctypes.c_long(R), K, N, _p(out))
    return out


def linear_backward(dout, inp, w, parts=("dinp", "dw", "db")):
    """dinp, dw, db of a linear layer; a product left out of `parts` is not
    computed and comes back as None (w may then be None for dinp, or inp
    for dw)."""
    dout = _d(dout)
    N = dout.shape[-1]
    R = dout.size // N
    inp = _d(inp) if inp is not None else None
    w = _d(w) if w is not None else None
    K = w.shape[1] if w is not None else inp.shape[-1]
    dinp = np.zeros((R, K)).reshape(dout.shape[:-1] + (K,)) if "dinp" in parts else None
    dw = np.zeros((N, K)) if "dw" in parts else None
    db = np.zeros(N) if "db" in parts else None
    lib().orc_linear_backward(_p(dout), _p(inp), _p(w), ctypes.c_long(R), K, N,
                              _p(dinp), _p(dw), _p(db))
    return dinp, dw, db


def rope(buf, B, T, stride, off, nheads, hd, base, inverse=False):
    """Returns a rotated copy of buf ([B*T, stride])."""
    out = _d(buf).copy()
    lib().orc_rope(_p(out), B, T, stride, off, nheads, hd, ctypes.c_double(base), int(inverse))
    return out


def attn_forward(qkv, B, T, C, NH, NKV):
    qkv = _d(qkv)
    out = np.empty((B, T, C))
    lse = np.empty((B, NH, T))
    lib().orc_attn_forward(_p(qkv), B, T, C, NH, NKV, _p(out), _p(lse))
    return out, lse


def attn_backward(qkv, dout, B, T, C, NH, NKV):
    qkv, dout = _d(qkv), _d(dout)
    dqkv = np.empty_like(qkv)
    lib().orc_attn_backward(_p(qkv), _p(dout), B, T, C, NH, NKV, _p(dqkv))
    return dqkv


def attn_forward_materialized(qkv, B, T, C, NH, NKV):
    qkv = _d(qkv)
    out = np.empty((B, T, C))
    att = np.empty((B, NH, T, T))
    lib().orc_attn_forward_materialized(_p(qkv), B, T, C, NH, NKV, _p(out), _p(att))
    return out, att


def attn_backward_materialized(qkv, att, dout, B, T, C, NH, NKV):
    qkv, att, dout = _d(qkv), _d(att), _d(dout)
    dqkv = np.empty_like(qkv)
    lib().orc_attn_backward_materialized(_p(qkv), _p(att), _p(dout), B, T, C, NH, NKV, _p(dqkv))
    return dqkv


def attn_tail(q_tail, k, v, dout_tail, T, R, NH, NKV, hd):
    """Attention of the last R query positions of one sequence (all keys):
    returns o_tail [R, NH*hd], lse_tail [NH, R], dq_tail [R, NH*hd] and the
    exact dk / dv of the last R key positions [R, NKV*hd]."""
    q_tail, k, v, dout_tail = _d(q_tail), _d(k), _d(v), _d(dout_tail)
    C, KV = NH * hd, NKV * hd
    o = np.empty((R, C)); lse = np.empty((NH, R)); dq = np.empty((R, C))
    dk = np.empty((R, KV)); dv = np.empty((R, KV))
    lib().orc_attn_tail(_p(q_tail), _p(k), _p(v), _p(dout_tail), T, R, NH, NKV, hd, _p(o), _p(lse), _p(dq),
                        _p(dk), _p(dv))
    return o, lse, dq, dk, dv


def attn_decode(q, k_cache, v_cache, lens, NH, NKV, hd):
    """One query per sequence against its KV cache: q [B, NH*hd], caches
    [B, Tmax, NKV*hd], lens [B] (cache rows in use).  Returns out [B, NH*hd]
    and lse [B, NH] (-inf for an empty cache)."""
    q, k_cache, v_cache = _d(q), _d(k_cache), _d(v_cache)
    B, Tmax = k_cache.shape[0], k_cache.shape[1]
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert q.shape == (B, NH * hd) and v_cache.shape == k_cache.shape and lens.shape == (B,)
    assert k_cache.shape[2] == NKV * hd and int(lens.max(initial=0)) <= Tmax and int(lens.min(initial=0)) >= 0
    out = np.empty((B, NH * hd))
    lse = np.empty((B, NH))
    lib().orc_attn_decode(_p(q), _p(k_cache), _p(v_cache), _ip(lens), B, NH, NKV, hd, Tmax, _p(out), _p(lse))
    return out, lse


def act_forward(mlp: str, up, H):
    up = _d(up)
    W = up.shape[-1]
    R = up.size // W
    h = np.empty(up.shape[:-1] + (H,))
    lib().orc_act_forward(MLP[mlp], _p(up), ctypes.c_long(R), H, _p(h))
    return h


def act_backward(mlp: str, dh, up, H):
    dh, up = _d(dh), _d(up)
    W = up.shape[-1]
    R = up.size // W
    dup = np.zeros_like(up)
    lib().orc_act_backward(MLP[mlp], _p(dh), _p(up), ctypes.c_long(R), H, _p(dup))
    return dup


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------
def _cfg(cfg, B=None, T=None) -> _Cfg:
    return _Cfg(B=cfg.B if B is None else B, T=cfg.T if T is None else T, C=cfg.C, NH=cfg.NH,
                NKV=cfg.NKV, H=cfg.H, norm=NORM[cfg.norm], mlp=MLP[cfg.mlp], rope=ROPE[cfg.rope],
                rope_base=float(cfg.rope_base), eps=float(cfg.eps), qkv_bias=int(cfg.qkv_bias),
                o_bias=int(cfg.o_bias), mlp_bias=int(cfg.mlp_bias))


def _dims(cfg):
    hd = cfg.C // cfg.NH
    QKV = cfg.C + 2 * cfg.NKV * hd
    W = 2 * cfg.H if cfg.mlp == "swiglu" else cfg.H
    return hd, QKV, W


def block_forward(cfg, weights: dict, x):
    """Returns (y [B,T,C], saved namespace of float64 arrays)."""
    B, T, C = cfg.B, cfg.T, cfg.C
    BT = B * T
    hd, QKV, W = _dims(cfg)
    x = _d(x).reshape(B, T, C)
    wd = {k: _d(v) for k, v in weights.items() if v is not None}
    cw = _W(**{n: _p(wd.get(n)) for n in _WNAMES})
    sv = SimpleNamespace(n1=np.empty((BT, C)), r1=np.empty(BT), mu1=np.empty(BT),
                         qkv=np.empty((BT, QKV)), o=np.empty((BT, C)), lse=np.empty((B, cfg.NH, T)),
                         x2=np.empty((BT, C)), n2=np.empty((BT, C)), r2=np.empty(BT),
                         mu2=np.empty(BT), up=np.empty((BT, W)), h=np.empty((BT, cfg.H)))
    cs = _S(**{n: _p(getattr(sv, n)) for n in _SNAMES})
    y = np.empty((B, T, C))
    c = _cfg(cfg)
    lib().orc_block_forward(ctypes.byref(c), ctypes.byref(cw), _p(x), _p(y), ctypes.byref(cs))
    return y, sv


def block_backward(cfg, weights: dict, x, saved, dy):
    """Returns (dx [B,T,C], grads dict).  Gradients start at zero."""
    B, T, C = cfg.B, cfg.T, cfg.C
    x = _d(x).reshape(B, T, C)
    dy = _d(dy).reshape(B, T, C)
    wd = {k: _d(v) for k, v in weights.items() if v is not None}
    cw = _W(**{n: _p(wd.get(n)) for n in _WNAMES})
    grads = {n: np.zeros_like(v) for n, v in wd.items()}
    cg = _W(**{n: _p(grads.get(n)) for n in _WNAMES})
    cs = _S(**{n: _p(getattr(saved, n)) for n in _SNAMES})
    dx = np.empty((B, T, C))
    c = _cfg(cfg)
    lib().orc_block_backward(ctypes.byref(c), ctypes.byref(cw), _p(x), ctypes.byref(cs),
                             _p(dy), _p(dx), ctypes.byref(cg))
    return dx, grads


def block_stack(cfg, layer_weights, x, dy):
    """Forward through all layers, then backward.  Returns (y, dx, grads per
    layer, saved per layer)."""
    saved, xs = [], []
    h = _d(x)
    for w in layer_weights:
        xs.append(h)
        h, sv = block_forward(cfg, w, h)
        saved.append(sv)
    y = h
    g = _d(dy)
    grads = [None] * len(layer_weights)
    for i in reversed(range(len(layer_weights))):
        g, grads[i] = block_backward(cfg, layer_weights[i], xs[i], saved[i], g)
    return y, g, grads, saved


# ---------------------------------------------------------------------------
# model harness: embedding, final norm, LM head, softmax cross-entropy
# ---------------------------------------------------------------------------
_IP = ctypes.POINTER(ctypes.c_int)


def _ip(a):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_IP)


def embed_forward(ids, wte, wpe=None):
    """x[b,t] = wte[ids[b,t]] (+ wpe[t]).  ids [B, T] int."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    B, T = ids.shape
    wte = _d(wte)
    C = wte.shape[1]
    x = np.empty((B, T, C))
    lib().orc_embed_forward(_ip(ids), _p(wte), _p(None if wpe is None else _d(wpe)), B, T, C, _p(x))
    return x


def embed_backward(ids, dx, V, with_wpe=False):
    """(dwte [V, C], dwpe [T, C] or None), both from zero."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    B, T = ids.shape
    dx = _d(dx)
    C = dx.shape[-1]
    dwte = np.zeros((V, C))
    dwpe = np.zeros((T, C)) if with_wpe else None
    lib().orc_embed_backward(_ip(ids), _p(dx), B, T, C, _p(dwte), _p(dwpe))
    return dwte, dwpe


def softmax_ce(logits, targets, scale):
    """Returns (scale * sum of row losses, dlogits, row losses); rows with a
    negative target are masked (zero loss, zero gradient)."""
    logits = _d(logits)
    V = logits.shape[-1]
    R = logits.size // V
    targets = np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
    assert targets.size == R
    dl = np.empty((R, V))
    rl = np.empty(R)
    f = lib().orc_softmax_ce
    f.restype = ctypes.c_double
    loss = f(_p(logits), _ip(targets), ctypes.c_long(R), V, ctypes.c_double(scale), _p(dl), _p(rl))
    return loss, dl, rl


def mtp_targets(ids, T, K):
    """Targets of K prediction heads ("nanoeuler — CUDA kernels": the batch
    fills K targets per position): head j at position t predicts token t+1+j.
    ids [B, T+K] -> [B, T, K] int32."""
    ids = np.asarray(ids)
    return np.stack([ids[:, 1 + j:T + 1 + j] for j in range(K)], axis=-1).astype(np.int32)


def mtp_head_ce(inp, w, targets, K, scale):
    """The LM head with K prediction heads and its softmax cross-entropy
    ("nanoeuler — CUDA kernels": the head GEMM with K*V output columns, the
    softmax_ce kernel over every (position, head) row of V logits, the head's
    matmul backward).  inp [R, C]; w [K*V, C] (head j = rows j*V .. j*V+V-1);
    targets [R, K] (negative: masked); loss = scale * sum of the unmasked row
    losses.  Returns (loss, row_loss [R, K], dinp [R, C], dw [K*V, C],
    dlogits [R, K*V])."""
    inp, w = _d(inp), _d(w)
    R = inp.shape[0]
    V = w.shape[0] // K
    assert w.shape[0] == K * V
    logits = linear_forward(inp, w)
    loss, dl, rl = softmax_ce(logits.reshape(R * K, V), np.asarray(targets).reshape(R * K), scale)
    dl = dl.reshape(R, K * V)
    dinp, dw, _ = linear_backward(dl, inp, w)
    return loss, rl.reshape(R, K), dinp, dw, dl


def model_step(cfg, layer_weights, hw: dict, ids):
    """Loss and every gradient of the whole model for one batch.

    Harness layout (the configuration's attributes): token embedding hw['wte']
    [V, C], position table hw['wpe'] [T, C] if cfg.wpe, an RMSNorm without gamma
    of the embedding if cfg.embed_norm, then the block stack, a final norm of
    the blocks' kind (gamma hw['gf'], beta hw['bf']) if cfg.final_norm, the LM
    head hw['head'] [V, C] (hw['wte'] itself if cfg.tied_head) and the mean
    softmax cross-entropy over the B*T positions with targets ids[:, t+1].
    With cfg.mtp = K > 1 prediction heads, hw['head'] is [K*V, C], ids are
    [B, T+K], head j predicts ids[:, t+1+j] and the mean runs over the B*T*K
    (position, head) pairs.  Returns (loss, grads: dict of harness gradients, per-layer block gradients,
    extras: logits, dlogits, row losses and the final hidden state)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    B, T = cfg.B, cfg.T
    K = getattr(cfg, "mtp", 1)
    assert K == 1 or not cfg.tied_head
    inp, tgt = ids[:, :T], mtp_targets(ids, T, K)
    V = hw["wte"].shape[0]
    x = embed_forward(inp, hw["wte"], hw.get("wpe") if cfg.wpe else None)
    if cfg.embed_norm:
        x0, r0, m0 = norm_forward("rms_nogamma", x, eps=cfg.eps)
    else:
        x0 = x
    saved, xs = [], []
    h = x0
    for w in layer_weights:
        xs.append(h)
        h, sv = block_forward(cfg, w, h)
        saved.append(sv)
    if cfg.final_norm:
        nf, rf, mf = norm_forward(cfg.norm, h, hw.get("gf"), hw.get("bf"), eps=cfg.eps)
    else:
        nf = h
    head = hw["wte"] if cfg.tied_head else hw["head"]
    loss, rows, dnf, dhead, dlogits = mtp_head_ce(nf.reshape(B * T, -1), head, tgt.reshape(B * T, K), K,
                                                  1.0 / (B * T * K))
    logits = linear_forward(nf, head)
    dnf = dnf.reshape(nf.shape)
    grads = {}
    if cfg.final_norm:
        g, dgf, dbf = norm_backward(cfg.norm, dnf, h, hw.get("gf"), rf, mf)
        if cfg.norm != "rms_nogamma":
            grads["gf"] = dgf
        if cfg.norm == "layer":
            grads["bf"] = dbf
    else:
        g = dnf
    bgrads = [None] * len(layer_weights)
    for i in reversed(range(len(layer_weights))):
        g, bgrads[i] = block_backward(cfg, layer_weights[i], xs[i], saved[i], g)
    if cfg.embed_norm:
        g = norm_backward("rms_nogamma", g, x, None, r0, m0)[0]
    dwte, dwpe = embed_backward(inp, g, V, with_wpe=bool(cfg.wpe))
    if cfg.tied_head:
        dwte = dwte + dhead
    else:
        grads["head"] = dhead
    grads["wte"] = dwte
    if cfg.wpe:
        grads["wpe"] = dwpe
    extras = SimpleNamespace(logits=logits.reshape(B * T, K * V), dlogits=dlogits, rows=rows.reshape(-1),
                             nf=nf.reshape(B * T, -1))
    return loss, grads, bgrads, extras


# ---------------------------------------------------------------------------
# optimizer
# ---------------------------------------------------------------------------
def adamw(p, g, m, v, lr, b1, b2, eps, wd, t):
    """One AdamW step (step number t >= 1); returns updated copies (p, m, v)."""
    p, g, m, v = _d(p).copy(), _d(g), _d(m).copy(), _d(v).copy()
    lib().orc_adamw(_p(p), _p(g), _p(m), _p(v), ctypes.c_long(p.size), ctypes.c_double(lr), ctypes.c_double(b1),
                    ctypes.c_double(b2), ctypes.c_double(eps), ctypes.c_double(wd), int(t))
    return p, m, v
