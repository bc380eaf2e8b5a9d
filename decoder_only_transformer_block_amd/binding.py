"""ctypes binding of libdtb.so.  Argument marshalling only: every step of the
block runs in the library's HIP kernels; torch supplies device memory and the
current stream.  The library must be built (python -m
decoder_only_transformer_block_amd.build); nothing here falls back to another
implementation."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdtb.so")

DTB_OK = 0
ERRORS = {-1: "DTB_EINVAL_SHAPE", -2: "DTB_EINVAL_PTR", -3: "DTB_EDTYPE", -4: "DTB_EINVAL_ENUM",
          -5: "DTB_ELAUNCH"}
DTYPE = {"f32": 0, "bf16": 1}
NORM = {"rms": 0, "rms_nogamma": 1, "layer": 2}
MLP = {"swiglu": 0, "relu": 1, "gelu_tanh": 2}
ROPE = {"none": 0, "neox": 1}

_VP = ctypes.c_void_p
_WNAMES = ("g1", "b1", "wqkv", "bqkv", "wo", "bo", "g2", "b2", "w_up", "b_up", "w_down", "b_down")


class BlockCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "C", "NH", "NKV", "H", "norm", "mlp", "rope")] + [
        ("rope_base", ctypes.c_float), ("eps", ctypes.c_float),
        ("qkv_bias", ctypes.c_int), ("o_bias", ctypes.c_int), ("mlp_bias", ctypes.c_int),
        ("dtype", ctypes.c_int)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, _VP) for n in _WNAMES] + [("rope_cs", _VP)]


class BlockGrads(ctypes.Structure):
    _fields_ = [(n, _VP) for n in _WNAMES]


class SavedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_longlong) for n in
                ("n1", "r1", "mu1", "qkv", "o", "lse", "x2", "n2", "r2", "mu2", "up", "h", "total")]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_longlong) for n in ("dh", "dup", "dn2", "dx2", "dO", "dqkv", "dn1", "total")]


class Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double), ("flops", ctypes.c_double), ("bytes", ctypes.c_double),
                ("launches", ctypes.c_longlong)]


class DtbError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdtb.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DtbError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decoder_only_transformer_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i, v, f, z = ctypes.c_int, _VP, ctypes.c_float, ctypes.c_size_t
        L.attn_forward.argtypes = [v, v, v, i, i, i, i, i, i, v]
        L.attn_backward.argtypes = [v, v, v, v, v, i, i, i, i, i, i, v, v]
        L.attn_backward_noalloc.argtypes = [v, v, v, v, v, i, i, i, i, i, i, v]
        L.attn_workspace_bytes.argtypes = [i, i, i]
        L.attn_workspace_bytes.restype = z
        L.attn_decode.argtypes = [v, v, v, v, v, v, i, i, i, i, i, i, i, v, v]
        ll = ctypes.c_longlong
        L.attn_decode_strided.argtypes = [v, v, v, v, v, v, i, i, i, i, i, ll, ll, ll, i, i, v, v]
        L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.attn_decode_workspace_bytes.restype = z
        cp = ctypes.POINTER(BlockCfg)
        L.block_saved_bytes.argtypes = [cp]
        L.block_saved_bytes.restype = z
        L.block_workspace_bytes.argtypes = [cp]
        L.block_workspace_bytes.restype = z
        L.block_saved_layout.argtypes = [cp, ctypes.POINTER(SavedLayout)]
        L.block_workspace_layout.argtypes = [cp, ctypes.POINTER(WorkspaceLayout)]
        L.block_forward.argtypes = [cp, ctypes.POINTER(BlockWeights), v, v, v, v, v]
        L.rope_table_build.argtypes = [v, i, i, ctypes.c_float, v]
        L.block_backward.argtypes = [cp, ctypes.POINTER(BlockWeights), v, v, v, v, ctypes.POINTER(BlockGrads), v, v]
        L.block_backward_overlap.argtypes = [cp, ctypes.POINTER(BlockWeights), v, v, v, v,
                                             ctypes.POINTER(BlockGrads), v, v, v]
        L.dtb_overlap_create.argtypes = [ctypes.POINTER(_VP)]
        L.dtb_overlap_destroy.argtypes = [v]
        L.linear_forward.argtypes = [v, v, v, v, v, i, i, i, i, v]
        L.linear_backward.argtypes = [v, v, v, v, v, v, i, i, i, i, v, v]
        L.linear_workspace_bytes.argtypes = [i, i, i, i]
        L.linear_workspace_bytes.restype = z
        L.encoder_forward.argtypes = [v, v, v, v, i, i, i, i, i, v]
        L.encoder_backward.argtypes = [v, v, v, v, i, i, i, i, i, v]
        L.norm_forward.argtypes = [v, v, v, v, v, v, i, i, i, f, i, v]
        L.norm_backward.argtypes = [v, v, v, v, v, v, v, v, v, i, i, i, i, v, v]
        L.norm_workspace_bytes.argtypes = [i, i]
        L.norm_workspace_bytes.restype = z
        L.activation_forward.argtypes = [v, v, i, i, i, i, v]
        L.activation_backward.argtypes = [v, v, v, i, i, i, i, v]
        L.lm_head_forward.argtypes = [v, i, v, v, i, i, i, i, v]
        L.lm_head_backward.argtypes = [v, v, v, i, v, v, i, i, i, i, v, v]
        L.lm_head_workspace_bytes.argtypes = [i, i, i, i]
        L.lm_head_workspace_bytes.restype = z
        L.softmax_ce.argtypes = [v, v, v, v, i, v, i, i, f, i, v]
        L.lm_head_ce.argtypes = [v, v, v, v, v, v, v, i, i, i, i, f, i, v, v]
        L.lm_head_mtp_ce.argtypes = [v, v, v, v, v, v, v, i, i, i, i, i, f, i, v, v]
        L.lm_head_ce_workspace_bytes.argtypes = [i, i, i, i, i]
        L.lm_head_ce_workspace_bytes.restype = z
        L.adamw_update.argtypes = [v, v, v, v, v, ctypes.c_longlong, f, f, f, f, f, i, i, i, v]
        L.dtb_strerror.argtypes = [i]
        L.dtb_strerror.restype = ctypes.c_char_p
        L.dtb_version.restype = ctypes.c_char_p
        L.dtb_debug_enable.argtypes = [i]
        L.dtb_timing_enable.argtypes = [i]
        L.dtb_timing_collect.argtypes = [ctypes.POINTER(Timing), i]
        _lib = L
    return _lib


def check(rc: int, what: str = "") -> None:
    if rc != DTB_OK:
        msg = lib().dtb_strerror(rc).decode()
        raise DtbError(f"{what}: {ERRORS.get(rc, rc)}: {msg}")


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_cfg(c, B=None, T=None) -> BlockCfg:
    """BlockCfg from any object with the workload attributes."""
    return BlockCfg(B=c.B if B is None else B, T=c.T if T is None else T, C=c.C, NH=c.NH, NKV=c.NKV, H=c.H,
                    norm=NORM[c.norm], mlp=MLP[c.mlp], rope=ROPE[c.rope], rope_base=float(c.rope_base),
                    eps=float(c.eps), qkv_bias=int(c.qkv_bias), o_bias=int(c.o_bias),
                    mlp_bias=int(c.mlp_bias), dtype=DTYPE[c.dtype])


def weights_struct(w: dict) -> BlockWeights:
    """The block's weights; the optional key "rope_cs" is a table from
    rope_table_build (absent: each call computes it)."""
    return BlockWeights(**{n: _ptr(w.get(n)) for n in _WNAMES + ("rope_cs",)})


def grads_struct(g: dict) -> BlockGrads:
    return BlockGrads(**{n: _ptr(g.get(n)) for n in _WNAMES})


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def attn_forward(out, lse, qkv, B, T, C, NH, NKV, dtype, stream=None):
    check(lib().attn_forward(_ptr(out), _ptr(lse), _ptr(qkv), B, T, C, NH, NKV, DTYPE[dtype], _stream(stream)),
          "attn_forward")


def attn_workspace_bytes(B, T, NH) -> int:
    return lib().attn_workspace_bytes(B, T, NH)


def attn_backward(dqkv, qkv, out, dout, lse, B, T, C, NH, NKV, dtype, workspace, stream=None):
    check(lib().attn_backward(_ptr(dqkv), _ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), B, T, C, NH, NKV,
                              DTYPE[dtype], _ptr(workspace), _stream(stream)), "attn_backward")


def attn_backward_noalloc(dqkv, qkv, out, dout, lse, B, T, C, NH, NKV, dtype, stream=None):
    check(lib().attn_backward_noalloc(_ptr(dqkv), _ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), B, T, C, NH, NKV,
                                      DTYPE[dtype], _stream(stream)), "attn_backward_noalloc")


def attn_decode_workspace_bytes(B, NH, NKV, hd, Tmax, chunk, dtype) -> int:
    return lib().attn_decode_workspace_bytes(B, NH, NKV, hd, Tmax, chunk, DTYPE[dtype])


def attn_decode(out, lse, q, k_cache, v_cache, lens, B, NH, NKV, hd, Tmax, chunk, dtype, workspace, stream=None):
    check(lib().attn_decode(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), B, NH, NKV,
                            hd, Tmax, chunk, DTYPE[dtype], _ptr(workspace), _stream(stream)), "attn_decode")


def attn_decode_strided(out, lse, q, k_cache, v_cache, lens, B, NH, NKV, hd, Tmax, stride_b, stride_t, stride_h,
                        chunk, dtype, workspace, stream=None):
    check(lib().attn_decode_strided(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), B, NH,
                                    NKV, hd, Tmax, stride_b, stride_t, stride_h, chunk, DTYPE[dtype],
                                    _ptr(workspace), _stream(stream)), "attn_decode_strided")


def linear_forward(out, inp, w, bias, res, R, K, N, dtype, stream=None):
    check(lib().linear_forward(_ptr(out), _ptr(inp), _ptr(w), _ptr(bias), _ptr(res), R, K, N, DTYPE[dtype],
                               _stream(stream)), "linear_forward")


def linear_workspace_bytes(R, K, N, dtype) -> int:
    return lib().linear_workspace_bytes(R, K, N, DTYPE[dtype])


def linear_backward(dinp, dw, db, dout, inp, w, R, K, N, dtype, workspace, stream=None):
    check(lib().linear_backward(_ptr(dinp), _ptr(dw), _ptr(db), _ptr(dout), _ptr(inp), _ptr(w), R, K, N,
                                DTYPE[dtype], _ptr(workspace), _stream(stream)), "linear_backward")


def encoder_forward(x, ids, wte, wpe, B, T, C, V, dtype, stream=None):
    check(lib().encoder_forward(_ptr(x), _ptr(ids), _ptr(wte), _ptr(wpe), B, T, C, V, DTYPE[dtype], _stream(stream)),
          "encoder_forward")


def encoder_backward(dwte, dwpe, ids, dx, B, T, C, V, dtype, stream=None):
    check(lib().encoder_backward(_ptr(dwte), _ptr(dwpe), _ptr(ids), _ptr(dx), B, T, C, V, DTYPE[dtype],
                                 _stream(stream)), "encoder_backward")


def norm_forward(out, rstd, mean, x, g, b, R, C, norm, eps, dtype, stream=None):
    check(lib().norm_forward(_ptr(out), _ptr(rstd), _ptr(mean), _ptr(x), _ptr(g), _ptr(b), R, C, NORM[norm],
                             float(eps), DTYPE[dtype], _stream(stream)), "norm_forward")


def norm_workspace_bytes(R, C) -> int:
    return lib().norm_workspace_bytes(R, C)


def norm_backward(dx, dg, db, dy, x, g, rstd, mean, dres, R, C, norm, dtype, workspace, stream=None):
    check(lib().norm_backward(_ptr(dx), _ptr(dg), _ptr(db), _ptr(dy), _ptr(x), _ptr(g), _ptr(rstd), _ptr(mean),
                              _ptr(dres), R, C, NORM[norm], DTYPE[dtype], _ptr(workspace), _stream(stream)),
          "norm_backward")


def activation_forward(h, up, R, H, mlp, dtype, stream=None):
    check(lib().activation_forward(_ptr(h), _ptr(up), R, H, MLP[mlp], DTYPE[dtype], _stream(stream)),
          "activation_forward")


def activation_backward(dup, dh, up, R, H, mlp, dtype, stream=None):
    check(lib().activation_backward(_ptr(dup), _ptr(dh), _ptr(up), R, H, MLP[mlp], DTYPE[dtype], _stream(stream)),
          "activation_backward")


def lm_head_forward(logits, ldl, inp, w, R, C, V, dtype, stream=None):
    check(lib().lm_head_forward(_ptr(logits), ldl, _ptr(inp), _ptr(w), R, C, V, DTYPE[dtype], _stream(stream)),
          "lm_head_forward")


def lm_head_workspace_bytes(R, C, V, dtype) -> int:
    return lib().lm_head_workspace_bytes(R, C, V, DTYPE[dtype])


def lm_head_backward(dinp, dw, dlogits, ldl, inp, w, R, C, V, dtype, workspace, stream=None):
    check(lib().lm_head_backward(_ptr(dinp), _ptr(dw), _ptr(dlogits), ldl, _ptr(inp), _ptr(w), R, C, V,
                                 DTYPE[dtype], _ptr(workspace), _stream(stream)), "lm_head_backward")


def softmax_ce(loss, row_loss, dlogits, logits, ldl, targets, R, V, scale, dtype, stream=None):
    check(lib().softmax_ce(_ptr(loss), _ptr(row_loss), _ptr(dlogits), _ptr(logits), ldl, _ptr(targets), R, V,
                           float(scale), DTYPE[dtype], _stream(stream)), "softmax_ce")


def lm_head_ce(loss, row_loss, dinp, dw, inp, w, targets, R, C, V, vchunk, scale, dtype, workspace, stream=None):
    check(lib().lm_head_ce(_ptr(loss), _ptr(row_loss), _ptr(dinp), _ptr(dw), _ptr(inp), _ptr(w), _ptr(targets), R, C,
                           V, vchunk, float(scale), DTYPE[dtype], _ptr(workspace), _stream(stream)), "lm_head_ce")


def lm_head_mtp_ce(loss, row_loss, dinp, dw, inp, w, targets, R, C, V, K, vchunk, scale, dtype, workspace,
                   stream=None):
    check(lib().lm_head_mtp_ce(_ptr(loss), _ptr(row_loss), _ptr(dinp), _ptr(dw), _ptr(inp), _ptr(w), _ptr(targets),
                               R, C, V, K, vchunk, ctypes.c_float(scale), DTYPE[dtype], _ptr(workspace),
                               _stream(stream)), "lm_head_mtp_ce")


def lm_head_ce_workspace_bytes(R, C, V, vchunk, dtype) -> int:
    return lib().lm_head_ce_workspace_bytes(R, C, V, vchunk, DTYPE[dtype])


def adamw_update(params, grads, m, v, params_lowp, n, lr, beta1, beta2, eps, weight_decay, step, lowp_dtype="bf16",
                 zero_grads=True, stream=None):
    check(lib().adamw_update(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), _ptr(params_lowp), int(n), float(lr),
                             float(beta1), float(beta2), float(eps), float(weight_decay), int(step),
                             DTYPE[lowp_dtype], int(bool(zero_grads)), _stream(stream)), "adamw_update")


def block_saved_bytes(cfg: BlockCfg) -> int:
    return lib().block_saved_bytes(ctypes.byref(cfg))


def block_workspace_bytes(cfg: BlockCfg) -> int:
    return lib().block_workspace_bytes(ctypes.byref(cfg))


def block_saved_layout(cfg: BlockCfg) -> SavedLayout:
    L = SavedLayout()
    check(lib().block_saved_layout(ctypes.byref(cfg), ctypes.byref(L)), "block_saved_layout")
    return L


def block_workspace_layout(cfg: BlockCfg) -> WorkspaceLayout:
    L = WorkspaceLayout()
    check(lib().block_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)), "block_workspace_layout")
    return L


def rope_table_build(cs, T, hd, base, stream=None):
    """cs (T * hd fp32, device): the NeoX (cos, sin) table for T positions of head width hd."""
    check(lib().rope_table_build(_ptr(cs), T, hd, base, _stream(stream)), "rope_table_build")


def block_forward(cfg: BlockCfg, weights: dict, x_in, x_out, saved, workspace, stream=None):
    w = weights_struct(weights)
    check(lib().block_forward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x_in), _ptr(x_out), _ptr(saved),
                              _ptr(workspace), _stream(stream)), "block_forward")


def block_backward(cfg: BlockCfg, weights: dict, x_in, saved, dx_out, dx_in, grads: dict, workspace, stream=None):
    w = weights_struct(weights)
    g = grads_struct(grads)
    check(lib().block_backward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x_in), _ptr(saved), _ptr(dx_out),
                               _ptr(dx_in), ctypes.byref(g), _ptr(workspace), _stream(stream)), "block_backward")


def dtb_overlap_create():
    """A caller-owned second stream (and its two events) on the current
    device, for block_backward_overlap; release it with dtb_overlap_destroy."""
    h = _VP()
    check(lib().dtb_overlap_create(ctypes.byref(h)), "dtb_overlap_create")
    return h


def dtb_overlap_destroy(h) -> None:
    check(lib().dtb_overlap_destroy(h), "dtb_overlap_destroy")


def block_backward_overlap(cfg: BlockCfg, weights: dict, x_in, saved, dx_out, dx_in, grads: dict, workspace, side,
                           stream=None):
    w = weights_struct(weights)
    g = grads_struct(grads)
    check(lib().block_backward_overlap(ctypes.byref(cfg), ctypes.byref(w), _ptr(x_in), _ptr(saved), _ptr(dx_out),
                                       _ptr(dx_in), ctypes.byref(g), _ptr(workspace), _stream(stream), side),
          "block_backward_overlap")


def dtb_debug_enable(level: int) -> None:
    """0: off; 1: check and wait after every kernel; 2: also log each kernel."""
    check(lib().dtb_debug_enable(int(level)), "dtb_debug_enable")


TIMING_CLASSES = ["gemm_fwd", "attn_fwd", "attn_bwd", "elementwise", "gemm_dinp", "gemm_dw", "attn_decode",
                  "decode_merge"]


def timing_enable(on: bool = True, classes=None) -> None:
    """Per-class kernel timing: every class (on), none (not on), or only the
    named classes."""
    if classes is not None:
        mask = sum(1 << TIMING_CLASSES.index(c) for c in classes)
    else:
        mask = -1 if on else 0
    lib().dtb_timing_enable(mask)


def timing_collect():
    names = TIMING_CLASSES
    arr = (Timing * len(names))()
    n = lib().dtb_timing_collect(arr, len(names))
    return {names[i]: {"ms": arr[i].ms, "flops": arr[i].flops, "bytes": arr[i].bytes,
                       "launches": arr[i].launches} for i in range(n)}
