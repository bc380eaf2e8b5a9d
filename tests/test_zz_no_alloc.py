"""attn_backward_noalloc (HIP, through the C ABI): the attention backward for
callers that cannot allocate, whose scratch lives in a device array inside
the library.  Checked against attn_backward (the entry point with a workspace
argument) on the same inputs, on calls in a row that share the array: a
larger call, then smaller ones (the array keeps the previous call's values,
which must not leak into a smaller problem), both dtypes, and the largest
problem the array holds (B * NH * T = 2^20, long-context head width); plus
the host-side rejection of a problem one sequence too large.  Every result
is also checked against the oracle at the small sizes."""
import numpy as np
import pytest

from gpu_util import TOL, announce, check, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(dtype, B, T, NH, NKV, hd, seed):
    from decoder_only_transformer_block_amd import inputs
    C = NH * hd
    QKV = C + 2 * NKV * hd
    qkv = inputs.tensor(seed, f"noalloc.qkv{B}.{T}.{NH}.{NKV}.{hd}", (B, T, QKV), dtype=dtype)
    dout = inputs.tensor(seed, f"noalloc.dout{B}.{T}.{NH}.{NKV}.{hd}", (B, T, C), dtype=dtype)
    return qkv, dout


def _both(dtype, B, T, NH, NKV, hd, seed=23, qkv=None, dout=None):
    """dqkv from attn_backward_noalloc and from attn_backward on one input."""
    import torch
    from decoder_only_transformer_block_amd import binding
    from decoder_only_transformer_block_amd.runtime import to_device
    C = NH * hd
    QKV = C + 2 * NKV * hd
    if qkv is None:
        qkv, dout = _inputs(dtype, B, T, NH, NKV, hd, seed)
    announce(f"noalloc attention backward dtype={dtype} B={B} T={T} NH={NH} NKV={NKV} hd={hd}")
    q = to_device(qkv, dtype)
    d = to_device(dout, dtype)
    out = torch.empty((B, T, C), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
    binding.attn_forward(out, lse, q, B, T, C, NH, NKV, dtype)
    dq_na = torch.full((B, T, QKV), float("nan"), dtype=q.dtype, device="cuda")
    binding.attn_backward_noalloc(dq_na, q, out, d, lse, B, T, C, NH, NKV, dtype)
    dq_ws = torch.full((B, T, QKV), float("nan"), dtype=q.dtype, device="cuda")
    ws = torch.empty(binding.attn_workspace_bytes(B, T, NH), dtype=torch.uint8, device="cuda")
    binding.attn_backward(dq_ws, q, out, d, lse, B, T, C, NH, NKV, dtype, ws)
    torch.cuda.synchronize()
    return dq_na, dq_ws, qkv, dout


def _against(dtype, B, T, NH, NKV, hd):
    import oracle
    from decoder_only_transformer_block_amd.runtime import to_numpy
    dq_na, dq_ws, qkv, dout = _both(dtype, B, T, NH, NKV, hd)
    a, b = to_numpy(dq_na), to_numpy(dq_ws)
    C = NH * hd
    # the same kernels on the same inputs: the workspace-argument entry's result, bit for bit
    assert np.array_equal(a, b)
    rd = oracle.attn_backward(qkv, dout, B, T, C, NH, NKV)
    check("dqkv", a, rd, TOL[dtype])


def test_noalloc_calls_in_a_row():
    require_gpu()
    # a larger call, then smaller ones on the same device array
    _against("bf16", 2, 300, 8, 2, 64)
    _against("bf16", 1, 100, 4, 2, 64)
    _against("f32", 2, 200, 4, 4, 64)
    _against("f32", 1, 33, 2, 1, 32)


def test_noalloc_largest_problem_then_smaller():
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    # B * NH * T = 2 * 32 * 16384 = 2^20: the array's whole 8 MiB
    cfg = configs.ATTN_LONG
    B, T, NH, NKV, hd = 2, cfg.T, cfg.NH, cfg.NKV, cfg.hd
    assert 8 * B * NH * T == 8 << 20
    g = torch.Generator().manual_seed(5)
    C = NH * hd
    QKV = C + 2 * NKV * hd
    qkv = torch.randn(B, T, QKV, generator=g).bfloat16().float().numpy()
    dout = torch.randn(B, T, C, generator=g).bfloat16().float().numpy()
    dq_na, dq_ws, _, _ = _both("bf16", B, T, NH, NKV, hd, qkv=qkv, dout=dout)
    assert bool(torch.equal(dq_na, dq_ws))
    assert bool(torch.isfinite(dq_na.float()).all())
    del dq_na, dq_ws
    # one sequence more does not fit: refused on the host, nothing launched
    L = binding.lib()
    assert L.attn_backward_noalloc(None, None, None, None, None, B + 1, T, C, NH, NKV, 1, None) == -1
    # and a smaller problem right after the largest one
    _against("bf16", 1, 130, 4, 1, 128)
    torch.cuda.synchronize()
