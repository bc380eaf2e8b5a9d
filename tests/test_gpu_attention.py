"""attn_forward / attn_backward (HIP, through the C ABI) against the oracle,
element by element, on seeded inputs: several query/key tiles with ragged
tails, every supported head width, MHA / GQA / MQA, T = 1, and B = 0."""
import numpy as np
import pytest

from gpu_util import TOL, announce, check, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, T, NH, NKV, hd
    ("f32", 1, 16, 4, 4, 4),       # microgpt shape
    ("f32", 1, 64, 1, 1, 16),      # mini-Qwen2 shape
    ("f32", 2, 200, 4, 4, 64),     # GPT-2 head width, ragged T
    ("f32", 1, 77, 4, 2, 32),
    ("f32", 2, 33, 6, 3, 8),
    ("f32", 1, 150, 2, 1, 128),
    ("bf16", 2, 200, 8, 2, 64),    # Llama GQA head width
    ("bf16", 1, 300, 8, 2, 128),   # long-context head width
    ("bf16", 1, 129, 4, 4, 32),
    ("bf16", 3, 17, 4, 1, 16),
    ("bf16", 1, 45, 2, 2, 8),
    ("f32", 1, 1, 4, 2, 16),       # T = 1
    ("bf16", 2, 1, 4, 2, 64),
]


def _run(dtype, B, T, NH, NKV, hd, seed=7):
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_device, to_numpy
    C = NH * hd
    QKV = C + 2 * NKV * hd
    qkv = inputs.tensor(seed, f"qkv{B}.{T}.{NH}.{NKV}.{hd}", (B, T, QKV), dtype=dtype)
    dout = inputs.tensor(seed, f"dout{B}.{T}.{NH}.{NKV}.{hd}", (B, T, C), dtype=dtype)
    announce(f"attention dtype={dtype} B={B} T={T} NH={NH} NKV={NKV} hd={hd}")
    q = to_device(qkv, dtype)
    d = to_device(dout, dtype)
    out = torch.empty((B, T, C), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
    dq = torch.full((B, T, QKV), float("nan"), dtype=q.dtype, device="cuda")
    ws = torch.empty(binding.attn_workspace_bytes(B, T, NH), dtype=torch.uint8, device="cuda")
    binding.attn_forward(out, lse, q, B, T, C, NH, NKV, dtype)
    binding.attn_backward(dq, q, out, d, lse, B, T, C, NH, NKV, dtype, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_forward(qkv, B, T, C, NH, NKV)
    rd = oracle.attn_backward(qkv, dout, B, T, C, NH, NKV)
    return (to_numpy(out), to_numpy(lse), to_numpy(dq)), (ro, rl, rd), C


@pytest.mark.parametrize("dtype,B,T,NH,NKV,hd", CASES)
def test_attention_parity(dtype, B, T, NH, NKV, hd):
    require_gpu()
    (o, l, d), (ro, rl, rd), C = _run(dtype, B, T, NH, NKV, hd)
    tol = TOL[dtype]
    check("out", o, ro, tol)
    check("lse", l, rl, tol)
    check("dq", d[..., :C], rd[..., :C], tol)
    check("dk", d[..., C:C + NKV * hd], rd[..., C:C + NKV * hd], tol)
    check("dv", d[..., C + NKV * hd:], rd[..., C + NKV * hd:], tol)


def test_attention_empty_is_noop():
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import binding
    announce("attention B=0 / T=0")
    x = torch.zeros(16, device="cuda")
    binding.attn_forward(x, x, x, 0, 16, 64, 4, 2, "f32")
    binding.attn_forward(x, x, x, 2, 0, 64, 4, 2, "f32")
    binding.attn_backward(x, x, x, x, x, 0, 16, 64, 4, 2, "bf16", x)
    torch.cuda.synchronize()
    assert torch.all(x == 0)
