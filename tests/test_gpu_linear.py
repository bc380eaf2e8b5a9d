"""linear_forward / linear_backward (the block's GEMMs, through the C ABI)
against the oracle's linear layer, element by element.  Shapes are chosen so
that every kernel path runs: the 256x256 bf16 kernel for the forward (k-major
operands), the input gradient (n-major weight) and the weight gradient (both
operands m/n-major) with split-K partials and without; the generic kernel;
ragged M, N and K tails; and tiny shapes."""
import numpy as np
import pytest

from gpu_util import TOL, announce, check, require_gpu

pytestmark = pytest.mark.gpu

# (name, R, K, N): out[R, N] = inp[R, K] W[N, K]^T
SHAPES = [
    ("fwd256_ragged", 1100, 136, 6144),     # forward on 5 x 24 tiles of 256 (ragged rows, ragged K slab)
    ("dinp256", 1100, 6144, 136),           # input gradient on 5 x 24 tiles
    # 64-k slabs: three whole groups of five slabs, a tail of one and a ragged
    # last slab (1000 = 15 x 64 + 40); and K shorter than one slab
    ("fwd256_longk", 1100, 1000, 6144),
    ("dinp256_longk", 1100, 6144, 1000),
    ("fwd256_shortk", 1100, 40, 6144),
    ("dw256_split", 600, 520, 776),         # weight gradient M=776, N=520 with split-K
    ("dw256_nosplit", 64, 1024, 2048),      # weight gradient M=2048, N=1024, K=64: one split
    # more than one round of 256 x 256 tiles (ragged rows and columns, 17 x 17 tiles)
    ("rounds_fwd", 4100, 384, 4352),        # forward on 289 tiles
    ("rounds_dinp", 4100, 4352, 384),       # input gradient on 289 tiles
    # the 16x16x32 forward kernel (K a multiple of 64) with ragged rows and
    # columns (9 x 17 tiles; the last tile's rows and weight rows past the end
    # read as zeros by the buffers' record counts): K of three slabs (tail
    # steps only) and of 21 slabs (four groups of five and a tail)
    ("m16_ragged", 2100, 192, 4200),
    ("m16_ragged_longk", 2100, 1344, 4200),
    ("generic_mid", 333, 264, 328),
    ("tiny", 7, 8, 16),
    ("one_row", 1, 64, 8),
]


def _run(dtype, R, K, N, seed=3):
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_device, to_numpy
    tag = f"{R}.{K}.{N}"
    x = inputs.tensor(seed, "lin.x" + tag, (R, K), dtype=dtype)
    w = inputs.tensor(seed, "lin.w" + tag, (N, K), std=0.05, dtype=dtype)
    b = inputs.tensor(seed, "lin.b" + tag, (N,), dtype=dtype)
    res = inputs.tensor(seed, "lin.res" + tag, (R, N), dtype=dtype)
    dy = inputs.tensor(seed, "lin.dy" + tag, (R, N), dtype=dtype)
    announce(f"linear dtype={dtype} R={R} K={K} N={N}")
    X, W, Bb, RS, DY = (to_device(a, dtype) for a in (x, w, b, res, dy))
    out = torch.empty((R, N), dtype=X.dtype, device="cuda")
    binding.linear_forward(out, X, W, Bb, RS, R, K, N, dtype)
    dinp = torch.full((R, K), float("nan"), dtype=X.dtype, device="cuda")
    dw = torch.full((N, K), 0.5, dtype=torch.float32, device="cuda")      # accumulates onto 0.5
    db = torch.full((N,), -0.25, dtype=torch.float32, device="cuda")
    ws = torch.empty(binding.linear_workspace_bytes(R, K, N, dtype), dtype=torch.uint8, device="cuda")
    binding.linear_backward(dinp, dw, db, DY, X, W, R, K, N, dtype, ws)
    torch.cuda.synchronize()
    ref_out = oracle.linear_forward(x, w, b) + res.astype(np.float64)
    r_dinp, r_dw, r_db = oracle.linear_backward(dy, x, w)
    return (to_numpy(out), to_numpy(dinp), to_numpy(dw) - 0.5, to_numpy(db) + 0.25), (ref_out, r_dinp, r_dw, r_db)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,R,K,N", SHAPES)
def test_linear_parity(dtype, name, R, K, N):
    require_gpu()
    got, ref = _run(dtype, R, K, N)
    tol = TOL[dtype]
    for nm, g, r in zip(("out", "dinp", "dw", "db"), got, ref):
        check(nm, g, r, tol)


def test_linear_rejects_bad_shapes():
    require_gpu()
    from decoder_only_transformer_block_amd import binding
    L = binding.lib()
    assert L.linear_forward(None, None, None, None, None, 4, 12, 16, 1, None) == -1   # K % 8
    assert L.linear_forward(None, None, None, None, None, 0, 16, 16, 1, None) == 0    # empty
    assert L.linear_workspace_bytes(4, 16, 16, 7) == 0


@pytest.mark.parametrize("R,K,N,splits", [(8192, 2048, 4096, 2), (8192, 2048, 2048, 4), (4096, 512, 512, 8),
                                           (65536, 256, 256, 16)])
def test_weight_grad_splits(R, K, N, splits):
    """Weight gradients whose row count is split over several workgroups per
    output tile (fp32 partials, then the split reduction into dW, which starts
    at 0.5): shapes on which the split choice takes 2, 4, 8 and 16 splits (read
    back from the workspace size).  Checked on a spread of output rows (dW[n] = sum_r
    dy[r, n] x[r]) against the oracle's linear backward of those rows."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_device, to_numpy
    wsb = binding.linear_workspace_bytes(R, K, N, "bf16")
    # the partials of splits 1 .. S-1 take (splits - 1) x N x K floats (split 0
    # adds into dW directly), then the bias gradient's row-range partials (at
    # most 512 ranges of 16 rows or more) of N floats, each region 256-byte
    # aligned, and 256 bytes of slack
    al = lambda n: (n + 255) // 256 * 256
    parts = min(512, max(1, (R + 15) // 16))
    assert wsb == al((splits - 1) * 4 * N * K) + al(parts * N * 4) + 256, (wsb, splits)
    announce(f"linear weight gradient ({splits} splits) R={R} K={K} N={N} bf16")
    x = inputs.tensor(11, "pw.x", (R, K), dtype="bf16")
    w = inputs.tensor(11, "pw.w", (N, K), std=0.05, dtype="bf16")
    dy = inputs.tensor(11, "pw.dy", (R, N), dtype="bf16")
    X, W, DY = (to_device(a, "bf16") for a in (x, w, dy))
    dw = torch.full((N, K), 0.5, dtype=torch.float32, device="cuda")
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    binding.linear_backward(None, dw, None, DY, X, W, R, K, N, "bf16", ws)
    torch.cuda.synchronize()
    cols = np.unique(np.array([0, 1, 255, 256, 511, 777, 1024, 1500, 2047, 3000, N - 1]) % N)
    _, r_dw, _ = oracle.linear_backward(dy[:, cols], x, w[cols])
    check("dW[cols]", to_numpy(dw)[cols] - 0.5, r_dw, TOL["bf16"])
