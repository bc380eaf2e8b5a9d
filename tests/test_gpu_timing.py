"""The per-class kernel timing of the C ABI (dtb_timing_enable / _collect):
only the enabled classes are recorded, a unit of several launches (a split
weight-gradient GEMM and its reduction) counts once, the recorded flops are
the algorithmic ones, and the block backward's results do not depend on
whether its weight gradients ran beside the input gradients (timing off) or
on one stream (a backward class timed)."""
import numpy as np
import pytest

from gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


def _linear_pair(R, K, N):
    import torch
    from decoder_only_transformer_block_amd import binding
    x = torch.randn(R, K, device="cuda").bfloat16()
    w = (torch.randn(N, K, device="cuda") * 0.05).bfloat16()
    out = torch.empty(R, N, device="cuda", dtype=torch.bfloat16)
    dinp = torch.empty(R, K, device="cuda", dtype=torch.bfloat16)
    dw = torch.zeros(N, K, device="cuda", dtype=torch.float32)
    ws = torch.empty(binding.linear_workspace_bytes(R, K, N, "bf16"), dtype=torch.uint8, device="cuda")

    def run():
        binding.linear_forward(out, x, w, None, None, R, K, N, "bf16")
        binding.linear_backward(dinp, dw, None, out, x, w, R, K, N, "bf16", ws)
    return run


def test_timing_classes_and_units():
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import binding
    R, K, N = 8192, 2048, 2048   # the weight gradient takes split K plus a reduction
    announce(f"timing classes R={R} K={K} N={N}")
    run = _linear_pair(R, K, N)
    run()
    torch.cuda.synchronize()
    try:
        binding.timing_enable(classes=["gemm_fwd"])
        binding.timing_collect()
        for _ in range(3):
            run()
        t = binding.timing_collect()
        assert t["gemm_fwd"]["launches"] == 3
        assert t["gemm_dinp"]["launches"] == 0 and t["gemm_dw"]["launches"] == 0
        assert t["gemm_fwd"]["flops"] == pytest.approx(3 * 2.0 * R * K * N)
        assert t["gemm_fwd"]["ms"] > 0
        binding.timing_enable(True)
        for _ in range(2):
            run()
        t = binding.timing_collect()
        # one unit per GEMM call: the weight gradient's split reduction is part of it
        assert t["gemm_fwd"]["launches"] == 2
        assert t["gemm_dinp"]["launches"] == 2
        assert t["gemm_dw"]["launches"] == 2
        assert t["gemm_dw"]["flops"] == pytest.approx(2 * 2.0 * R * K * N)
        assert all(t[c]["ms"] > 0 for c in ("gemm_fwd", "gemm_dinp", "gemm_dw"))
        binding.timing_enable(False)
        run()
        torch.cuda.synchronize()
        t = binding.timing_collect()
        assert all(v["launches"] == 0 for v in t.values())
    finally:
        binding.timing_enable(False)


def test_block_backward_same_with_and_without_side_stream():
    """Weight gradients of a block backward with the caller-owned second
    stream in use (block_backward_overlap, timing off), with everything on
    the caller's stream because a backward class is timed, and through the
    single-stream block_backward are bit-identical, as are dx and the other
    gradients."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    from decoder_only_transformer_block_amd.runtime import BlockStack, to_device
    cfg = configs.LLAMA_GQA.replace(B=2, T=512, L=2)
    announce(f"block backward side stream vs one stream {cfg.name} B={cfg.B} T={cfg.T} L={cfg.L}")
    ws = [configs.block_weights(cfg, l) for l in range(cfg.L)]
    x = to_device(configs.block_input(cfg), cfg.dtype)
    dy = to_device(configs.block_dout(cfg), cfg.dtype)
    res = []
    for timed, overlap in ((False, True), (True, True), (False, False)):
        st = BlockStack(cfg, ws, overlap=overlap)
        try:
            if timed:
                binding.timing_enable(classes=["elementwise"])
            st.forward(x)
            dx = st.backward(dy).clone()
            torch.cuda.synchronize()
        finally:
            binding.timing_enable(False)
            binding.timing_collect()
        res.append((dx.float().cpu().numpy(),
                    [{k: v.cpu().numpy() for k, v in g.items()} for g in st.grads]))
        st.close()
    dx0, g0 = res[0]
    for dx1, g1 in res[1:]:
        assert np.array_equal(dx0, dx1)
        for a, b in zip(g0, g1):
            for k in a:
                assert np.array_equal(a[k], b[k]), k


def test_overlap_handle_checks():
    """block_backward_overlap refuses a NULL handle; a handle is created on the
    current device and destroyed without waiting for the host."""
    require_gpu()
    import ctypes
    from decoder_only_transformer_block_amd import binding, configs
    announce("overlap handle checks")
    L = binding.lib()
    c = binding.make_cfg(configs.LLAMA_GQA.replace(B=1, T=64, L=1))
    assert L.block_backward_overlap(ctypes.byref(c), None, None, None, None, None, None, None, None, None) == -2
    h = binding.dtb_overlap_create()
    assert h.value
    binding.dtb_overlap_destroy(h)
    assert L.dtb_overlap_destroy(None) == 0


def test_debug_mode_checks_every_kernel(capfd):
    """dtb_debug_enable: at level 2 every kernel of an attention forward +
    backward is checked, waited for and logged by name; the results are the
    same bits as with debugging off."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import binding
    announce("debug mode: attention forward + backward")
    B, T, NH, NKV, hd = 1, 130, 4, 2, 64
    C, QKV = NH * hd, NH * hd + 2 * NKV * hd
    g = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn(B, T, QKV, device="cuda", generator=g).bfloat16()
    d = torch.randn(B, T, C, device="cuda", generator=g).bfloat16()
    ws = torch.empty(binding.attn_workspace_bytes(B, T, NH), dtype=torch.uint8, device="cuda")
    res = []
    for level in (0, 2):
        out = torch.empty(B, T, C, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(B, NH, T, device="cuda")
        dq = torch.empty_like(q)
        binding.dtb_debug_enable(level)
        try:
            binding.attn_forward(out, lse, q, B, T, C, NH, NKV, "bf16")
            binding.attn_backward(dq, q, out, d, lse, B, T, C, NH, NKV, "bf16", ws)
        finally:
            binding.dtb_debug_enable(0)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone(), dq.clone()))
    err = capfd.readouterr().err
    for name in ("fwd_bf16_kernel", "dq_bf16_kernel", "dkv_bf16_kernel"):
        assert f"{name}" in err and "ok" in err, err[-2000:]
    for a, b in zip(*res):
        assert torch.equal(a, b)
