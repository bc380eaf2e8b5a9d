"""The model harness on the GPU (through the C ABI) against the oracle:
encoder_forward / encoder_backward, norm_forward / norm_backward on their own,
lm_head_forward / lm_head_backward with a ragged vocabulary and a padded row
stride, softmax_ce (masked rows, in place), and the whole model -- embedding,
block stack, final norm, LM head, mean cross-entropy -- element by element on
the loss and every gradient, for each workload family at sizes the oracle
finishes in seconds."""
import numpy as np
import pytest

from gpu_util import TOL, announce, check, require_gpu

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    from decoder_only_transformer_block_amd.runtime import to_device
    return to_device(a, dtype)


def _ids_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_encoder_forward_backward(dtype):
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    B, T, C, V = 3, 37, 264, 23            # few ids: many repeats
    announce(f"encoder fwd/bwd B={B} T={T} C={C} V={V} {dtype}")
    wte = inputs.tensor(11, "wte", (V, C), std=0.5, dtype=dtype)
    wpe = inputs.tensor(11, "wpe", (T, C), std=0.5, dtype=dtype)
    ids = inputs.ids(11, "ids", B * T, V).reshape(B, T)
    dx = inputs.tensor(11, "dx", (B, T, C), dtype=dtype)
    x = torch.empty((B, T, C), dtype=_dev(wte, dtype).dtype, device="cuda")
    binding.encoder_forward(x, _ids_dev(ids), _dev(wte, dtype), _dev(wpe, dtype), B, T, C, V, dtype)
    dwte = torch.zeros((V, C), device="cuda")
    dwpe = torch.zeros((T, C), device="cuda")
    binding.encoder_backward(dwte, dwpe, _ids_dev(ids), _dev(dx, dtype), B, T, C, V, dtype)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    check("x", to_numpy(x), oracle.embed_forward(ids, wte, wpe), tol)
    rw, rp = oracle.embed_backward(ids, dx, V, with_wpe=True)
    check("dwte", to_numpy(dwte), rw, tol)
    check("dwpe", to_numpy(dwpe), rp, tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", ["rms", "rms_nogamma", "layer"])
def test_norm_standalone(dtype, norm):
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    R, C = 333, 520
    announce(f"norm {norm} R={R} C={C} {dtype}")
    x = inputs.tensor(5, "x", (R, C), std=2.0, mean=0.3, dtype=dtype)
    g = inputs.tensor(5, "g", (C,), std=0.1, mean=1.0, dtype=dtype)
    b = inputs.tensor(5, "b", (C,), std=0.1, dtype=dtype)
    dy = inputs.tensor(5, "dy", (R, C), dtype=dtype)
    gd = None if norm == "rms_nogamma" else _dev(g, dtype)
    bd = _dev(b, dtype) if norm == "layer" else None
    out = torch.empty((R, C), dtype=_dev(x, dtype).dtype, device="cuda")
    rstd = torch.empty(R, device="cuda")
    mean = torch.empty(R, device="cuda")
    xd = _dev(x, dtype)
    binding.norm_forward(out, rstd, mean, xd, gd, bd, R, C, norm, 1e-5, dtype)
    dx = torch.empty_like(out)
    dg = torch.zeros(C, device="cuda")
    db = torch.zeros(C, device="cuda")
    ws = torch.empty(binding.norm_workspace_bytes(R, C), dtype=torch.uint8, device="cuda")
    binding.norm_backward(dx, dg if gd is not None else None, db if bd is not None else None, _dev(dy, dtype), xd,
                          gd, rstd, mean if norm == "layer" else None, None, R, C, norm, dtype, ws)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    ro, rr, rm = oracle.norm_forward(norm, x, None if gd is None else g, b if bd is not None else None)
    check("out", to_numpy(out), ro, tol)
    rdx, rdg, rdb = oracle.norm_backward(norm, dy, x, None if gd is None else g, rr, rm)
    check("dx", to_numpy(dx), rdx, tol)
    if gd is not None:
        check("dg", to_numpy(dg), rdg, tol)
    if bd is not None:
        check("db", to_numpy(db), rdb, tol)


@pytest.mark.parametrize("dtype,V", [("f32", 1003), ("bf16", 997), ("bf16", 2048)])
def test_lm_head_and_softmax_ce(dtype, V):
    """Ragged vocabularies (padded row stride), a masked target, the gradient
    written over the logits in place, and the head's backward products."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    R, C = 300, 256
    ldl = (V + 7) // 8 * 8
    announce(f"lm_head + softmax_ce R={R} C={C} V={V} ldl={ldl} {dtype}")
    inp = inputs.tensor(3, "inp", (R, C), dtype=dtype)
    w = inputs.tensor(3, "w", (V, C), std=0.1, dtype=dtype)
    tgt = inputs.ids(3, "tgt", R, V)
    tgt[[0, 17, R - 1]] = -1                        # masked positions
    inpd, wd = _dev(inp, dtype), _dev(w, dtype)
    # padded columns start non-zero: softmax_ce must ignore them and zero the gradient there
    logits = torch.full((R, ldl), 7.0, dtype=inpd.dtype, device="cuda")
    binding.lm_head_forward(logits, ldl, inpd, wd, R, C, V, dtype)
    torch.cuda.synchronize()
    lg = to_numpy(logits)
    rl = oracle.linear_forward(inp, w)
    tol = TOL[dtype]
    check("logits", lg[:, :V], rl, tol)
    loss = torch.empty(1, device="cuda")
    rows = torch.empty(R, device="cuda")
    binding.softmax_ce(loss, rows, logits, logits, ldl, _ids_dev(tgt), R, V, 1.0 / R, dtype)   # in place
    dinp = torch.empty((R, C), dtype=inpd.dtype, device="cuda")
    dw = torch.zeros((V, C), device="cuda")
    ws = torch.empty(binding.lm_head_workspace_bytes(R, C, V, dtype), dtype=torch.uint8, device="cuda")
    binding.lm_head_backward(dinp, dw, logits, ldl, inpd, wd, R, C, V, dtype, ws)
    torch.cuda.synchronize()
    # the oracle's cross-entropy on the GPU's own logits (the head was checked above)
    rloss, rdl, rrows = oracle.softmax_ce(lg[:, :V], tgt, 1.0 / R)
    check("row loss", to_numpy(rows), rrows, tol)
    check("loss", to_numpy(loss), np.array([rloss]), tol)
    dl = to_numpy(logits)
    check("dlogits", dl[:, :V], rdl, tol)
    assert not dl[:, V:].any(), "padded gradient columns must be zero"
    assert not dl[[0, 17, R - 1]].any(), "masked rows must have a zero gradient"
    rdinp, rdw, _ = oracle.linear_backward(dl[:, :V], inp, w)
    check("dinp", to_numpy(dinp), rdinp, tol)
    check("dw", to_numpy(dw), rdw, tol)


def _models():
    from decoder_only_transformer_block_amd import configs as K
    return {
        "microgpt": K.MICROGPT,
        "mini_qwen2": K.MINI_QWEN2,
        "gpt2_reduced": K.GPT2_SMALL.replace(L=2, B=2, T=100, C=256, NH=4, NKV=4, H=1024, vocab=1003),
        "llama_gqa_reduced": K.LLAMA_GQA.replace(L=2, B=2, T=130, C=512, NH=8, NKV=2, H=1408, vocab=997),
    }


@pytest.mark.parametrize("case", list(_models()))
def test_model_parity(case):
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import Model, to_numpy
    cfg = _models()[case]
    announce(f"model {case} L={cfg.L} B={cfg.B} T={cfg.T} C={cfg.C} V={cfg.vocab} {cfg.dtype}")
    lw = [configs.block_weights(cfg, l, perturb=True) for l in range(cfg.L)]
    hw = configs.harness_weights(cfg, perturb=True)
    ids = configs.token_ids(cfg)
    m = Model(cfg, lw, hw)
    loss = m.step(_ids_dev(ids))
    torch.cuda.synchronize()
    rloss, rg, rbg, _ = oracle.model_step(cfg, lw, hw, ids)
    tol = TOL[cfg.dtype]
    print(f"    loss gpu {to_numpy(loss)[0]:.6f} oracle {rloss:.6f} (ln V = {np.log(cfg.vocab):.4f})")
    check("loss", to_numpy(loss), np.array([rloss]), tol)
    assert set(rg) == set(m.hgrads)
    for k in rg:
        check(f"d{k}", to_numpy(m.hgrads[k]), rg[k], tol)
    for l in range(cfg.L):
        for k in rbg[l]:
            check(f"L{l}.d{k}", to_numpy(m.stack.grads[l][k]), rbg[l][k], tol)
