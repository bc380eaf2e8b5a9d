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


NORM_SHAPES = [(333, 520, False),     # two chunks per lane in bf16, a ragged last chunk
               (2500, 2048, True),    # the Llama-GQA width (4 chunks per lane in bf16) with the residual gradient
               (700, 768, True),      # the GPT-2-small width
               (257, 4096, True)]     # the widest fp32 rows (8192 for bf16 below)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", ["rms", "rms_nogamma", "layer"])
@pytest.mark.parametrize("R,C,with_res", NORM_SHAPES + [(129, 8192, True)])
def test_norm_standalone(dtype, norm, R, C, with_res):
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    if C > (8192 if dtype == "bf16" else 4096):
        pytest.skip("wider than the norm kernels' row limit for this dtype")
    announce(f"norm {norm} R={R} C={C} {dtype} residual={with_res}")
    x = inputs.tensor(5, f"x{R}.{C}", (R, C), std=2.0, mean=0.3, dtype=dtype)
    g = inputs.tensor(5, f"g{C}", (C,), std=0.1, mean=1.0, dtype=dtype)
    b = inputs.tensor(5, f"b{C}", (C,), std=0.1, dtype=dtype)
    dy = inputs.tensor(5, f"dy{R}.{C}", (R, C), dtype=dtype)
    res = inputs.tensor(5, f"res{R}.{C}", (R, C), dtype=dtype) if with_res else None
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
                          gd, rstd, mean if norm == "layer" else None, None if res is None else _dev(res, dtype),
                          R, C, norm, dtype, ws)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    ro, rr, rm = oracle.norm_forward(norm, x, None if gd is None else g, b if bd is not None else None)
    check("out", to_numpy(out), ro, tol)
    rdx, rdg, rdb = oracle.norm_backward(norm, dy, x, None if gd is None else g, rr, rm)
    if res is not None:
        rdx = rdx + res.astype(np.float64)
    check("dx", to_numpy(dx), rdx, tol)
    if gd is not None:
        check("dg", to_numpy(dg), rdg, tol)
    if bd is not None:
        check("db", to_numpy(db), rdb, tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mlp", ["swiglu", "relu", "gelu_tanh"])
@pytest.mark.parametrize("R,H", [(37, 64), (1000, 5632)])
def test_activation_standalone(dtype, mlp, R, H):
    """activation_forward / activation_backward through the C ABI against the
    oracle's activation and its backward."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    W = 2 * H if mlp == "swiglu" else H
    announce(f"activation {mlp} R={R} H={H} {dtype}")
    up = inputs.tensor(6, f"act.up{R}.{W}", (R, W), std=2.0, dtype=dtype)
    if mlp == "relu":
        up[:, :8] = 0.0    # the gradient at exactly 0 is 0 (strict >)
    dh = inputs.tensor(6, f"act.dh{R}.{H}", (R, H), dtype=dtype)
    upd = _dev(up, dtype)
    h = torch.full((R, H), float("nan"), dtype=upd.dtype, device="cuda")
    dup = torch.full((R, W), float("nan"), dtype=upd.dtype, device="cuda")
    binding.activation_forward(h, upd, R, H, mlp, dtype)
    binding.activation_backward(dup, _dev(dh, dtype), upd, R, H, mlp, dtype)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    check("h", to_numpy(h), oracle.act_forward(mlp, up, H), tol)
    check("dup", to_numpy(dup), oracle.act_backward(mlp, dh, up, H), tol)


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


@pytest.mark.parametrize("dtype,V,vchunk", [("f32", 1003, 256), ("bf16", 997, 256), ("bf16", 2048, 512),
                                           ("bf16", 700, 0)])
def test_lm_head_ce_chunked(dtype, V, vchunk):
    """The fused, vocabulary-chunked head + cross-entropy against the oracle's
    unfused definition (linear head, softmax cross-entropy, linear backward):
    several chunks with a ragged last one, one chunk, masked targets."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    R, C = 300, 256
    announce(f"lm_head_ce R={R} C={C} V={V} vchunk={vchunk} {dtype}")
    inp = inputs.tensor(4, "inp", (R, C), dtype=dtype)
    w = inputs.tensor(4, "w", (V, C), std=0.1, dtype=dtype)
    tgt = inputs.ids(4, "tgt", R, V)
    tgt[[0, 17, R - 1]] = -1
    inpd, wd = _dev(inp, dtype), _dev(w, dtype)
    loss = torch.empty(1, device="cuda")
    rows = torch.empty(R, device="cuda")
    dinp = torch.empty((R, C), dtype=inpd.dtype, device="cuda")
    dw = torch.zeros((V, C), device="cuda")
    ws = torch.empty(binding.lm_head_ce_workspace_bytes(R, C, V, vchunk, dtype), dtype=torch.uint8, device="cuda")
    binding.lm_head_ce(loss, rows, dinp, dw, inpd, wd, _ids_dev(tgt), R, C, V, vchunk, 1.0 / R, dtype, ws)
    torch.cuda.synchronize()
    rl = oracle.linear_forward(inp, w)
    rloss, rdl, rrows = oracle.softmax_ce(rl, tgt, 1.0 / R)
    rdinp, rdw, _ = oracle.linear_backward(rdl, inp, w)
    tol = TOL[dtype]
    check("row loss", to_numpy(rows), rrows, tol)
    check("loss", to_numpy(loss), np.array([rloss]), tol)
    check("dinp", to_numpy(dinp), rdinp, tol)
    check("dw", to_numpy(dw), rdw, tol)


@pytest.mark.parametrize("dtype,V,K,vchunk,sft", [("f32", 1003, 3, 256, False), ("bf16", 997, 4, 256, True),
                                                   ("bf16", 2048, 2, 512, False), ("f32", 300, 4, 0, True)])
def test_lm_head_mtp_ce(dtype, V, K, vchunk, sft):
    """K prediction heads through the fused, vocabulary-chunked head against
    the oracle's definition (one head GEMM with K*V columns, the softmax
    cross-entropy of every (position, head) row, the head's matmul backward).
    Pretraining: every target live, scale 1/(R K).  Fine-tuning: prompt and
    past-the-end targets masked with -1, scale 1/(supervised targets)."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    R, C = 300, 256
    announce(f"lm_head_mtp_ce R={R} C={C} V={V} K={K} vchunk={vchunk} {dtype} sft={sft}")
    inp = inputs.tensor(5, "inp", (R, C), dtype=dtype)
    w = inputs.tensor(5, "w", (K * V, C), std=0.1, dtype=dtype)
    tgt = inputs.ids(5, "tgt", R * K, V).reshape(R, K)
    if sft:
        tgt[:40] = -1                   # prompt positions
        tgt[250:, 1:] = -1              # targets past the end of the example
        tgt[123, 2] = -1
    scale = 1.0 / max(int((tgt >= 0).sum()), 1) if sft else 1.0 / (R * K)
    inpd, wd = _dev(inp, dtype), _dev(w, dtype)
    loss = torch.empty(1, device="cuda")
    rows = torch.empty(R * K, device="cuda")
    dinp = torch.empty((R, C), dtype=inpd.dtype, device="cuda")
    dw = torch.zeros((K * V, C), device="cuda")
    ws = torch.empty(binding.lm_head_ce_workspace_bytes(R, C, V, vchunk, dtype), dtype=torch.uint8, device="cuda")
    binding.lm_head_mtp_ce(loss, rows, dinp, dw, inpd, wd, _ids_dev(np.ascontiguousarray(tgt)), R, C, V, K, vchunk,
                           scale, dtype, ws)
    torch.cuda.synchronize()
    rloss, rrows, rdinp, rdw, _ = oracle.mtp_head_ce(inp, w, tgt, K, scale)
    tol = TOL[dtype]
    got_rows = to_numpy(rows).reshape(R, K)
    assert np.all(got_rows[tgt < 0] == 0)
    check("row loss", got_rows, rrows, tol)
    check("loss", to_numpy(loss), np.array([rloss]), tol)
    check("dinp", to_numpy(dinp), rdinp, tol)
    check("dw", to_numpy(dw), rdw, tol)


def _models():
    from decoder_only_transformer_block_amd import configs as K
    return {
        "microgpt": K.MICROGPT,
        "mini_qwen2": K.MINI_QWEN2,
        "gpt2_reduced": K.GPT2_SMALL.replace(L=2, B=2, T=100, C=256, NH=4, NKV=4, H=1024, vocab=1003),
        "llama_gqa_reduced": K.LLAMA_GQA.replace(L=2, B=2, T=130, C=512, NH=8, NKV=2, H=1408, vocab=997),
        # multi-token prediction: four heads (nanoeuler's K)
        "mini_qwen2_mtp4": K.MINI_QWEN2.replace(mtp=4),
        "llama_gqa_reduced_mtp3": K.LLAMA_GQA.replace(L=2, B=2, T=130, C=512, NH=8, NKV=2, H=1408, vocab=997,
                                                      mtp=3),
    }


@pytest.mark.parametrize("case,vchunk", [(c, None) for c in ("microgpt", "mini_qwen2", "gpt2_reduced",
                                                               "llama_gqa_reduced")] +
                         [("gpt2_reduced", 256), ("llama_gqa_reduced", 256), ("mini_qwen2_mtp4", None),
                          ("llama_gqa_reduced_mtp3", 256)])
def test_model_parity(case, vchunk):
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import Model, to_numpy
    cfg = _models()[case]
    announce(f"model {case} L={cfg.L} B={cfg.B} T={cfg.T} C={cfg.C} V={cfg.vocab} {cfg.dtype} vchunk={vchunk}")
    lw = [configs.block_weights(cfg, l, perturb=True) for l in range(cfg.L)]
    hw = configs.harness_weights(cfg, perturb=True)
    ids = configs.token_ids(cfg)
    m = Model(cfg, lw, hw, vchunk=vchunk)
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


def test_adamw_update_flat():
    """adamw_update through the C ABI against the oracle over three steps, on a
    ragged length (vector body + scalar tail), with the bf16 storage copy and
    the gradient cleared after each step."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import binding, inputs
    from decoder_only_transformer_block_amd.runtime import to_numpy
    n = 100003
    announce(f"adamw_update n={n}")
    p0 = inputs.tensor(21, "p", (n,), std=0.05)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.95, 1e-8, 0.1
    p = torch.from_numpy(p0.copy()).cuda()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    lowp = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    rp, rm, rv = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 4):
        g0 = inputs.tensor(21, f"g{t}", (n,), std=0.01 * t)
        g = torch.from_numpy(g0).cuda()
        binding.adamw_update(p, g, m, v, lowp, n, lr, b1, b2, eps, wd, t, "bf16", True)
        torch.cuda.synchronize()
        rp, rm, rv = oracle.adamw(rp, g0, rm, rv, lr, b1, b2, eps, wd, t)
        check(f"p[t={t}]", to_numpy(p), rp, 1e-4)
        check(f"m[t={t}]", to_numpy(m), rm, 1e-4)
        check(f"v[t={t}]", to_numpy(v), rv, 1e-4)
        assert not to_numpy(g).any(), "gradient must be cleared"
        assert torch.equal(lowp, p.to(torch.bfloat16)), "bf16 copy must be the rounded master"


@pytest.mark.parametrize("case", ["mini_qwen2", "llama_gqa_reduced"])
def test_model_two_training_steps(case):
    """One full training step (forward, backward, AdamW over the flat buffers)
    followed by a second forward + backward, against the oracle doing the same
    from the GPU's own step-1 gradients.  (The step-1 gradients are checked
    against the oracle in test_model_parity, the optimizer in
    test_adamw_update_flat; feeding the oracle's gradients instead would let
    AdamW's first step, a signed step of lr, turn tolerated bf16 errors on
    near-zero gradients into sign flips.)  bf16 models: the oracle's updated
    parameters are rounded to bf16 for the second forward, as the GPU's storage
    copy is."""
    require_gpu()
    import torch
    import oracle
    from decoder_only_transformer_block_amd import configs, inputs
    from decoder_only_transformer_block_amd.runtime import Model, to_numpy
    cfg = _models()[case]
    announce(f"model two steps {case} {cfg.dtype}")
    lw = [configs.block_weights(cfg, l, perturb=True) for l in range(cfg.L)]
    hw = configs.harness_weights(cfg, perturb=True)
    ids = configs.token_ids(cfg)
    hp = dict(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    m = Model(cfg, lw, hw)
    l1 = float(to_numpy(m.step(_ids_dev(ids)))[0])
    g1 = [{k: to_numpy(v) for k, v in g.items()} for g in m.stack.grads]
    h1 = {k: to_numpy(v) for k, v in m.hgrads.items()}
    m.optimizer_step(**hp)
    l2 = float(to_numpy(m.step(_ids_dev(ids)))[0])
    torch.cuda.synchronize()
    rl1 = oracle.model_step(cfg, lw, hw, ids)[0]
    rnd = (lambda a: inputs.round_bf16(a.astype(np.float32))) if cfg.dtype == "bf16" else (lambda a: a)

    def upd(w, g):
        p, _, _ = oracle.adamw(w, g, np.zeros(w.size), np.zeros(w.size), hp["lr"], hp["beta1"], hp["beta2"],
                               hp["eps"], hp["weight_decay"], 1)
        return rnd(p.reshape(w.shape))
    lw2 = [{k: upd(w[k], g1[l][k]) for k in w} for l, w in enumerate(lw)]
    hw2 = {k: upd(hw[k], h1[k]) for k in hw}
    rl2, rg2, rbg2, _ = oracle.model_step(cfg, lw2, hw2, ids)
    tol = TOL[cfg.dtype]
    print(f"    loss step 1 gpu {l1:.6f} oracle {rl1:.6f}; step 2 gpu {l2:.6f} oracle {rl2:.6f}")
    check("loss1", np.array([l1]), np.array([rl1]), tol)
    check("loss2", np.array([l2]), np.array([rl2]), tol)
    assert abs(rl2 - rl1) > 1e-3 * abs(rl1), "the update must change the loss measurably"
    for k in rg2:
        check(f"d{k}@2", to_numpy(m.hgrads[k]), rg2[k], tol)
    for l in range(cfg.L):
        for k in rbg2[l]:
            check(f"L{l}.d{k}@2", to_numpy(m.stack.grads[l][k]), rbg2[l][k], tol)
