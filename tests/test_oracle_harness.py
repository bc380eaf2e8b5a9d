"""Pins of the oracle's model harness: token / position embedding, softmax
cross-entropy, and the whole model (embedding, block stack, final norm, LM
head, mean cross-entropy on shifted targets) as the "nanoeuler — CUDA
kernels" page (encoder_forward_kernel, softmax_ce_cpu, forward_cpu), the
"microgpt.cu" page (forward_position: wte + wpe, embedding RMSNorm, no final
norm) and llm.c's gpt2_forward / gpt2_backward (tied head, wpe, final
LayerNorm) compose it.

1. Embedding forward against plain indexing; backward against numpy's
   unbuffered np.add.at (which also adds repeated ids in position order).
2. Cross-entropy against torch float64 cross_entropy + autograd; closed forms:
   zero logits give ln V, a one-hot-dominant row gives ~0; every gradient row
   sums to zero; a masked row (target -1) has no loss and no gradient.
3. The whole model against an independent torch float64 composition
   differentiated by autograd, for the four workload families, and central
   finite differences of the oracle's own loss.
CPU only."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from test_oracle_block import make_weights, rel, torch_block

rng = np.random.default_rng(7)


def test_embed_forward_is_indexing(orc):
    V, C, B, T = 11, 6, 3, 5
    wte = rng.standard_normal((V, C))
    wpe = rng.standard_normal((T, C))
    ids = rng.integers(0, V, (B, T)).astype(np.int32)
    np.testing.assert_array_equal(orc.embed_forward(ids, wte, wpe), wte[ids] + wpe[None])
    np.testing.assert_array_equal(orc.embed_forward(ids, wte), wte[ids])


def test_embed_backward_scatter_add(orc):
    V, C, B, T = 7, 5, 4, 9          # many repeated ids
    ids = rng.integers(0, V, (B, T)).astype(np.int32)
    dx = rng.standard_normal((B, T, C))
    dwte, dwpe = orc.embed_backward(ids, dx, V, with_wpe=True)
    ref = np.zeros((V, C))
    np.add.at(ref, ids.reshape(-1), dx.reshape(-1, C))
    np.testing.assert_array_equal(dwte, ref)
    np.testing.assert_allclose(dwpe, dx.sum(0), rtol=1e-14, atol=1e-14)
    # total mass is conserved
    np.testing.assert_allclose(dwte.sum(0), dx.reshape(-1, C).sum(0), rtol=1e-12)


def test_softmax_ce_vs_torch(orc):
    R, V = 13, 29
    logits = 3.0 * rng.standard_normal((R, V))
    tgt = rng.integers(0, V, R).astype(np.int32)
    loss, dl, rows = orc.softmax_ce(logits, tgt, 1.0 / R)
    lt = torch.tensor(logits, requires_grad=True)
    lr = F.cross_entropy(lt, torch.tensor(tgt, dtype=torch.long), reduction="mean")
    lr.backward()
    assert abs(loss - lr.item()) < 1e-13
    assert rel(dl, lt.grad.numpy()) < 1e-13
    rr = F.cross_entropy(torch.tensor(logits), torch.tensor(tgt, dtype=torch.long), reduction="none").numpy()
    assert rel(rows, rr) < 1e-13


def test_softmax_ce_closed_forms(orc):
    V = 40
    # zero logits: every row's loss is ln V, the gradient is (1/V - onehot) * scale
    z = np.zeros((3, V))
    tgt = np.array([0, 7, 39], dtype=np.int32)
    loss, dl, rows = orc.softmax_ce(z, tgt, 1.0 / 3)
    np.testing.assert_allclose(rows, np.log(V), rtol=1e-15)
    assert abs(loss - np.log(V)) < 1e-14
    exp = np.full((3, V), 1.0 / V) / 3
    exp[np.arange(3), tgt] -= 1.0 / 3
    np.testing.assert_allclose(dl, exp, rtol=1e-14, atol=1e-16)
    # huge logits (no overflow: the max is subtracted first)
    big = rng.standard_normal((4, V)) + 800.0
    t4 = rng.integers(0, V, 4).astype(np.int32)
    l4, d4, r4 = orc.softmax_ce(big, t4, 0.25)
    assert np.isfinite(l4) and np.all(np.isfinite(d4))
    ref = F.cross_entropy(torch.tensor(big - 800.0), torch.tensor(t4, dtype=torch.long)).item()
    assert abs(l4 - ref) < 1e-12
    # a dominant correct logit: loss ~ exp(-gap) * (V - 1)
    d = np.zeros((1, V)); d[0, 5] = 30.0
    l1, _, _ = orc.softmax_ce(d, np.array([5], dtype=np.int32), 1.0)
    # (lse - logit is formed from two numbers near 30: absolute error ~ 30 eps)
    assert abs(l1 - np.log1p((V - 1) * np.exp(-30.0))) < 1e-13
    # every gradient row sums to zero
    logits = rng.standard_normal((6, V))
    _, dl6, _ = orc.softmax_ce(logits, rng.integers(0, V, 6).astype(np.int32), 0.5)
    np.testing.assert_allclose(dl6.sum(1), 0.0, atol=1e-15)


def test_softmax_ce_masked_rows(orc):
    V = 9
    logits = rng.standard_normal((5, V))
    tgt = np.array([3, -1, 0, -1, 8], dtype=np.int32)
    loss, dl, rows = orc.softmax_ce(logits, tgt, 0.2)
    assert rows[1] == 0.0 and rows[3] == 0.0
    assert not dl[1].any() and not dl[3].any()
    keep = tgt >= 0
    ref = F.cross_entropy(torch.tensor(logits[keep]), torch.tensor(tgt[keep], dtype=torch.long),
                          reduction="sum").item() * 0.2
    assert abs(loss - ref) < 1e-13


# ---------------------------------------------------------------------------
# whole model
# ---------------------------------------------------------------------------
FAMILIES = {
    # microgpt: wpe, embedding RMSNorm without gamma, no final norm, ReLU
    "microgpt": dict(norm="rms_nogamma", mlp="relu", rope="none", bias=False, wpe=True, embed_norm=True,
                     final_norm=False, tied=False),
    # mini-Qwen2: RoPE, QKV bias, final RMSNorm gamma, untied head
    "qwen2": dict(norm="rms", mlp="swiglu", rope="neox", bias=True, wpe=False, embed_norm=False,
                  final_norm=True, tied=False),
    # GPT-2: wpe, LayerNorm, GELU, all biases, tied head
    "gpt2": dict(norm="layer", mlp="gelu_tanh", rope="none", bias=True, wpe=True, embed_norm=False,
                 final_norm=True, tied=True),
    # Llama: RoPE, RMSNorm gamma, SwiGLU, GQA, untied head
    "llama": dict(norm="rms", mlp="swiglu", rope="neox", bias=False, wpe=False, embed_norm=False,
                  final_norm=True, tied=False),
}


def make_model(fam, L=2, B=2, T=6, C=8, NH=2, NKV=1, H=12, V=13, K=1):
    f = FAMILIES[fam]
    c = SimpleNamespace(B=B, T=T, C=C, NH=NH, NKV=NKV, H=H, norm=f["norm"], mlp=f["mlp"], rope=f["rope"],
                        rope_base=1e4 if f["rope"] == "neox" else 0.0, eps=1e-5, qkv_bias=f["bias"],
                        o_bias=f["bias"] and fam == "gpt2", mlp_bias=f["bias"] and fam == "gpt2",
                        wpe=f["wpe"], embed_norm=f["embed_norm"], final_norm=f["final_norm"],
                        tied_head=f["tied"], mtp=K)
    lw = [make_weights(c, scale=0.5) for _ in range(L)]
    hw = {"wte": rng.standard_normal((V, C))}
    if c.wpe:
        hw["wpe"] = 0.5 * rng.standard_normal((T, C))
    if c.final_norm:
        hw["gf"] = 1 + 0.3 * rng.standard_normal(C)
        if c.norm == "layer":
            hw["bf"] = 0.2 * rng.standard_normal(C)
    if not c.tied_head:
        hw["head"] = rng.standard_normal((K * V, C))
    ids = rng.integers(0, V, (B, T + K)).astype(np.int32)
    return c, lw, hw, ids


def torch_model(c, lw, hw, ids):
    """Independent float64 model: torch embedding, the torch block, norms,
    linear head, mean cross_entropy."""
    T, K = c.T, getattr(c, "mtp", 1)
    inp = torch.tensor(ids[:, :T], dtype=torch.long)
    # head j at position t predicts token t + 1 + j
    tgt = torch.stack([torch.tensor(ids[:, 1 + j:T + 1 + j], dtype=torch.long) for j in range(K)], dim=-1)
    x = F.embedding(inp, hw["wte"])
    if c.wpe:
        x = x + hw["wpe"][None]
    if c.embed_norm:
        x = F.rms_norm(x, (c.C,), None, c.eps)
    for w in lw:
        x = torch_block(c, w, x)
    if c.final_norm:
        x = F.layer_norm(x, (c.C,), hw["gf"], hw.get("bf"), c.eps) if c.norm == "layer" else \
            F.rms_norm(x, (c.C,), hw.get("gf"), c.eps)
    logits = F.linear(x, hw["wte"] if c.tied_head else hw["head"])
    V = logits.shape[-1] // K
    return F.cross_entropy(logits.reshape(-1, V), tgt.reshape(-1))


@pytest.mark.parametrize("fam", list(FAMILIES))
def test_model_vs_torch_autograd(orc, fam):
    c, lw, hw, ids = make_model(fam)
    loss, grads, bgrads, ex = orc.model_step(c, lw, hw, ids)
    lwt = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in lw]
    hwt = {k: torch.tensor(v, requires_grad=True) for k, v in hw.items()}
    lt = torch_model(c, lwt, hwt, ids)
    lt.backward()
    assert abs(loss - lt.item()) < 1e-12 * max(1.0, abs(loss))
    assert set(grads) == set(hw)
    for k in hw:
        assert rel(grads[k], hwt[k].grad.numpy()) < 1e-10, k
    for l in range(len(lw)):
        for k in lw[l]:
            assert rel(bgrads[l][k], lwt[l][k].grad.numpy()) < 1e-10, (l, k)


@pytest.mark.parametrize("fam", ["qwen2", "llama"])
def test_model_mtp_vs_torch_autograd(orc, fam):
    """Three prediction heads: the loss is the mean over (position, head)
    pairs, head j predicting token t + 1 + j."""
    c, lw, hw, ids = make_model(fam, K=3)
    loss, grads, bgrads, ex = orc.model_step(c, lw, hw, ids)
    lwt = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in lw]
    hwt = {k: torch.tensor(v, requires_grad=True) for k, v in hw.items()}
    lt = torch_model(c, lwt, hwt, ids)
    lt.backward()
    assert abs(loss - lt.item()) < 1e-12 * max(1.0, abs(loss))
    for k in hw:
        assert rel(grads[k], hwt[k].grad.numpy()) < 1e-10, k
    for l in range(len(lw)):
        for k in lw[l]:
            assert rel(bgrads[l][k], lwt[l][k].grad.numpy()) < 1e-10, (l, k)


def test_mtp_targets_definition(orc):
    ids = np.arange(2 * 9, dtype=np.int32).reshape(2, 9)
    t = orc.mtp_targets(ids, 6, 3)
    for b in range(2):
        for pos in range(6):
            for j in range(3):
                assert t[b, pos, j] == ids[b, pos + 1 + j]


def test_mtp_head_ce_sft_masking_and_closed_form(orc):
    """Masked (position, head) pairs as in supervised fine-tuning (prompt and
    padding targets -1, scale 1 / number of supervised targets) against torch
    float64 autograd; zero head weights give ln V per supervised target."""
    R, C, V, K = 7, 5, 11, 4
    inp = rng.standard_normal((R, C))
    w = rng.standard_normal((K * V, C))
    tgt = rng.integers(0, V, (R, K)).astype(np.int32)
    tgt[:2] = -1          # prompt positions
    tgt[5:, 2:] = -1      # targets past the end of the example
    nsup = int((tgt >= 0).sum())
    loss, rows, dinp, dw, dl = orc.mtp_head_ce(inp, w, tgt, K, 1.0 / nsup)
    it = torch.tensor(inp, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    lg = F.linear(it, wt).reshape(R * K, V)
    ref = F.cross_entropy(lg, torch.tensor(tgt.reshape(-1), dtype=torch.long), ignore_index=-1, reduction="sum") / nsup
    ref.backward()
    assert abs(loss - ref.item()) < 1e-13
    assert rel(dinp, it.grad.numpy()) < 1e-12 and rel(dw, wt.grad.numpy()) < 1e-12
    assert np.all(rows[tgt < 0] == 0)
    loss0, _, dinp0, _, _ = orc.mtp_head_ce(inp, np.zeros_like(w), tgt, K, 1.0 / nsup)
    assert abs(loss0 - np.log(V)) < 1e-14 and not dinp0.any()


@pytest.mark.parametrize("fam", ["microgpt", "gpt2"])
def test_model_finite_difference(orc, fam):
    """Central differences (h = 1e-5) of the oracle's loss against its
    gradients, on sampled entries of every harness tensor and one block
    tensor per layer."""
    c, lw, hw, ids = make_model(fam, L=1, B=2, T=4, C=8, NH=2, NKV=2, H=8, V=7)
    loss, grads, bgrads, _ = orc.model_step(c, lw, hw, ids)
    h = 1e-5

    def f():
        return orc.model_step(c, lw, hw, ids)[0]

    for k, arr, g in [(k, hw[k], grads[k]) for k in hw] + [("L0.wqkv", lw[0]["wqkv"], bgrads[0]["wqkv"])]:
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + h; lp = f()
            flat[i] = old - h; lm = f()
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g.reshape(-1)[i]) < 1e-7 * max(1.0, abs(fd)), (k, i, fd, g.reshape(-1)[i])


def test_model_initial_loss_near_ln_vocab(orc):
    """With small weights the logits are near zero and the loss is ~ ln V (a
    sanity band, as for the workloads' initial loss)."""
    c, lw, hw, ids = make_model("llama", V=50)
    for w in lw:
        for k in w:
            if k.startswith("w"):
                w[k] *= 0.01
    hw["head"] *= 0.001
    loss = orc.model_step(c, lw, hw, ids)[0]
    assert abs(loss - np.log(50)) < 1e-3


# ---------------------------------------------------------------------------
# optimizer
# ---------------------------------------------------------------------------
def test_adamw_vs_torch(orc):
    """Five AdamW steps against torch.optim.AdamW in float64 (decoupled decay,
    which equals the pages' lr * (mhat / (sqrt(vhat) + eps) + wd * p))."""
    n = 1000
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * (0.1 + i) for i in range(5)]
    lr, b1, b2, eps, wd = 3e-3, 0.9, 0.95, 1e-8, 0.1
    pt = torch.tensor(p0.copy(), requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        pt.grad = torch.tensor(g)
        opt.step()
        p, m, v = orc.adamw(p, g, m, v, lr, b1, b2, eps, wd, t)
        assert rel(p, pt.detach().numpy()) < 1e-13, t
    st = opt.state[pt]
    assert rel(m, st["exp_avg"].numpy()) < 1e-13
    assert rel(v, st["exp_avg_sq"].numpy()) < 1e-13


def test_adamw_first_step_closed_form(orc):
    """Step 1 from zero moments: mhat = g, vhat = g^2, so the update is
    lr * (g / (|g| + eps) + wd * p) -- a signed step of lr plus the decay."""
    g = np.array([2.0, -0.5, 1e-3, -7.0])
    p = np.array([1.0, -1.0, 0.5, 0.0])
    lr, wd, eps = 0.01, 0.1, 1e-8
    p1, m1, v1 = orc.adamw(p, g, np.zeros(4), np.zeros(4), lr, 0.9, 0.999, eps, wd, 1)
    np.testing.assert_allclose(p1, p - lr * (g / (np.abs(g) + eps) + wd * p), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12)
