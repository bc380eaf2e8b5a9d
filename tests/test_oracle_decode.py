"""Pins of the oracle's decode attention (one query per sequence against its
KV cache) to things other than itself: torch's scaled_dot_product_attention
in float64, the causal training-attention oracle's newest row, closed forms
and the structural properties of the cache.  CPU only."""
import numpy as np
import torch
import torch.nn.functional as F

rng = np.random.default_rng(4321)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _case(B, Tmax, NH, NKV, hd, lens):
    q = rng.standard_normal((B, NH * hd))
    kc = rng.standard_normal((B, Tmax, NKV * hd))
    vc = rng.standard_normal((B, Tmax, NKV * hd))
    return q, kc, vc, np.asarray(lens, np.int32)


def test_decode_vs_torch_sdpa(orc):
    """Each sequence on its own against torch's attention (float64, the kv
    heads repeated over their query groups, no mask: every cached row is
    visible to the newest query)."""
    B, Tmax, NH, NKV, hd = 5, 37, 6, 2, 8
    lens = [1, 37, 20, 2, 33]
    q, kc, vc, lens = _case(B, Tmax, NH, NKV, hd, lens)
    out, lse = orc.attn_decode(q, kc, vc, lens, NH, NKV, hd)
    for b in range(B):
        n = int(lens[b])
        qt = torch.tensor(q[b].reshape(1, NH, 1, hd))
        kt = torch.tensor(kc[b, :n].reshape(n, NKV, hd)).permute(1, 0, 2)[None]
        vt = torch.tensor(vc[b, :n].reshape(n, NKV, hd)).permute(1, 0, 2)[None]
        kt = kt.repeat_interleave(NH // NKV, dim=1)
        vt = vt.repeat_interleave(NH // NKV, dim=1)
        ref = F.scaled_dot_product_attention(qt, kt, vt).reshape(NH * hd).numpy()
        assert rel(out[b], ref) < 1e-13
        s = (qt @ kt.transpose(-1, -2))[0, :, 0, :].numpy() / np.sqrt(hd)
        ref_lse = torch.logsumexp(torch.tensor(s), dim=-1).numpy()
        assert np.abs(lse[b] - ref_lse).max() < 1e-12


def test_decode_is_newest_row_of_causal_attention(orc):
    """With the cache holding a sequence's keys and values, decoding its last
    position equals the last query row of the causal (training) attention."""
    T, NH, NKV, hd = 19, 4, 2, 16
    C, KV = NH * hd, NKV * hd
    qkv = rng.standard_normal((1, T, C + 2 * KV))
    o, lse = orc.attn_forward(qkv, 1, T, C, NH, NKV)
    for n in (1, 7, T):
        kc = np.zeros((1, T + 3, KV)); vc = np.zeros((1, T + 3, KV))
        kc[0, :n] = qkv[0, :n, C:C + KV]
        vc[0, :n] = qkv[0, :n, C + KV:]
        od, ld = orc.attn_decode(qkv[:, n - 1, :C], kc, vc, [n], NH, NKV, hd)
        assert rel(od[0], o[0, n - 1]) < 1e-13
        assert np.abs(ld[0] - lse[0, :, n - 1]).max() < 1e-13


def test_decode_closed_forms(orc):
    B, Tmax, NH, NKV, hd = 3, 9, 4, 1, 4
    q, kc, vc, _ = _case(B, Tmax, NH, NKV, hd, [0, 0, 0])
    # one cached row: out = v_0, lse = q.k_0 / sqrt(hd)
    out, lse = orc.attn_decode(q, kc, vc, [1, 1, 1], NH, NKV, hd)
    for b in range(B):
        for h in range(NH):
            assert np.array_equal(out[b, h * hd:(h + 1) * hd], vc[b, 0])
            assert abs(lse[b, h] - q[b, h * hd:(h + 1) * hd] @ kc[b, 0] / 2.0) < 1e-14
    # all keys equal: out = mean of the first n values, lse = s + ln n
    k2 = np.repeat(kc[:, :1], Tmax, axis=1)
    lens = np.array([9, 4, 2], np.int32)
    out, lse = orc.attn_decode(q, k2, vc, lens, NH, NKV, hd)
    for b in range(B):
        n = lens[b]
        for h in range(NH):
            assert rel(out[b, h * hd:(h + 1) * hd], vc[b, :n].mean(0)) < 1e-14
            s = q[b, h * hd:(h + 1) * hd] @ kc[b, 0] / 2.0
            assert abs(lse[b, h] - (s + np.log(n))) < 1e-13
    # an empty cache: zero output, lse = -inf
    out, lse = orc.attn_decode(q, kc, vc, [0, 3, 0], NH, NKV, hd)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


def test_decode_ignores_rows_past_length_and_gqa_is_repeated_mha(orc):
    B, Tmax, NH, NKV, hd = 2, 12, 4, 2, 8
    lens = [5, 12]
    q, kc, vc, lens = _case(B, Tmax, NH, NKV, hd, lens)
    out, lse = orc.attn_decode(q, kc, vc, lens, NH, NKV, hd)
    kn, vn = kc.copy(), vc.copy()
    kn[0, 5:] = np.nan
    vn[0, 5:] = np.nan
    o2, l2 = orc.attn_decode(q, kn, vn, lens, NH, NKV, hd)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # GQA == MHA with every kv head repeated over its query group
    rep = lambda c: c.reshape(B, Tmax, NKV, hd).repeat(NH // NKV, axis=2).reshape(B, Tmax, NH * hd)
    om, lm = orc.attn_decode(q, rep(kc), rep(vc), lens, NH, NH, hd)
    assert np.array_equal(out, om) and np.array_equal(lse, lm)
