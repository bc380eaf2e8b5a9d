"""attn_decode (HIP, through the C ABI) against the oracle: one query per
sequence against a KV cache with ragged lengths, element by element, in both
dtypes, at every supported head width, for MHA / GQA / MQA groups (including
groups wider than one wave's 32 head columns, and more kv heads than a
workgroup's eight waves), at chunk boundaries, with empty
caches, and with the rows past each length filled with NaN (they must never
be read).  The full-size case is the benchmark's own workload and launch
configuration, checked on sampled sequences."""
import numpy as np
import pytest

from gpu_util import TOL, announce, check, require_gpu

pytestmark = pytest.mark.gpu


def _run(cfg, chunk=0, fill=np.nan, lens=None):
    import torch
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device, to_numpy
    q, kc, vc, gl = configs.decode_inputs(cfg, fill=fill)
    if lens is not None:  # shorter lengths over fully drawn caches: rows past them go to `fill`
        assert cfg.len_lo == cfg.Tmax
        gl = np.asarray(lens, np.int32)
        for b in range(cfg.B):
            kc[b, gl[b]:] = fill
            vc[b, gl[b]:] = fill
    announce(f"decode {cfg.name} B={cfg.B} Tmax={cfg.Tmax} NH={cfg.NH} NKV={cfg.NKV} hd={cfg.hd} {cfg.dtype} "
             f"chunk={chunk} lens={gl.tolist() if cfg.B <= 12 else '...'}")
    dec = DecodeAttention(cfg.B, cfg.NH, cfg.NKV, cfg.hd, cfg.Tmax, cfg.dtype, chunk=chunk)
    out, lse = dec(to_device(q, cfg.dtype), to_device(kc, cfg.dtype), to_device(vc, cfg.dtype),
                   torch.from_numpy(gl).cuda())
    torch.cuda.synchronize()
    return q, kc, vc, gl, to_numpy(out), to_numpy(lse)


def _oracle(q, kc, vc, lens, cfg):
    import oracle
    kc = np.where(np.isfinite(kc), kc, 0.0)  # the oracle never reads those rows either
    vc = np.where(np.isfinite(vc), vc, 0.0)
    return oracle.attn_decode(q, kc, vc, lens, cfg.NH, cfg.NKV, cfg.hd)


def _cases():
    from decoder_only_transformer_block_amd.configs import DecodeConfig
    base = dict(seed=0xD7B0 + 16)
    out = []
    for dt in ("bf16", "f32"):
        hds = (8, 16, 32, 64, 128) if dt == "bf16" else (4, 8, 16, 32, 64, 128)
        for hd in hds:
            out.append((DecodeConfig(f"hd{hd}_gqa4_{dt}", B=5, Tmax=300, NH=8, NKV=2, hd=hd, dtype=dt, **base), 64))
        out.append((DecodeConfig(f"mha_{dt}", B=3, Tmax=200, NH=6, NKV=6, hd=64, dtype=dt, **base), 0))
        out.append((DecodeConfig(f"mqa_{dt}", B=3, Tmax=257, NH=12, NKV=1, hd=64, dtype=dt, **base), 32))
        out.append((DecodeConfig(f"grp40_{dt}", B=2, Tmax=150, NH=80, NKV=2, hd=32, dtype=dt, **base), 64))
        out.append((DecodeConfig(f"grp3_{dt}", B=4, Tmax=333, NH=12, NKV=4, hd=64, dtype=dt, **base), 0))
        # more kv heads than one workgroup's waves: two groups of eight per position
        out.append((DecodeConfig(f"kv16_{dt}", B=3, Tmax=300, NH=32, NKV=16, hd=64, dtype=dt, **base), 64))
        out.append((DecodeConfig(f"one_chunk_{dt}", B=4, Tmax=1000, NH=8, NKV=2, hd=64, dtype=dt, **base), 1024))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0].name for c in CASES])
def test_decode_parity(case):
    require_gpu()
    cfg, chunk = CASES[case]
    q, kc, vc, lens, out, lse = _run(cfg, chunk=chunk)
    ro, rl = _oracle(q, kc, vc, lens, cfg)
    tol = TOL[cfg.dtype]
    check("out", out, ro, tol)
    check("lse", lse, rl, tol)


def test_decode_chunk_boundaries_and_empty():
    """Lengths 0, 1, at and around multiples of the chunk (64) and of the
    32-position tile, and Tmax itself, in both dtypes."""
    require_gpu()
    from decoder_only_transformer_block_amd.configs import DecodeConfig
    lens = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 256]
    for dt in ("bf16", "f32"):
        cfg = DecodeConfig(f"bounds_{dt}", B=len(lens), Tmax=256, NH=8, NKV=2, hd=64, dtype=dt, seed=0xD7B0 + 17,
                           len_lo=256)
        q, kc, vc, gl, out, lse = _run(cfg, chunk=64, lens=lens)
        ro, rl = _oracle(q, kc, vc, gl, cfg)
        assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
        check("out", out[1:], ro[1:], TOL[dt])
        check("lse", lse[1:], rl[1:], TOL[dt])


def test_decode_invalid_length_gives_nan():
    """A length past the cache capacity is reported as NaN in that sequence
    only; nothing past the caches is read (the kernel skips it)."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device, to_numpy
    cfg = configs.DecodeConfig("invalid_len", B=3, Tmax=96, NH=4, NKV=2, hd=32, dtype="bf16", seed=0xD7B0 + 18)
    q, kc, vc, gl = configs.decode_inputs(cfg)
    bad = gl.copy()
    bad[1] = cfg.Tmax + 5
    announce(f"decode invalid length lens={bad.tolist()}")
    dec = DecodeAttention(cfg.B, cfg.NH, cfg.NKV, cfg.hd, cfg.Tmax, cfg.dtype, chunk=32)
    out, lse = dec(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"), torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    out, lse = to_numpy(out), to_numpy(lse)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    ro, rl = _oracle(q, kc, vc, gl, cfg)
    check("out", out[[0, 2]], ro[[0, 2]], TOL["bf16"])


def test_decode_long_context_hd128():
    """The long-context attention geometry (NH 32, NKV 8, hd 128) decoding
    against caches of up to 16384 positions."""
    require_gpu()
    from decoder_only_transformer_block_amd.configs import DecodeConfig
    cfg = DecodeConfig("decode_long_hd128", B=2, Tmax=16384, NH=32, NKV=8, hd=128, dtype="bf16",
                       seed=0xD7B0 + 19, len_lo=16384)
    q, kc, vc, lens, out, lse = _run(cfg, lens=[16384, 9001])
    ro, rl = _oracle(q, kc, vc, lens, cfg)
    check("out", out, ro, TOL["bf16"])
    check("lse", lse, rl, TOL["bf16"])


def test_decode_full_size_sampled():
    """The benchmark's workload (256 sequences, lengths uniform in [1, 4096],
    Llama-GQA heads, bf16) in its launch configuration; the oracle checks the
    longest, the shortest and a spread of other sequences."""
    require_gpu()
    from decoder_only_transformer_block_amd import configs
    cfg = configs.DECODE_LLAMA_GQA
    q, kc, vc, lens, out, lse = _run(cfg, fill=0.0)
    order = np.argsort(lens)
    pick = sorted(set([int(order[0]), int(order[-1])] + list(range(0, cfg.B, 37))))
    sub = cfg.replace(B=len(pick))
    ro, rl = _oracle(q[pick], kc[pick], vc[pick], lens[pick], sub)
    check("out", out[pick], ro, TOL["bf16"])
    check("lse", lse[pick], rl, TOL["bf16"])
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_decode_workspace_reuse():
    """One workspace (and output buffers) for two calls in a row: 64 long
    ragged sequences, then three short ones (padded to the same buffers with
    empty caches): the second call must read none of the first call's
    leftover chunk partials."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device, to_numpy
    big = configs.DECODE_LLAMA_GQA.replace(B=64, Tmax=2048)
    small = configs.DecodeConfig("small", B=3, Tmax=2048, NH=32, NKV=8, hd=64, dtype="bf16", seed=0xD7B0 + 20,
                                 len_hi=70)
    dec = DecodeAttention(64, 32, 8, 64, 2048, "bf16")
    for cfg in (big, small):
        q, kc, vc, lens = configs.decode_inputs(cfg)
        announce(f"decode reuse B={cfg.B} lens={lens.tolist() if cfg.B <= 8 else '...'}")
        qq = np.zeros((64, 32 * 64), np.float32)
        qq[:cfg.B] = q
        kk = np.zeros((64, 2048, 8 * 64), np.float32)
        vv = np.zeros_like(kk)
        kk[:cfg.B], vv[:cfg.B] = kc, vc
        ll = np.zeros(64, np.int32)
        ll[:cfg.B] = lens
        out, lse = dec(to_device(qq, "bf16"), to_device(kk, "bf16"), to_device(vv, "bf16"), torch.from_numpy(ll).cuda())
        torch.cuda.synchronize()
        ro, rl = _oracle(q, kc, vc, lens, cfg)
        check("out", to_numpy(out)[:cfg.B], ro, TOL["bf16"])
        check("lse", to_numpy(lse)[:cfg.B], rl, TOL["bf16"])
        assert np.all(to_numpy(out)[cfg.B:] == 0) and np.all(np.isneginf(to_numpy(lse)[cfg.B:]))


def _head_major(cache, cfg):
    """[B][Tmax][NKV*hd] -> [B][NKV][Tmax][hd] (the same values)."""
    B, T = cache.shape[0], cache.shape[1]
    return np.ascontiguousarray(cache.reshape(B, T, cfg.NKV, cfg.hd).transpose(0, 2, 1, 3))


HEAD_MAJOR = [("hd64_gqa4_bf16", 64), ("hd64_gqa4_f32", 64), ("hd128_gqa4_bf16", 64), ("hd16_gqa4_f32", 64),
              ("kv16_bf16", 64), ("mqa_bf16", 32), ("grp40_f32", 64), ("one_chunk_bf16", 1024)]


@pytest.mark.parametrize("name,chunk", HEAD_MAJOR, ids=[n for n, _ in HEAD_MAJOR])
def test_decode_head_major(name, chunk):
    """attn_decode_strided on head-major caches [B][NKV][Tmax][hd] holding the
    same values as the position-major caches of attn_decode: the same results
    bit for bit (same chunks, same arithmetic, other addresses), and the oracle
    on the position-major values.  Rows past each length hold NaN in both."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device, to_numpy
    cfg = next(c for c, _ in CASES if c.name == name)
    q, kc, vc, lens, out_pm, lse_pm = _run(cfg, chunk=chunk)
    announce(f"decode head-major {cfg.name} chunk={chunk}")
    dec = DecodeAttention(cfg.B, cfg.NH, cfg.NKV, cfg.hd, cfg.Tmax, cfg.dtype, chunk=chunk, layout="head")
    out, lse = dec(to_device(q, cfg.dtype), to_device(_head_major(kc, cfg), cfg.dtype),
                   to_device(_head_major(vc, cfg), cfg.dtype), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    out, lse = to_numpy(out), to_numpy(lse)
    assert np.array_equal(out, out_pm) and np.array_equal(lse, lse_pm)
    ro, rl = _oracle(q, kc, vc, lens, cfg)
    check("out", out, ro, TOL[cfg.dtype])
    check("lse", lse, rl, TOL[cfg.dtype])


def test_decode_head_major_full_size_sampled():
    """The benchmark's workload with head-major caches, in its launch
    configuration: bit-identical to the position-major call, and the oracle on
    sampled sequences."""
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device, to_numpy
    cfg = configs.DECODE_LLAMA_GQA
    q, kc, vc, lens, out_pm, lse_pm = _run(cfg, fill=0.0)
    announce("decode head-major full size")
    dec = DecodeAttention(cfg.B, cfg.NH, cfg.NKV, cfg.hd, cfg.Tmax, cfg.dtype, layout="head")
    out, lse = dec(to_device(q, cfg.dtype), to_device(_head_major(kc, cfg), cfg.dtype),
                   to_device(_head_major(vc, cfg), cfg.dtype), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    out, lse = to_numpy(out), to_numpy(lse)
    assert np.array_equal(out, out_pm) and np.array_equal(lse, lse_pm)
    pick = sorted(set([int(np.argmin(lens)), int(np.argmax(lens))] + list(range(5, cfg.B, 41))))
    ro, rl = _oracle(q[pick], kc[pick], vc[pick], lens[pick], cfg.replace(B=len(pick)))
    check("out", out[pick], ro, TOL["bf16"])
    check("lse", lse[pick], rl, TOL["bf16"])
