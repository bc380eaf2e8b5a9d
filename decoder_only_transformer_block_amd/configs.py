"""The five synthetic workloads and their seeded weights/inputs.

Shapes follow the (B, T, C, NH, NKV) problem statement of the flash-attention
kernels on the "nanoeuler — CUDA kernels" page; QKV = C + 2*NKV*(C/NH) is the
packed row width (q heads, then k heads, then v heads).  Weight matrices are
row-major [out, in] as in that page's parameter layout and in llm.c's
train_gpt2.c ParameterTensors.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import inputs

NORMS = {"rms": 0, "rms_nogamma": 1, "layer": 2}
MLPS = {"swiglu": 0, "relu": 1, "gelu_tanh": 2}
ROPES = {"none": 0, "neox": 1}
DTYPES = {"f32": 0, "bf16": 1}


@dataclass(frozen=True)
class BlockConfig:
    name: str
    L: int
    B: int
    T: int
    C: int
    NH: int
    NKV: int
    H: int
    norm: str
    mlp: str
    rope: str
    rope_base: float
    eps: float
    qkv_bias: bool
    o_bias: bool
    mlp_bias: bool
    dtype: str
    vocab: int
    std: float
    seed: int
    # model harness around the block stack: learned position table, an RMSNorm
    # (no gamma) of the embedding, a final norm of the blocks' kind, and an LM
    # head tied to the token embedding
    wpe: bool = False
    embed_norm: bool = False
    final_norm: bool = True
    tied_head: bool = False
    # K prediction heads: head j at position t predicts token t+1+j
    mtp: int = 1

    @property
    def hd(self) -> int:
        return self.C // self.NH

    @property
    def QKV(self) -> int:
        return self.C + 2 * self.NKV * self.hd

    @property
    def BT(self) -> int:
        return self.B * self.T

    @property
    def up_rows(self) -> int:
        return 2 * self.H if self.mlp == "swiglu" else self.H

    def replace(self, **kw) -> "BlockConfig":
        return dataclasses.replace(self, **kw)

    # algorithmic work (forward + backward, one layer) --------------------
    def gemm_flops_per_layer(self) -> float:
        n_mat = 3 if self.mlp == "swiglu" else 2
        fwd_per_tok = 2 * self.C * self.QKV + 2 * self.C * self.C + n_mat * 2 * self.C * self.H
        return 3.0 * fwd_per_tok * self.BT

    def attn_flops_per_layer(self) -> float:
        fwd = 4.0 * self.hd * self.NH * self.T * (self.T + 1) / 2 * self.B
        return fwd * 3.5  # forward + backward (2.5x the forward)


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    T: int
    NH: int
    NKV: int
    hd: int
    dtype: str
    seed: int

    @property
    def C(self) -> int:
        return self.NH * self.hd

    @property
    def QKV(self) -> int:
        return self.C + 2 * self.NKV * self.hd

    def replace(self, **kw) -> "AttnConfig":
        return dataclasses.replace(self, **kw)

    def fwd_flops(self) -> float:
        return 4.0 * self.hd * self.NH * self.T * (self.T + 1) / 2 * self.B


@dataclass(frozen=True)
class DecodeConfig:
    """One decode step of attention: one new query per sequence against a KV
    cache of capacity Tmax whose rows 0 .. len-1 are in use, lengths drawn
    uniformly from [len_lo, len_hi]."""
    name: str
    B: int
    Tmax: int
    NH: int
    NKV: int
    hd: int
    dtype: str
    seed: int
    len_lo: int = 1
    len_hi: int = 0  # 0: Tmax

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


MICROGPT = BlockConfig("microgpt", L=1, B=1, T=16, C=16, NH=4, NKV=4, H=64,
                       norm="rms_nogamma", mlp="relu", rope="none", rope_base=0.0,
                       eps=1e-5, qkv_bias=False, o_bias=False, mlp_bias=False,
                       dtype="f32", vocab=27, std=0.08, seed=0xD7B0 + 1,
                       wpe=True, embed_norm=True, final_norm=False)
MINI_QWEN2 = BlockConfig("mini_qwen2", L=2, B=1, T=64, C=16, NH=1, NKV=1, H=32,
                         norm="rms", mlp="swiglu", rope="neox", rope_base=1e6,
                         eps=1e-5, qkv_bias=True, o_bias=False, mlp_bias=False,
                         dtype="f32", vocab=40, std=0.02, seed=0xD7B0 + 2)
GPT2_SMALL = BlockConfig("gpt2_small", L=12, B=4, T=1024, C=768, NH=12, NKV=12, H=3072,
                         norm="layer", mlp="gelu_tanh", rope="none", rope_base=0.0,
                         eps=1e-5, qkv_bias=True, o_bias=True, mlp_bias=True,
                         dtype="f32", vocab=50257, std=0.02, seed=0xD7B0 + 3,
                         wpe=True, tied_head=True)
LLAMA_GQA = BlockConfig("llama_gqa", L=4, B=8, T=2048, C=2048, NH=32, NKV=8, H=5632,
                        norm="rms", mlp="swiglu", rope="neox", rope_base=1e4,
                        eps=1e-5, qkv_bias=False, o_bias=False, mlp_bias=False,
                        dtype="bf16", vocab=32000, std=0.02, seed=0xD7B0 + 4)
ATTN_LONG = AttnConfig("attn_long", B=1, T=16384, NH=32, NKV=8, hd=128, dtype="bf16",
                       seed=0xD7B0 + 5)

# decode over the Llama-GQA attention geometry: 256 sequences with cache
# lengths uniform in [1, 4096] (about 537 MB of bf16 keys and values in use,
# twice the last-level cache)
DECODE_LLAMA_GQA = DecodeConfig("decode_llama_gqa", B=256, Tmax=4096, NH=32, NKV=8, hd=64, dtype="bf16",
                                seed=0xD7B0 + 6)

BLOCK_CONFIGS = {c.name: c for c in (MICROGPT, MINI_QWEN2, GPT2_SMALL, LLAMA_GQA)}
ALL_CONFIGS = dict(BLOCK_CONFIGS, attn_long=ATTN_LONG)


# ---------------------------------------------------------------------------
# seeded tensors
# ---------------------------------------------------------------------------
WEIGHT_NAMES = ("g1", "b1", "wqkv", "bqkv", "wo", "bo", "g2", "b2",
                "w_up", "b_up", "w_down", "b_down")


def weight_shapes(cfg: BlockConfig) -> dict:
    C, H = cfg.C, cfg.H
    s = {}
    if cfg.norm != "rms_nogamma":
        s["g1"] = (C,)
        s["g2"] = (C,)
    if cfg.norm == "layer":
        s["b1"] = (C,)
        s["b2"] = (C,)
    s["wqkv"] = (cfg.QKV, C)
    if cfg.qkv_bias:
        s["bqkv"] = (cfg.QKV,)
    s["wo"] = (C, C)
    if cfg.o_bias:
        s["bo"] = (C,)
    s["w_up"] = (cfg.up_rows, C)
    if cfg.mlp_bias:
        s["b_up"] = (cfg.up_rows,)
    s["w_down"] = (C, H)
    if cfg.mlp_bias:
        s["b_down"] = (C,)
    return s


def block_weights(cfg: BlockConfig, layer: int, perturb: bool = False) -> dict:
    """Seeded weights of one layer as fp32 arrays (bf16-representable when the
    workload stores bf16).  Matrices ~ N(0, std^2); gammas = 1, betas and
    biases = 0, or with perturb=True gammas ~ 1 + N(0, 0.1^2) and betas/biases
    ~ N(0, 0.02^2) so that those code paths see non-trivial values."""
    out = {}
    for name, shape in weight_shapes(cfg).items():
        tag = f"L{layer}.{name}"
        if name in ("g1", "g2"):
            v = (inputs.tensor(cfg.seed, tag, shape, std=0.1, mean=1.0, dtype=cfg.dtype)
                 if perturb else inputs.const(shape, 1.0))
        elif name.startswith("b"):
            v = (inputs.tensor(cfg.seed, tag, shape, std=0.02, dtype=cfg.dtype)
                 if perturb else inputs.const(shape, 0.0))
        else:
            v = inputs.tensor(cfg.seed, tag, shape, std=cfg.std, dtype=cfg.dtype)
        out[name] = v
    return out


def token_ids(cfg: BlockConfig) -> np.ndarray:
    """T+K ids per sequence for K = cfg.mtp prediction heads (the last K are
    only targets)."""
    n = cfg.T + cfg.mtp
    return inputs.ids(cfg.seed, "ids", cfg.B * n, cfg.vocab).reshape(cfg.B, n)


def block_input(cfg: BlockConfig) -> np.ndarray:
    """x_in of layer 0: rows of the seeded embedding matrix E[vocab, C]
    (N(0, std^2)) picked by the seeded token ids.  [B, T, C] fp32 values."""
    tid = token_ids(cfg)[:, : cfg.T].reshape(-1)
    x = inputs.rows(cfg.seed, "E", tid, cfg.C, cfg.std, dtype=cfg.dtype)
    return x.reshape(cfg.B, cfg.T, cfg.C)


def block_dout(cfg: BlockConfig, std: float = 1.0) -> np.ndarray:
    """Upstream gradient of the top block's output, N(0, std^2), [B, T, C]."""
    return inputs.tensor(cfg.seed, "dy", (cfg.B, cfg.T, cfg.C), std=std, dtype=cfg.dtype)


def harness_weights(cfg: BlockConfig, perturb: bool = False) -> dict:
    """Seeded harness parameters: token embedding 'wte' [vocab, C] (the same
    seeded matrix whose rows block_input picks), position table 'wpe' [T, C],
    final-norm 'gf' / 'bf' and LM head 'head' [mtp*vocab, C] (head j = rows
    j*vocab ..) as the configuration has them.  Matrices ~ N(0, std^2); gamma 1 and beta 0 unless perturb."""
    V, C = cfg.vocab, cfg.C
    out = {"wte": inputs.tensor(cfg.seed, "E", (V, C), std=cfg.std, dtype=cfg.dtype)}
    if cfg.wpe:
        out["wpe"] = inputs.tensor(cfg.seed, "wpe", (cfg.T, C), std=cfg.std, dtype=cfg.dtype)
    if cfg.final_norm and cfg.norm != "rms_nogamma":
        out["gf"] = (inputs.tensor(cfg.seed, "gf", (C,), std=0.1, mean=1.0, dtype=cfg.dtype)
                     if perturb else inputs.const((C,), 1.0))
    if cfg.final_norm and cfg.norm == "layer":
        out["bf"] = (inputs.tensor(cfg.seed, "bf", (C,), std=0.02, dtype=cfg.dtype)
                     if perturb else inputs.const((C,), 0.0))
    if not cfg.tied_head:
        out["head"] = inputs.tensor(cfg.seed, "head", (cfg.mtp * V, C), std=cfg.std, dtype=cfg.dtype)
    return out


def attn_inputs(cfg: AttnConfig):
    """Packed qkv [B, T, QKV] and dout [B, T, C] ~ N(0, 1)."""
    qkv = inputs.tensor(cfg.seed, "qkv", (cfg.B, cfg.T, cfg.QKV), dtype=cfg.dtype)
    dout = inputs.tensor(cfg.seed, "dout", (cfg.B, cfg.T, cfg.C), dtype=cfg.dtype)
    return qkv, dout


def decode_lens(cfg: DecodeConfig) -> np.ndarray:
    """Cache lengths [B] (int32), uniform in [len_lo, len_hi]."""
    hi = cfg.len_hi or cfg.Tmax
    return (cfg.len_lo + inputs.ids(cfg.seed, "lens", cfg.B, hi - cfg.len_lo + 1)).astype(np.int32)


def decode_inputs(cfg: DecodeConfig, fill: float = 0.0):
    """q [B, NH*hd] and k / v caches [B, Tmax, NKV*hd] ~ N(0, 1) in the rows in
    use; rows past a sequence's length hold `fill`.  Returns (q, k, v, lens)."""
    lens = decode_lens(cfg)
    KV = cfg.NKV * cfg.hd
    q = inputs.tensor(cfg.seed, "q", (cfg.B, cfg.NH * cfg.hd), dtype=cfg.dtype)
    caches = []
    for name in ("k_cache", "v_cache"):
        c = np.full((cfg.B, cfg.Tmax, KV), fill, dtype=np.float32)

        def seq(b, c=c, name=name):
            n = int(lens[b])
            if n:
                v = inputs.normal(cfg.seed, name, n * KV, start=b * cfg.Tmax * KV).astype(np.float32)
                c[b, :n] = (inputs.round_bf16(v) if cfg.dtype == "bf16" else v).reshape(n, KV)

        with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
            list(ex.map(seq, range(cfg.B)))
        caches.append(c)
    return q, caches[0], caches[1], lens
