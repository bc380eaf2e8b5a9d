"""Device buffers for a stack of blocks (torch owns the memory; the library
computes).  Used by the tests, the smoke check and the benchmark."""
from __future__ import annotations

import numpy as np

from . import binding

_TORCH_DTYPE = {}


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """fp32 numpy array (bf16-representable when dtype == 'bf16') -> device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device).to(torch_dtype(dtype)).contiguous()


def to_numpy(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class FlatBuffer:
    """One device allocation holding named tensors as views, each starting on a
    256-byte boundary (so every view passes the library's 16-byte alignment
    check and a kernel can sweep the whole buffer at once)."""

    ALIGN = 64  # elements

    def __init__(self, shapes: dict, torch_dt, device="cuda", zero=True):
        import torch
        self.offsets, off = {}, 0
        for k, shp in shapes.items():
            self.offsets[k] = off
            n = int(np.prod(shp)) if len(shp) else 1
            off += (n + self.ALIGN - 1) // self.ALIGN * self.ALIGN
        self.numel = off
        self.flat = (torch.zeros if zero else torch.empty)(max(off, 1), dtype=torch_dt, device=device)
        self.views = {}
        for k, shp in shapes.items():
            n = int(np.prod(shp)) if len(shp) else 1
            self.views[k] = self.flat[self.offsets[k]:self.offsets[k] + n].view(*shp)


class BlockStack:
    """L blocks of one configuration: weights, fp32 gradients, per-layer saved
    activations and one shared workspace.  weight_views / grad_views (lists of
    dicts of device tensors) place the weights and gradients in buffers the
    caller owns (e.g. views of one flat buffer); otherwise they are allocated
    here."""

    def __init__(self, cfg, layer_weights, device="cuda", weight_views=None, grad_views=None, overlap=True):
        import torch
        self.cfg = cfg
        # overlap: the backward's weight-gradient GEMMs run on a second stream
        # this stack owns (block_backward_overlap); otherwise block_backward
        # runs everything on the caller's stream
        self.overlap = overlap
        self._side = None
        self.c = binding.make_cfg(cfg)
        self.device = device
        if weight_views is None:
            self.weights = [{k: to_device(v, cfg.dtype, device) for k, v in w.items()} for w in layer_weights]
        else:
            self.weights = weight_views
            for w, wv in zip(layer_weights, weight_views):
                for k, v in w.items():
                    wv[k].copy_(to_device(v, cfg.dtype, device))
        if grad_views is None:
            self.grads = [{k: torch.zeros(v.shape, dtype=torch.float32, device=device) for k, v in w.items()}
                          for w in layer_weights]
        else:
            self.grads = grad_views
        nsv = binding.block_saved_bytes(self.c)
        nws = binding.block_workspace_bytes(self.c)
        if nsv == 0 or nws == 0:
            raise binding.DtbError("invalid block configuration")
        self.saved = [torch.empty(nsv, dtype=torch.uint8, device=device) for _ in layer_weights]
        self.workspace = torch.empty(nws, dtype=torch.uint8, device=device)
        # the NeoX rotation table, built once for every layer and step (the
        # block calls would otherwise each compute it)
        self.rope_cs = None
        if cfg.rope == "neox":
            hd = cfg.C // cfg.NH
            self.rope_cs = torch.empty(cfg.T * hd, dtype=torch.float32, device=device)
            binding.rope_table_build(self.rope_cs, cfg.T, hd, cfg.rope_base)
        self.layout = binding.block_saved_layout(self.c)
        shape = (cfg.B, cfg.T, cfg.C)
        td = torch_dtype(cfg.dtype)
        self.acts = [torch.empty(shape, dtype=td, device=device) for _ in range(len(layer_weights) + 1)]
        self.inp = self.acts[0]   # the first block's input (acts[0] unless forward was given x)
        self.dx = torch.empty(shape, dtype=td, device=device)

    @property
    def L(self):
        return len(self.weights)

    def forward(self, x=None, stream=None):
        """x (device tensor [B,T,C]) -> output of the last block.  x is read
        where it is (not copied) and is the input the backward uses: it must
        stay unchanged until then.  Without x, acts[0] is the input."""
        self.inp = x if x is not None else self.acts[0]
        for i in range(self.L):
            xin = self.inp if i == 0 else self.acts[i]
            binding.block_forward(self.c, self._w(i), xin, self.acts[i + 1], self.saved[i], self.workspace, stream)
        return self.acts[self.L]

    def backward(self, dy, stream=None):
        """dy: gradient w.r.t. the last output (only read); returns dx of the
        first input (self.dx).  The top block reads dy and writes self.dx, every
        block below it works in place on self.dx.  Parameter gradients
        accumulate into self.grads."""
        if self.overlap and self._side is None:
            self._side = binding.dtb_overlap_create()
        for i in reversed(range(self.L)):
            xin = self.inp if i == 0 else self.acts[i]
            dout = dy if i == self.L - 1 else self.dx
            if self.overlap:
                binding.block_backward_overlap(self.c, self._w(i), xin, self.saved[i], dout, self.dx,
                                               self.grads[i], self.workspace, self._side, stream)
            else:
                binding.block_backward(self.c, self._w(i), xin, self.saved[i], dout, self.dx, self.grads[i],
                                       self.workspace, stream)
        return self.dx

    def _w(self, i):
        """Layer i's weights as the block calls take them (with the shared table)."""
        return self.weights[i] if self.rope_cs is None else dict(self.weights[i], rope_cs=self.rope_cs)

    def close(self):
        """Release the second stream (its pending work still completes)."""
        if self._side is not None:
            binding.dtb_overlap_destroy(self._side)
            self._side = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def zero_grads(self):
        for g in self.grads:
            for t in g.values():
                t.zero_()

    def workspace_tensor(self, name: str, shape):
        """View of one intermediate gradient the last block_backward left in the
        shared workspace (see dtb_workspace_layout): dh, dup, dn2, dx2, dO,
        dqkv, dn1."""
        import torch
        off = getattr(binding.block_workspace_layout(self.c), name)
        dt = torch_dtype(self.cfg.dtype)
        n = int(np.prod(shape))
        es = torch.tensor([], dtype=dt).element_size()
        return self.workspace[off:off + n * es].view(dt).view(*shape)

    def saved_tensor(self, layer: int, name: str, shape, dtype=None):
        """View of one saved activation (see dtb_saved_layout)."""
        import torch
        off = getattr(self.layout, name)
        if off < 0:
            return None
        dt = dtype or (torch.float32 if name in ("r1", "mu1", "r2", "mu2", "lse") else torch_dtype(self.cfg.dtype))
        n = int(np.prod(shape))
        es = torch.tensor([], dtype=dt).element_size()
        return self.saved[layer][off:off + n * es].view(dt).view(*shape)


class Model:
    """The whole model of one configuration around a BlockStack: token (and
    position) embedding, the embedding RMSNorm (cfg.embed_norm), the block
    stack, the final norm (cfg.final_norm), the LM head (tied to the token
    table if cfg.tied_head) and the mean softmax cross-entropy over the B*T
    positions with targets ids[:, t+1] (with cfg.mtp = K > 1 prediction
    heads: head j predicts ids[:, t+1+j], mean over the B*T*K pairs, through
    the fused head).  Every step runs in libdtb through the C ABI; torch only
    holds the buffers."""

    def __init__(self, cfg, layer_weights, harness_weights: dict, device="cuda", vchunk=None):
        """vchunk None: the head's logits for the whole vocabulary are
        materialised once ([B*T, V]) and overwritten with their gradient;
        an int: the fused, vocabulary-chunked head + cross-entropy
        (lm_head_ce) with chunks of vchunk rows (0: the library's default)."""
        import torch
        self.cfg = cfg
        self.K = getattr(cfg, "mtp", 1)
        if self.K > 1 and vchunk is None:
            vchunk = 0  # several heads: the fused head + cross-entropy
        self.vchunk = vchunk
        td = torch_dtype(cfg.dtype)
        # every parameter (block layers, then the harness) is a view of one
        # flat storage buffer, and every gradient a view of one flat fp32
        # buffer: the optimizer updates them all in one launch
        shapes = {}
        for l, w in enumerate(layer_weights):
            for k, v in w.items():
                shapes[f"L{l}.{k}"] = tuple(v.shape)
        for k, v in harness_weights.items():
            shapes[k] = tuple(v.shape)
        self.wbuf = FlatBuffer(shapes, td, device)
        self.gbuf = FlatBuffer(shapes, torch.float32, device)
        wv = [{k: self.wbuf.views[f"L{l}.{k}"] for k in w} for l, w in enumerate(layer_weights)]
        gv = [{k: self.gbuf.views[f"L{l}.{k}"] for k in w} for l, w in enumerate(layer_weights)]
        self.stack = BlockStack(cfg, layer_weights, device, weight_views=wv, grad_views=gv)
        self.hw = {k: self.wbuf.views[k] for k in harness_weights}
        for k, v in harness_weights.items():
            self.hw[k].copy_(to_device(v, cfg.dtype, device))
        self.hgrads = {k: self.gbuf.views[k] for k in harness_weights}
        self._master_init = (layer_weights, harness_weights)
        self.opt = None
        B, T, C = cfg.B, cfg.T, cfg.C
        self.V = self.hw["wte"].shape[0]
        self.ldl = (self.V + 7) // 8 * 8
        R = B * T
        self.x = torch.empty((B, T, C), dtype=td, device=device)        # embedding output
        self.x0 = torch.empty((B, T, C), dtype=td, device=device)       # after the embedding norm
        self.r0 = torch.empty(R, dtype=torch.float32, device=device)
        self.nf = torch.empty((B, T, C), dtype=td, device=device)       # final norm output
        self.rf = torch.empty(R, dtype=torch.float32, device=device)
        self.mf = torch.empty(R, dtype=torch.float32, device=device)
        self.logits = (torch.empty((R, self.ldl), dtype=td, device=device) if vchunk is None  # dlogits in place
                       else None)
        self.rows = torch.empty(R * self.K, dtype=torch.float32, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.dnf = torch.empty((B, T, C), dtype=td, device=device)
        self.dtop = torch.empty((B, T, C), dtype=td, device=device)
        self.dx = torch.empty((B, T, C), dtype=td, device=device)
        nws = max(binding.norm_workspace_bytes(R, C), binding.lm_head_workspace_bytes(R, C, self.V, cfg.dtype))
        if vchunk is not None:
            nws = max(nws, binding.lm_head_ce_workspace_bytes(R, C, self.V, vchunk, cfg.dtype))
        self.ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=device)

    def _head_w(self):
        return self.hw["wte"] if self.cfg.tied_head else self.hw["head"]

    def step(self, ids, stream=None):
        """ids: int32 device tensor [B, T+K] (K = cfg.mtp).  Forward and
        backward of the whole model; returns the loss tensor [1] (gradients
        accumulate)."""
        import torch
        cfg, s = self.cfg, self.stack
        B, T, C, V, dt, K = cfg.B, cfg.T, cfg.C, self.V, cfg.dtype, self.K
        R = B * T
        inp = ids[:, :T].contiguous()
        # targets [B, T, K]: head j at position t predicts token t+1+j
        tgt = torch.stack([ids[:, 1 + j:T + 1 + j] for j in range(K)], dim=-1).contiguous()
        self._inp = inp
        binding.encoder_forward(self.x, inp, self.hw["wte"], self.hw.get("wpe") if cfg.wpe else None,
                                B, T, C, V, dt, stream)
        x0 = self.x
        if cfg.embed_norm:
            binding.norm_forward(self.x0, self.r0, None, self.x, None, None, R, C, "rms_nogamma", cfg.eps, dt,
                                 stream)
            x0 = self.x0
        h = s.forward(x0, stream)
        nf = h
        if cfg.final_norm:
            binding.norm_forward(self.nf, self.rf, self.mf, h, self.hw.get("gf"), self.hw.get("bf"), R, C,
                                 cfg.norm, cfg.eps, dt, stream)
            nf = self.nf
        dhead = self.hgrads["wte"] if cfg.tied_head else self.hgrads["head"]
        if self.vchunk is None:
            binding.lm_head_forward(self.logits, self.ldl, nf, self._head_w(), R, C, V, dt, stream)
            binding.softmax_ce(self.loss, self.rows, self.logits, self.logits, self.ldl, tgt, R, V, 1.0 / R, dt,
                               stream)
            # backward (self.logits now holds dlogits)
            binding.lm_head_backward(self.dnf, dhead, self.logits, self.ldl, nf, self._head_w(), R, C, V, dt,
                                     self.ws, stream)
        elif K == 1:
            binding.lm_head_ce(self.loss, self.rows, self.dnf, dhead, nf, self._head_w(), tgt, R, C, V, self.vchunk,
                               1.0 / R, dt, self.ws, stream)
        else:
            binding.lm_head_mtp_ce(self.loss, self.rows, self.dnf, dhead, nf, self._head_w(), tgt, R, C, V, K,
                                   self.vchunk, 1.0 / (R * K), dt, self.ws, stream)
        dtop = self.dnf
        if cfg.final_norm:
            binding.norm_backward(self.dtop, self.hgrads.get("gf"), self.hgrads.get("bf"), self.dnf, h,
                                  self.hw.get("gf"), self.rf, self.mf, None, R, C, cfg.norm, dt, self.ws, stream)
            dtop = self.dtop
        g = s.backward(dtop, stream)
        if cfg.embed_norm:
            binding.norm_backward(self.dx, None, None, g, self.x, None, self.r0, None, None, R, C, "rms_nogamma",
                                  dt, self.ws, stream)
            g = self.dx
        binding.encoder_backward(self.hgrads["wte"], self.hgrads.get("wpe") if cfg.wpe else None, inp, g,
                                 B, T, C, V, dt, stream)
        return self.loss

    def zero_grads(self):
        self.gbuf.flat.zero_()

    def optimizer_step(self, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, stream=None):
        """One AdamW step over every parameter (a single launch over the flat
        buffers); the gradients are cleared for the next step.  fp32 models
        update their storage directly; bf16 models keep fp32 master values
        (from the seeded fp32 initial values) and refresh the bf16 storage."""
        import torch
        if self.opt is None:
            n = self.wbuf.numel
            if self.cfg.dtype == "bf16":
                master = FlatBuffer({k: v.shape for k, v in self.wbuf.views.items()}, torch.float32, self.wbuf.flat.device)
                lw, hw = self._master_init
                for l, w in enumerate(lw):
                    for k, v in w.items():
                        master.views[f"L{l}.{k}"].copy_(torch.from_numpy(np.ascontiguousarray(v, np.float32)))
                for k, v in hw.items():
                    master.views[k].copy_(torch.from_numpy(np.ascontiguousarray(v, np.float32)))
                params, lowp = master.flat, self.wbuf.flat
            else:
                params, lowp = self.wbuf.flat, None
            self.opt = {"params": params, "lowp": lowp, "n": n, "t": 0,
                        "m": torch.zeros(n, dtype=torch.float32, device=params.device),
                        "v": torch.zeros(n, dtype=torch.float32, device=params.device)}
        o = self.opt
        o["t"] += 1
        binding.adamw_update(o["params"], self.gbuf.flat, o["m"], o["v"], o["lowp"], o["n"], lr, beta1, beta2, eps,
                             weight_decay, o["t"], "bf16", True, stream)


class DecodeAttention:
    """Buffers of one decode-attention call (one new query per sequence
    against a KV cache of capacity Tmax): the output, the lse and the chunk
    workspace are allocated once; __call__ enqueues attn_decode.  With
    layout="head" the caches are head-major [B][NKV][Tmax][hd] and the call
    goes to attn_decode_strided."""

    def __init__(self, B, NH, NKV, hd, Tmax, dtype, chunk=0, device="cuda", layout="position"):
        import torch
        if layout not in ("position", "head"):
            raise ValueError(f"unknown cache layout {layout!r}")
        self.layout = layout
        self.B, self.NH, self.NKV, self.hd, self.Tmax, self.dtype, self.chunk = B, NH, NKV, hd, Tmax, dtype, chunk
        self.out = torch.empty((B, NH * hd), dtype=torch_dtype(dtype), device=device)
        self.lse = torch.empty((B, NH), dtype=torch.float32, device=device)
        nb = binding.attn_decode_workspace_bytes(B, NH, NKV, hd, Tmax, chunk, dtype)
        if nb == 0:
            raise ValueError("attn_decode: unsupported shape")
        self.ws = torch.empty(nb, dtype=torch.uint8, device=device)

    def __call__(self, q, k_cache, v_cache, lens):
        if self.layout == "head":
            T, hd = self.Tmax, self.hd
            binding.attn_decode_strided(self.out, self.lse, q, k_cache, v_cache, lens, self.B, self.NH, self.NKV,
                                        hd, T, self.NKV * T * hd, hd, T * hd, self.chunk, self.dtype, self.ws)
        else:
            binding.attn_decode(self.out, self.lse, q, k_cache, v_cache, lens, self.B, self.NH, self.NKV, self.hd,
                                self.Tmax, self.chunk, self.dtype, self.ws)
        return self.out, self.lse
