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


class BlockStack:
    """L blocks of one configuration: weights, fp32 gradients, per-layer saved
    activations and one shared workspace."""

    def __init__(self, cfg, layer_weights, device="cuda"):
        import torch
        self.cfg = cfg
        self.c = binding.make_cfg(cfg)
        self.device = device
        self.weights = [{k: to_device(v, cfg.dtype, device) for k, v in w.items()} for w in layer_weights]
        self.grads = [{k: torch.zeros(v.shape, dtype=torch.float32, device=device) for k, v in w.items()}
                      for w in layer_weights]
        nsv = binding.block_saved_bytes(self.c)
        nws = binding.block_workspace_bytes(self.c)
        if nsv == 0 or nws == 0:
            raise binding.DtbError("invalid block configuration")
        self.saved = [torch.empty(nsv, dtype=torch.uint8, device=device) for _ in layer_weights]
        self.workspace = torch.empty(nws, dtype=torch.uint8, device=device)
        self.layout = binding.block_saved_layout(self.c)
        shape = (cfg.B, cfg.T, cfg.C)
        td = torch_dtype(cfg.dtype)
        self.acts = [torch.empty(shape, dtype=td, device=device) for _ in range(len(layer_weights) + 1)]
        self.dx = torch.empty(shape, dtype=td, device=device)

    @property
    def L(self):
        return len(self.weights)

    def forward(self, x=None, stream=None):
        """x (device tensor [B,T,C]) -> output of the last block."""
        if x is not None:
            self.acts[0].copy_(x)
        for i in range(self.L):
            binding.block_forward(self.c, self.weights[i], self.acts[i], self.acts[i + 1], self.saved[i],
                                  self.workspace, stream)
        return self.acts[self.L]

    def backward(self, dy, stream=None):
        """dy: gradient w.r.t. the last output; returns dx of the first input.
        Parameter gradients accumulate into self.grads."""
        self.dx.copy_(dy)
        for i in reversed(range(self.L)):
            binding.block_backward(self.c, self.weights[i], self.acts[i], self.saved[i], self.dx, self.dx,
                                   self.grads[i], self.workspace, stream)
        return self.dx

    def zero_grads(self):
        for g in self.grads:
            for t in g.values():
                t.zero_()

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
