"""Shared helpers of the GPU parity tests (no test functions here)."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible (run with -m 'not gpu' on a CPU host)")
    from decoder_only_transformer_block_amd import binding
    binding.lib()      # raises if libdtb.so is not built


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def check(name, got, ref, tol):
    e = rel_err(got, ref)
    print(f"    {name:10s} rel err {e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: relative error {e:.3e} > {tol:.0e}"
    return e
