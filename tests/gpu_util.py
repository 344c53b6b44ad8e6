"""Helpers for GPU tests: device copies of generated inputs and the error metric."""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}   # max|gpu - ref| / max|ref| per tensor


def dev(arr: np.ndarray, device="cuda"):
    """float32 array or uint16 bf16 bit patterns -> torch tensor on the GPU."""
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def relerr(gpu, ref) -> float:
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / den) if den > 0 else float(np.max(np.abs(g - r)))


def inputs_to_device(inp):
    return {k: dev(v) for k, v in inp.dev.items()}


def banner(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
