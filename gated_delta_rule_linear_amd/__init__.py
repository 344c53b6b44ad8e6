"""Causal linear-attention state recurrence (KATH / GLA / Gated DeltaNet) on MI355X.

The compute path is the C-ABI library ``liblinattn.so`` (hand-written HIP
kernels for gfx950); ``binding`` marshals torch tensors into it. Importing
this package does not load the library; the first call of ``prefill`` /
``decode_step`` does, and raises if it is missing.
"""
from __future__ import annotations

__all__ = ["prefill", "decode_step", "prefill_workspace_bytes", "LinAttnError", "binding",
           "workloads"]


def __getattr__(name):
    if name in ("prefill", "decode_step", "prefill_workspace_bytes", "LinAttnError"):
        from . import binding
        return getattr(binding, name)
    if name in ("binding", "workloads"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
