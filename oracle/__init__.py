"""fp64 CPU oracle for the causal linear-attention state recurrence and the selective scan.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The GPU library never imports this
package, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (token-by-token fp64 recurrence; see the
header of that file for the equations and the pages they come from). This
module is ctypes marshalling: it builds ``liboracle.so`` when it is missing,
checks shapes, and passes contiguous float64 arrays.

Pins: every function here is checked against facts fixed by the pages and by
mathematics (explicit masked quadratic form, split/carry invariance, closed
forms, the worked delta-rule example, the hand count, special cases) in
``tests/test_oracle_pins.py``. No part is "parity unpinned" except the
conventions documented alongside the input generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KATH, GLA, GDN, KDA, SSD = 0, 1, 2, 3, 4
VARIANTS = {"kath": KATH, "gla": GLA, "gdn": GDN, "kda": KDA, "ssd": SSD}


class _Counts(ctypes.Structure):
    _fields_ = [
        ("state_update_macs", ctypes.c_uint64),
        ("state_read_macs", ctypes.c_uint64),
        ("norm_update_adds", ctypes.c_uint64),
        ("norm_read_macs", ctypes.c_uint64),
        ("tokens", ctypes.c_uint64),
    ]


@dataclass
class Counts:
    state_update_macs: int
    state_read_macs: int
    norm_update_adds: int
    norm_read_macs: int
    tokens: int


def compile_library(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle C source into a shared library (gcc, fp64, OpenMP)."""
    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
        "-fno-fast-math", src, "-o", out, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return out


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is not there)."""
    path = path or _LIB
    if path in _lib_cache:
        return _lib_cache[path]
    if path == _LIB and not os.path.exists(_LIB):
        compile_library()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_prefill.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_double, dp, dp, dp, i, ctypes.POINTER(_Counts)]
    lib.oracle_prefill.restype = i
    lib.oracle_decode_step.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, ctypes.c_double,
                                       dp, dp, dp, i]
    lib.oracle_decode_step.restype = i
    lib.oracle_prefill_backward.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp,
                                            ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                            dp, i]
    lib.oracle_prefill_backward.restype = i
    lib.oracle_selective_scan.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i, dp, dp, dp,
                                          i]
    lib.oracle_selective_scan.restype = i
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    _lib_cache[path] = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _variant(v) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


def prefill(variant, q, k, v, g=None, beta=None, S0=None, z0=None, eps=1e-6,
            threads: int = 0, lib_path: str | None = None, with_counts: bool = False):
    """Run the token recurrence over whole sequences.

    q, k: [B,H,N,dk]; v: [B,H,N,dv]; g: GLA [B,H,N,dk], GDN alpha [B,H,N] or KDA
    alpha [B,H,N,dk] or SSD decay [B,H,N]; beta: GDN / KDA [B,H,N]; S0: [B,H,dk,dv] or None; z0:
    [B,H,dk] or None (KATH).
    Returns (o [B,H,N,dv], S [B,H,dk,dv], z [B,H,dk] or None[, Counts]).
    """
    lib = load(lib_path)
    vt = _variant(variant)
    q, k, v, g, beta, S0, z0 = map(_f64, (q, k, v, g, beta, S0, z0))
    B, H, N, dk = q.shape
    dv = v.shape[3]
    assert k.shape == (B, H, N, dk) and v.shape == (B, H, N, dv)
    if vt == GLA:
        assert g is not None and g.shape == (B, H, N, dk)
    if vt == GDN:
        assert g is not None and g.shape == (B, H, N)
        assert beta is not None and beta.shape == (B, H, N)
    if vt == KDA:
        assert g is not None and g.shape == (B, H, N, dk)
        assert beta is not None and beta.shape == (B, H, N)
    if vt == SSD:
        assert g is not None and g.shape == (B, H, N)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if z0 is not None:
        assert z0.shape == (B, H, dk)
    o = np.zeros((B, H, N, dv), np.float64)
    S = np.zeros((B, H, dk, dv), np.float64)
    z = np.zeros((B, H, dk), np.float64) if vt == KATH else None
    c = _Counts()
    rc = lib.oracle_prefill(vt, B, H, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(S0), _ptr(z0), float(eps), _ptr(o), _ptr(S), _ptr(z),
                            int(threads), ctypes.byref(c))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    if with_counts:
        return o, S, z, Counts(c.state_update_macs, c.state_read_macs, c.norm_update_adds,
                               c.norm_read_macs, c.tokens)
    return o, S, z


def decode_step(variant, q, k, v, S, g=None, beta=None, z=None, eps=1e-6, threads: int = 0,
                lib_path: str | None = None):
    """One in-place decode step on float64 arrays S [B,H,dk,dv] (and z [B,H,dk] for KATH).

    q, k: [B,H,dk]; v: [B,H,dv]; g: GLA [B,H,dk], GDN alpha [B,H] or KDA alpha
    [B,H,dk]; beta: GDN / KDA [B,H].
    Returns o [B,H,dv]. S and z must be C-contiguous float64 and are updated in place.
    """
    lib = load(lib_path)
    vt = _variant(variant)
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    assert S.dtype == np.float64 and S.flags.c_contiguous
    B, H, dk = q.shape
    dv = v.shape[2]
    assert S.shape == (B, H, dk, dv)
    if vt == KATH:
        assert z is not None and z.dtype == np.float64 and z.flags.c_contiguous
    o = np.zeros((B, H, dv), np.float64)
    rc = lib.oracle_decode_step(vt, B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                float(eps), _ptr(S), _ptr(z), _ptr(o), int(threads))
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    return o


def prefill_backward(variant, q, k, v, g=None, beta=None, S0=None, z0=None, dO=None,
                     dS_final=None, dz_final=None, eps=1e-6, threads: int = 0,
                     lib_path: str | None = None):
    """Reverse-mode gradients of ``prefill`` for the loss with dL/do = dO, dL/dS_final =
    dS_final (and dL/dz_final = dz_final, KATH); None means zero.

    Returns a dict: dq, dk [B,H,N,dk], dv [B,H,N,dv], dg (shaped like g, or None for
    KATH), dbeta [B,H,N] (GDN, KDA) or None, dS0 [B,H,dk,dv], dz0 [B,H,dk] (KATH) or None.
    """
    lib = load(lib_path)
    vt = _variant(variant)
    q, k, v, g, beta, S0, z0, dO, dS_final, dz_final = map(
        _f64, (q, k, v, g, beta, S0, z0, dO, dS_final, dz_final))
    B, H, N, dk = q.shape
    dv = v.shape[3]
    assert dO is not None and dO.shape == (B, H, N, dv)
    if dS_final is not None:
        assert dS_final.shape == (B, H, dk, dv)
    out = {"dq": np.zeros((B, H, N, dk)), "dk": np.zeros((B, H, N, dk)),
           "dv": np.zeros((B, H, N, dv)),
           "dg": None if vt == KATH else np.zeros(g.shape),
           "dbeta": np.zeros((B, H, N)) if vt in (GDN, KDA) else None,
           "dS0": np.zeros((B, H, dk, dv)),
           "dz0": np.zeros((B, H, dk)) if vt == KATH else None}
    rc = lib.oracle_prefill_backward(vt, B, H, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _ptr(beta), _ptr(S0), _ptr(z0), float(eps), _ptr(dO),
                                     _ptr(dS_final), _ptr(dz_final), _ptr(out["dq"]),
                                     _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                     _ptr(out["dbeta"]), _ptr(out["dS0"]), _ptr(out["dz0"]),
                                     int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill_backward rejected its arguments")
    return out


def selective_scan(dt, A, Bm, Cm, x, Dskip=None, dt_bias=None, dt_softplus: bool = False,
                   h0=None, threads: int = 0, lib_path: str | None = None):
    """Mamba-1 selective scan over whole sequences (equations in the header of oracle.c).

    dt, x: [Bt,T,D]; A: [D,n]; Bm, Cm: [Bt,T,n]; Dskip, dt_bias: [D] or None;
    h0: [Bt,D,n] or None. Returns (y [Bt,T,D], hT [Bt,D,n]).
    """
    lib = load(lib_path)
    dt, A, Bm, Cm, x, Dskip, dt_bias, h0 = map(_f64, (dt, A, Bm, Cm, x, Dskip, dt_bias, h0))
    Bt, T, D = x.shape
    n = A.shape[1]
    assert dt.shape == (Bt, T, D) and A.shape == (D, n)
    assert Bm.shape == (Bt, T, n) and Cm.shape == (Bt, T, n)
    if Dskip is not None:
        assert Dskip.shape == (D,)
    if dt_bias is not None:
        assert dt_bias.shape == (D,)
    if h0 is not None:
        assert h0.shape == (Bt, D, n)
    y = np.zeros((Bt, T, D), np.float64)
    hT = np.zeros((Bt, D, n), np.float64)
    rc = lib.oracle_selective_scan(Bt, T, D, n, _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(x),
                                   _ptr(Dskip), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0),
                                   _ptr(y), _ptr(hT), int(threads))
    if rc != 0:
        raise ValueError("oracle_selective_scan rejected its arguments")
    return y, hT


def max_threads(lib_path: str | None = None) -> int:
    return int(load(lib_path).oracle_max_threads())
