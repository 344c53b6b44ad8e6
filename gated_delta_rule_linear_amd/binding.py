"""ctypes binding of ``liblinattn.so`` (declared in ``include/linattn.h``).

Argument marshalling only: torch supplies device memory and the stream, every
step of the computation runs in the library's HIP kernels. If the library is
missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import NamedTuple
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblinattn.so")

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_HIP, LA_ERR_WORKSPACE = 0, 1, 2, 3, 4
LA_KATH, LA_GLA, LA_GDN, LA_KDA, LA_SSD = 0, 1, 2, 3, 4
LA_F32, LA_BF16 = 0, 1
LA_PATH_AUTO, LA_PATH_VALU, LA_PATH_MFMA = 0, 1, 2

VARIANTS = {"kath": LA_KATH, "gla": LA_GLA, "gdn": LA_GDN, "kda": LA_KDA, "ssd": LA_SSD}
PATHS = {"auto": LA_PATH_AUTO, "valu": LA_PATH_VALU, "mfma": LA_PATH_MFMA}
EXPORTS = ("la_prefill", "la_prefill_workspace_size", "la_prefill_noalloc", "la_prefill_varlen",
           "la_prefill_varlen_workspace_size", "la_decode_step", "la_prefill_backward",
           "la_prefill_backward_workspace_size", "la_selective_scan", "la_stream_rmw",
           "la_status_str", "la_abi_version")


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("variant", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32), ("eps", ctypes.c_float),
        ("path", ctypes.c_int32), ("chunk", ctypes.c_int32), ("segments", ctypes.c_int32),
    ]


class ScanDesc(ctypes.Structure):
    _fields_ = [
        ("Bt", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("n", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises FileNotFoundError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                f"`python -m gated_delta_rule_linear_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    lib.la_prefill.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.la_prefill.restype = ctypes.c_int
    lib.la_prefill_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.la_prefill_noalloc.restype = ctypes.c_int
    lib.la_prefill_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    lib.la_prefill_workspace_size.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.la_prefill_varlen.argtypes = [dp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.la_prefill_varlen.restype = ctypes.c_int
    lib.la_prefill_varlen_workspace_size.argtypes = [dp, i32, i32, ctypes.POINTER(sz)]
    lib.la_prefill_varlen_workspace_size.restype = ctypes.c_int
    lib.la_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.la_decode_step.restype = ctypes.c_int
    lib.la_prefill_backward.argtypes = [dp] + [vp] * 18 + [sz, vp]
    lib.la_prefill_backward.restype = ctypes.c_int
    lib.la_prefill_backward_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    lib.la_prefill_backward_workspace_size.restype = ctypes.c_int
    lib.la_selective_scan.argtypes = [ctypes.POINTER(ScanDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp]
    lib.la_selective_scan.restype = ctypes.c_int
    lib.la_stream_rmw.argtypes = [vp, ctypes.c_uint64, ctypes.c_float, vp]
    lib.la_stream_rmw.restype = ctypes.c_int
    lib.la_status_str.argtypes = [ctypes.c_int]
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_abi_version.argtypes = []
    lib.la_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().la_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != LA_OK:
        raise LinAttnError(status, where)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(variant, B, H, N, dk, dv, io_dtype, gate_dtype=LA_F32, eps=1e-6, path="auto",
              chunk=0, segments=0) -> Desc:
    return Desc(B, H, N, dk, dv, VARIANTS[variant] if isinstance(variant, str) else int(variant),
                io_dtype, gate_dtype, float(eps), PATHS[path] if isinstance(path, str) else path,
                chunk, segments)


def _require_contig(name, t):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().la_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "la_prefill_workspace_size")
    return int(n.value)


def prefill(q, k, v, g=None, beta=None, *, variant: str, S0=None, z0=None, eps: float = 1e-6,
            path: str = "auto", chunk: int = 0, segments: int = 0, o=None, S_final=None,
            z_final=None, workspace=None, stream=None):
    """Chunked prefill through ``la_prefill``.

    q, k [B,H,N,dk], v [B,H,N,dv] (float32 or bfloat16, one dtype); g (GLA
    [B,H,N,dk] / GDN alpha [B,H,N] / KDA alpha [B,H,N,dk]) and beta (GDN / KDA
    [B,H,N]) float32 or bfloat16;
    S0 [B,H,dk,dv] and z0 [B,H,dk] float32 or None. Outputs are allocated with
    torch unless given. Returns (o, S_final, z_final or None).
    """
    import torch
    lib = load()
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S0", S0),
                    ("z0", z0), ("o", o), ("S_final", S_final), ("z_final", z_final)):
        _require_contig(name, t)
    io = _dtype_code(q)
    gate_t = g if g is not None else beta
    gd = _dtype_code(gate_t) if gate_t is not None else LA_F32
    desc = make_desc(variant, B, H, N, dk, dv, io, gd, eps, path, chunk, segments)
    dev = q.device
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if z_final is None and desc.variant == LA_KATH:
        z_final = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    ws_bytes = prefill_workspace_bytes(desc)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.la_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                        _ptr(S0), _ptr(z0), _ptr(o), _ptr(S_final), _ptr(z_final),
                        _ptr(workspace if ws_bytes else None), wsz, _stream_handle(stream, dev))
    _check(rc, "la_prefill")
    return o, S_final, z_final


def prefill_varlen(q, k, v, g=None, beta=None, *, variant: str, cu_seqlens, max_seqlen: int,
                   S0=None, z0=None, eps: float = 1e-6, path: str = "auto", segments: int = 0,
                   o=None, S_final=None, z_final=None, workspace=None, stream=None):
    """Packed variable-length prefill through ``la_prefill_varlen``.

    q, k [1,H,N,dk], v [1,H,N,dv] with the sequences concatenated along N; cu_seqlens an
    int32 device tensor [nseq + 1] of cumulative lengths; max_seqlen >= every length.
    g / beta as for ``prefill`` with B = 1. S0 / S_final [nseq,H,dk,dv], z0 / z_final
    [nseq,H,dk]. Returns (o, S_final, z_final or None).
    """
    import torch
    lib = load()
    one, H, N, dk = q.shape
    dv = v.shape[-1]
    nseq = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S0", S0),
                    ("z0", z0), ("o", o), ("S_final", S_final), ("z_final", z_final),
                    ("cu_seqlens", cu_seqlens)):
        _require_contig(name, t)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    io = _dtype_code(q)
    gate_t = g if g is not None else beta
    gd = _dtype_code(gate_t) if gate_t is not None else LA_F32
    desc = make_desc(variant, one, H, N, dk, dv, io, gd, eps, path, 0, segments)
    dev = q.device
    if o is None:
        o = torch.empty((one, H, N, dv), dtype=q.dtype, device=dev)
    if S_final is None:
        S_final = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    if z_final is None and desc.variant == LA_KATH:
        z_final = torch.empty((nseq, H, dk), dtype=torch.float32, device=dev)
    n = ctypes.c_size_t(0)
    _check(lib.la_prefill_varlen_workspace_size(ctypes.byref(desc), nseq, int(max_seqlen),
                                                ctypes.byref(n)), "la_prefill_varlen_workspace_size")
    ws_bytes = int(n.value)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.la_prefill_varlen(ctypes.byref(desc), nseq, _ptr(cu_seqlens), int(max_seqlen),
                               _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(z0),
                               _ptr(o), _ptr(S_final), _ptr(z_final),
                               _ptr(workspace if ws_bytes else None), wsz,
                               _stream_handle(stream, dev))
    _check(rc, "la_prefill_varlen")
    return o, S_final, z_final


def decode_step(q, k, v, S, g=None, beta=None, *, variant: str, z=None, eps: float = 1e-6,
                o=None, stream=None):
    """One in-place decode step through ``la_decode_step``.

    q, k [B,H,dk]; v [B,H,dv]; S [B,H,dk,dv] float32 (updated in place);
    g (GLA [B,H,dk] / GDN alpha [B,H] / KDA alpha [B,H,dk]); beta (GDN / KDA [B,H]); z [B,H,dk] (KATH,
    updated in place). Returns o [B,H,dv].
    """
    import torch
    lib = load()
    B, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S", S),
                    ("z", z), ("o", o)):
        _require_contig(name, t)
    io = _dtype_code(q)
    gate_t = g if g is not None else beta
    gd = _dtype_code(gate_t) if gate_t is not None else LA_F32
    desc = make_desc(variant, B, H, 1, dk, dv, io, gd, eps)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    rc = lib.la_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(S), _ptr(z), _ptr(o), _stream_handle(stream, q.device))
    _check(rc, "la_decode_step")
    return o


class BackwardGrads(NamedTuple):
    dq: object
    dk: object
    dv: object
    dg: object
    dbeta: object   # GDN only, else None
    dS0: object
    dz0: object = None   # KATH only


def prefill_backward(q, k, v, g, dO, *, variant: str, beta=None, S0=None, z0=None,
                     dS_final=None, dz_final=None, dq=None, dk=None, dv=None, dg=None,
                     dbeta=None, dS0=None, dz0=None, eps: float = 1e-6, path: str = "auto",
                     workspace=None, stream=None) -> BackwardGrads:
    """Gradients of ``prefill`` through ``la_prefill_backward`` (KATH, GLA, SSD, GDN).

    q, k, v, g (None for KATH), beta (GDN), S0, z0 (KATH) as given to ``prefill``; dO
    [B,H,N,dv] (q's dtype); dS_final [B,H,dk,dv] and dz_final [B,H,dk] float32 or None.
    Returns BackwardGrads(dq, dk, dv, dg, dbeta, dS0, dz0).
    """
    import torch
    lib = load()
    B, H, N, dk_ = q.shape
    dv_ = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("dO", dO),
                    ("S0", S0), ("z0", z0), ("dS_final", dS_final), ("dz_final", dz_final),
                    ("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg), ("dbeta", dbeta),
                    ("dS0", dS0), ("dz0", dz0)):
        _require_contig(name, t)
    kath = variant == "kath"
    desc = make_desc(variant, B, H, N, dk_, dv_, _dtype_code(q),
                     _dtype_code(q if g is None else g), eps, path)
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if g is not None and dg is None:
        dg = torch.empty_like(g)
    if kath and dz0 is None:
        dz0 = torch.empty((B, H, dk_), dtype=torch.float32, device=dev)
    if beta is not None and dbeta is None:
        dbeta = torch.empty_like(beta)
    if dS0 is None:
        dS0 = torch.empty((B, H, dk_, dv_), dtype=torch.float32, device=dev)
    n = ctypes.c_size_t(0)
    _check(lib.la_prefill_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "la_prefill_backward_workspace_size")
    ws_bytes = int(n.value)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.la_prefill_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(S0), _ptr(z0), _ptr(dO), _ptr(dS_final),
                                 _ptr(dz_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                 _ptr(dbeta), _ptr(dS0), _ptr(dz0),
                                 _ptr(workspace if ws_bytes else None), wsz,
                                 _stream_handle(stream, dev))
    _check(rc, "la_prefill_backward")
    return BackwardGrads(dq, dk, dv, dg, dbeta, dS0, dz0)


def selective_scan(dt, A, Bm, Cm, x, Dskip=None, dt_bias=None, *, dt_softplus: bool = True,
                   h0=None, y=None, h_final=None, stream=None):
    """Mamba-1 selective scan through ``la_selective_scan``.

    dt, x [Bt,T,D] and Bm, Cm [Bt,T,n] (float32 or bfloat16, one dtype); A [D,n],
    Dskip [D], dt_bias [D] and h0 [Bt,D,n] float32 (the last three optional).
    h_final may be h0 (in place). Returns (y [Bt,T,D], h_final [Bt,D,n]).
    """
    import torch
    lib = load()
    Bt, T, D = x.shape
    n = A.shape[1]
    for name, t in (("dt", dt), ("A", A), ("Bm", Bm), ("Cm", Cm), ("x", x), ("Dskip", Dskip),
                    ("dt_bias", dt_bias), ("h0", h0), ("y", y), ("h_final", h_final)):
        _require_contig(name, t)
    desc = ScanDesc(Bt, T, D, n, _dtype_code(x), 1 if dt_softplus else 0)
    dev = x.device
    if y is None:
        y = torch.empty((Bt, T, D), dtype=x.dtype, device=dev)
    if h_final is None:
        h_final = torch.empty((Bt, D, n), dtype=torch.float32, device=dev)
    rc = lib.la_selective_scan(ctypes.byref(desc), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(x),
                               _ptr(Dskip), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final),
                               _stream_handle(stream, dev))
    _check(rc, "la_selective_scan")
    return y, h_final
