"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects
invalid calls before touching any buffer (no GPU needed: validation precedes all HIP calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_delta_rule_linear_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from gated_delta_rule_linear_amd import build
        build.build()
    return bd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(bd.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {bd.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_version_and_status(lib):
    hdr = open(HEADER).read()
    ver = int(re.search(r"#define LA_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.la_abi_version() == ver
    for code in range(5):
        assert bd.status_str(code)
    assert bd.status_str(99) == "unknown status"


# fake, suitably aligned, non-overlapping "device" addresses: validation never dereferences
BASE = 1 << 40
GAP = 1 << 34


def addr(i, off=0):
    return ctypes.c_void_p(BASE + i * GAP + off)


def call_prefill(lib, desc, q=None, k=None, v=None, g=None, beta=None, S0=None, z0=None,
                 o=None, S=None, z=None, ws=None, ws_bytes=0):
    return lib.la_prefill(ctypes.byref(desc) if desc is not None else None, q, k, v, g, beta,
                          S0, z0, o, S, z, ws, ws_bytes, None)


def good(variant="gla", **kw):
    base = dict(variant=variant, B=2, H=3, N=40, dk=64, dv=32, io_dtype=bd.LA_BF16,
                gate_dtype=bd.LA_BF16, eps=1e-6, path="valu")
    base.update(kw)
    return bd.make_desc(base.pop("variant"), base.pop("B"), base.pop("H"), base.pop("N"),
                        base.pop("dk"), base.pop("dv"), base.pop("io_dtype"),
                        base.pop("gate_dtype"), base.pop("eps"), base.pop("path"),
                        base.pop("chunk", 0), base.pop("segments", 0))


def ptrs(variant):
    p = dict(q=addr(0), k=addr(1), v=addr(2), o=addr(7), S=addr(8))
    if variant in ("gla", "gdn", "kda", "ssd"):
        p["g"] = addr(3)
    if variant in ("gdn", "kda"):
        p["beta"] = addr(4)
    if variant == "kath":
        p["z"] = addr(9)
    return p


@pytest.mark.parametrize("case,expect", [
    ("null_desc", bd.LA_ERR_INVALID),
    ("bad_variant", bd.LA_ERR_INVALID),
    ("bad_io_dtype", bd.LA_ERR_INVALID),
    ("negative_N", bd.LA_ERR_INVALID),
    ("nan_eps", bd.LA_ERR_INVALID),
    ("bad_path", bd.LA_ERR_INVALID),
    ("dk_48", bd.LA_ERR_UNSUPPORTED),
    ("dv_256", bd.LA_ERR_UNSUPPORTED),
    ("mfma_f32", bd.LA_ERR_UNSUPPORTED),
    ("chunk_mismatch", bd.LA_ERR_UNSUPPORTED),
    ("null_q", bd.LA_ERR_INVALID),
    ("null_S_final", bd.LA_ERR_INVALID),
    ("misaligned_v", bd.LA_ERR_INVALID),
    ("misaligned_gla_gate", bd.LA_ERR_INVALID),
    ("o_overlaps_q", bd.LA_ERR_INVALID),
    ("S_partial_overlap_S0", bd.LA_ERR_INVALID),
    ("S_overlaps_k", bd.LA_ERR_INVALID),
    ("gla_missing_gate", bd.LA_ERR_INVALID),
    ("gla_with_beta", bd.LA_ERR_INVALID),
    ("gdn_missing_beta", bd.LA_ERR_INVALID),
    ("kda_missing_beta", bd.LA_ERR_INVALID),
    ("kda_missing_gate", bd.LA_ERR_INVALID),
    ("misaligned_kda_gate", bd.LA_ERR_INVALID),
    ("ssd_missing_gate", bd.LA_ERR_INVALID),
    ("ssd_with_beta", bd.LA_ERR_INVALID),
    ("misaligned_ssd_gate", bd.LA_ERR_INVALID),
    ("kath_with_gate", bd.LA_ERR_INVALID),
    ("kath_missing_z", bd.LA_ERR_INVALID),
    ("gla_with_z", bd.LA_ERR_INVALID),
])
def test_prefill_rejects(lib, case, expect):
    variant = {"gdn_missing_beta": "gdn", "kath_with_gate": "kath", "kath_missing_z": "kath",
               "kda_missing_beta": "kda", "kda_missing_gate": "kda",
               "misaligned_kda_gate": "kda", "ssd_missing_gate": "ssd", "ssd_with_beta": "ssd",
               "misaligned_ssd_gate": "ssd"}.get(case, "gla")
    d = good(variant)
    p = ptrs(variant)
    if case == "null_desc":
        d = None
    elif case == "bad_variant":
        d.variant = 7
    elif case == "bad_io_dtype":
        d.io_dtype = 3
    elif case == "negative_N":
        d.N = -1
    elif case == "nan_eps":
        d = good("kath", eps=float("nan"))
        p = ptrs("kath")
    elif case == "bad_path":
        d.path = 9
    elif case == "dk_48":
        d.dk = 48
    elif case == "dv_256":
        d.dv = 256
    elif case == "mfma_f32":
        d = good("gdn", io_dtype=bd.LA_F32, path="mfma")
        p = ptrs("gdn")
    elif case == "chunk_mismatch":
        d.chunk = 48
    elif case == "null_q":
        p["q"] = None
    elif case == "null_S_final":
        p["S"] = None
    elif case == "misaligned_v":
        p["v"] = addr(2, 8)
    elif case == "misaligned_gla_gate":
        p["g"] = addr(3, 2)
    elif case == "o_overlaps_q":
        p["o"] = addr(0, 256)
    elif case == "S_partial_overlap_S0":
        p["S0"] = addr(8, 64)
    elif case == "S_overlaps_k":
        p["S"] = addr(1, 1024)
    elif case == "gla_missing_gate":
        p.pop("g")
    elif case == "gla_with_beta":
        p["beta"] = addr(4)
    elif case in ("gdn_missing_beta", "kda_missing_beta"):
        p.pop("beta")
    elif case in ("kda_missing_gate", "ssd_missing_gate"):
        p.pop("g")
    elif case == "ssd_with_beta":
        p["beta"] = addr(4)
    elif case == "misaligned_ssd_gate":
        p["g"] = addr(3, 1)
    elif case == "misaligned_kda_gate":
        p["g"] = addr(3, 2)
    elif case == "kath_with_gate":
        p["g"] = addr(3)
    elif case == "kath_missing_z":
        p.pop("z")
    elif case == "gla_with_z":
        p["z"] = addr(9)
    assert call_prefill(lib, d, **p) == expect


def test_invalid_call_touches_nothing(lib):
    """A rejected call must leave every output byte as it was (host buffers stand in)."""
    d = good("gdn", B=1, H=1, N=8, dk=16, dv=16)
    bufs = {n: np.full(4096, 7, np.uint8) for n in ("q", "k", "v", "g", "o", "S")}
    p = {n: ctypes.c_void_p(b.ctypes.data) for n, b in bufs.items()}
    # beta missing -> invalid before any access
    assert call_prefill(lib, d, **p) == bd.LA_ERR_INVALID
    for b in bufs.values():
        assert np.all(b == 7)


@pytest.mark.parametrize("case,expect", [
    ("N_not_1", bd.LA_ERR_INVALID),
    ("null_S", bd.LA_ERR_INVALID),
    ("o_overlaps_S", bd.LA_ERR_INVALID),
    ("kath_missing_z", bd.LA_ERR_INVALID),
    ("gdn_missing_alpha", bd.LA_ERR_INVALID),
    ("dk_24", bd.LA_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, case, expect):
    variant = {"kath_missing_z": "kath"}.get(case, "gdn")
    d = good(variant, N=1)
    p = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), S=addr(8), z=None,
             o=addr(7))
    if variant == "kath":
        p["g"] = p["beta"] = None
        p["z"] = addr(9)
    if case == "N_not_1":
        d.N = 2
    elif case == "null_S":
        p["S"] = None
    elif case == "o_overlaps_S":
        p["o"] = addr(8, 512)
    elif case == "kath_missing_z":
        p["z"] = None
    elif case == "gdn_missing_alpha":
        p["g"] = None
    elif case == "dk_24":
        d.dk = 24
    rc = lib.la_decode_step(ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], p["S"],
                            p["z"], p["o"], None)
    assert rc == expect


def test_gdn_scalar_gates_need_element_alignment_only(lib):
    """GDN alpha/beta are per-token scalars: a 2-byte offset (bf16) is accepted by the
    validation (the call then fails later only because no GPU / fake pointers)."""
    d = good("gdn", B=0)          # empty batch: validated fully, then a no-op
    p = ptrs("gdn")
    p["g"], p["beta"] = addr(3, 2), addr(4, 6)
    assert call_prefill(lib, d, **p) == bd.LA_OK
    p["g"] = addr(3, 1)           # not even element aligned
    assert call_prefill(lib, d, **p) == bd.LA_ERR_INVALID


def test_workspace_query(lib):
    assert bd.prefill_workspace_bytes(good("gla")) == 0      # VALU path needs none
    n = ctypes.c_size_t(123)
    assert lib.la_prefill_workspace_size(None, ctypes.byref(n)) == bd.LA_ERR_INVALID
    d = good("gla", dk=48)
    assert lib.la_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == \
        bd.LA_ERR_UNSUPPORTED


def test_empty_batch_is_noop(lib):
    d = good("gla", B=0)
    assert call_prefill(lib, d) == bd.LA_OK
    d = good("gdn", B=2, H=0, N=1)
    assert lib.la_decode_step(ctypes.byref(d), None, None, None, None, None, None, None, None,
                              None) == bd.LA_OK


@pytest.mark.parametrize("case", ["B_not_1", "max_over_N", "negative_nseq", "null_cu", "misaligned_cu",
                                  "S_overlaps_cu"])
def test_prefill_varlen_rejects(lib, case):
    d = good("gdn", B=1, N=40)
    p = ptrs("gdn")
    nseq, cu, maxlen = 3, addr(5), 20
    if case == "B_not_1":
        d.B = 2
    elif case == "max_over_N":
        maxlen = 41
    elif case == "negative_nseq":
        nseq = -1
    elif case == "null_cu":
        cu = None
    elif case == "misaligned_cu":
        cu = addr(5, 2)
    elif case == "S_overlaps_cu":
        cu = addr(8, 16)
    rc = lib.la_prefill_varlen(ctypes.byref(d), nseq, cu, maxlen, p["q"], p["k"], p["v"],
                               p.get("g"), p.get("beta"), None, None, p["o"], p["S"], None,
                               None, 0, None)
    assert rc == bd.LA_ERR_INVALID, (case, rc)


# ------------------------------------------------------------------ selective scan


def scan_args():
    return dict(dt=addr(0), A=addr(1), Bm=addr(2), Cm=addr(3), x=addr(4), Dskip=addr(5),
                dt_bias=addr(6), h0=addr(7), y=addr(8), h_final=addr(9))


def call_scan(lib, desc, **p):
    return lib.la_selective_scan(ctypes.byref(desc) if desc is not None else None, p["dt"],
                                 p["A"], p["Bm"], p["Cm"], p["x"], p["Dskip"], p["dt_bias"],
                                 p["h0"], p["y"], p["h_final"], None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", bd.LA_ERR_INVALID),
    ("bad_io", bd.LA_ERR_INVALID),
    ("bad_softplus_flag", bd.LA_ERR_INVALID),
    ("negative_T", bd.LA_ERR_INVALID),
    ("n_48", bd.LA_ERR_UNSUPPORTED),
    ("n_256", bd.LA_ERR_UNSUPPORTED),
    ("null_x", bd.LA_ERR_INVALID),
    ("null_A", bd.LA_ERR_INVALID),
    ("null_h_final", bd.LA_ERR_INVALID),
    ("misaligned_B", bd.LA_ERR_INVALID),
    ("misaligned_h0", bd.LA_ERR_INVALID),
    ("misaligned_dt_bf16", bd.LA_ERR_INVALID),
    ("y_overlaps_x", bd.LA_ERR_INVALID),
    ("h_partial_overlap_h0", bd.LA_ERR_INVALID),
    ("h_overlaps_A", bd.LA_ERR_INVALID),
    ("row_over_2GiB", bd.LA_ERR_UNSUPPORTED),
])
def test_selective_scan_rejects(lib, case, expect):
    d = bd.ScanDesc(2, 50, 40, 16, bd.LA_BF16, 1)
    p = scan_args()
    if case == "null_desc":
        d = None
    elif case == "bad_io":
        d.io_dtype = 5
    elif case == "bad_softplus_flag":
        d.dt_softplus = 2
    elif case == "negative_T":
        d.T = -1
    elif case == "n_48":
        d.n = 48
    elif case == "n_256":
        d.n = 256
    elif case == "null_x":
        p["x"] = None
    elif case == "null_A":
        p["A"] = None
    elif case == "null_h_final":
        p["h_final"] = None
    elif case == "misaligned_B":
        p["Bm"] = addr(2, 8)
    elif case == "misaligned_h0":
        p["h0"] = addr(7, 4)
    elif case == "misaligned_dt_bf16":
        p["dt"] = addr(0, 1)
    elif case == "y_overlaps_x":
        p["y"] = addr(4, 64)
    elif case == "h_partial_overlap_h0":
        p["h_final"] = addr(7, 16)
    elif case == "h_overlaps_A":
        p["h_final"] = addr(1, 16)
    elif case == "row_over_2GiB":
        d.T, d.D = 1 << 20, 1024   # 2 GiB of bf16 per batch row
    assert call_scan(lib, d, **p) == expect


def test_selective_scan_accepts_and_noops(lib):
    p = scan_args()
    # no rows or no channels: validated, then nothing to do
    assert call_scan(lib, bd.ScanDesc(0, 50, 40, 16, bd.LA_BF16, 1), **p) == bd.LA_OK
    assert call_scan(lib, bd.ScanDesc(2, 50, 0, 16, bd.LA_F32, 0), **p) == bd.LA_OK
    # optional inputs may be absent; h_final may be h0 exactly (in place)
    p2 = dict(p, Dskip=None, dt_bias=None, h0=None)
    assert call_scan(lib, bd.ScanDesc(0, 5, 8, 32, bd.LA_F32, 0), **p2) == bd.LA_OK
    p3 = dict(p, h_final=p["h0"])
    assert call_scan(lib, bd.ScanDesc(0, 5, 8, 32, bd.LA_F32, 0), **p3) == bd.LA_OK


# ------------------------------------------------------------------------------ backward


def bwd_args():
    return dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=None, S0=addr(5), z0=None,
                dO=addr(6), dSf=addr(7), dzf=None, dq=addr(10), dk=addr(11), dv=addr(12),
                dg=addr(13), dbeta=None, dS0=addr(14), dz0=None)


def call_bwd(lib, desc, ws=None, ws_bytes=0, **p):
    return lib.la_prefill_backward(ctypes.byref(desc) if desc is not None else None, p["q"],
                                   p["k"], p["v"], p["g"], p["beta"], p["S0"], p["z0"], p["dO"],
                                   p["dSf"], p["dzf"], p["dq"], p["dk"], p["dv"], p["dg"],
                                   p["dbeta"], p["dS0"], p["dz0"], ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", bd.LA_ERR_INVALID),
    ("kda_null_beta", bd.LA_ERR_INVALID),
    ("kath_g_given", bd.LA_ERR_INVALID),
    ("kath_null_dz0", bd.LA_ERR_INVALID),
    ("kath_dz0_overlaps_z0", bd.LA_ERR_INVALID),
    ("gla_z0_given", bd.LA_ERR_INVALID),
    ("gdn_null_beta", bd.LA_ERR_INVALID),
    ("gdn_null_dbeta", bd.LA_ERR_INVALID),
    ("gdn_dbeta_overlaps_beta", bd.LA_ERR_INVALID),
    ("gdn_dbeta_overlaps_dg", bd.LA_ERR_INVALID),
    ("gdn_z0_given", bd.LA_ERR_INVALID),
    ("mfma_path", bd.LA_ERR_UNSUPPORTED),
    ("beta_given", bd.LA_ERR_INVALID),
    ("null_dO", bd.LA_ERR_INVALID),
    ("null_dS0", bd.LA_ERR_INVALID),
    ("null_dg", bd.LA_ERR_INVALID),
    ("misaligned_dq", bd.LA_ERR_INVALID),
    ("dq_overlaps_dk", bd.LA_ERR_INVALID),
    ("dv_overlaps_dO", bd.LA_ERR_INVALID),
    ("dS0_overlaps_S0", bd.LA_ERR_INVALID),
    ("no_workspace", bd.LA_ERR_WORKSPACE),
])
def test_backward_rejects(lib, case, expect):
    variant = "gla"
    if case.startswith("gdn_"):
        variant = "gdn"
    if case.startswith("kda_"):
        variant = "kda"
    if case.startswith("kath_"):
        variant = "kath"
    d = good(variant)
    p = bwd_args()
    if variant in ("gdn", "kda"):
        p["beta"], p["dbeta"] = addr(4), addr(15)
    if variant == "kath":
        p["g"], p["dg"] = None, None
        p["z0"], p["dz0"] = addr(8), addr(16)
    ws, wsb = addr(20), 1 << 32
    if case == "null_desc":
        d = None
    elif case == "mfma_path":
        d = good("gla", path="mfma")
    elif case == "beta_given":
        p["beta"] = addr(4)
    elif case == "null_dO":
        p["dO"] = None
    elif case == "null_dS0":
        p["dS0"] = None
    elif case == "null_dg":
        p["dg"] = None
    elif case == "misaligned_dq":
        p["dq"] = addr(10, 4)
    elif case == "dq_overlaps_dk":
        p["dk"] = addr(10, 512)
    elif case == "dv_overlaps_dO":
        p["dv"] = addr(6, 256)
    elif case == "dS0_overlaps_S0":
        p["dS0"] = addr(5)
    elif case == "no_workspace":
        ws, wsb = None, 0
    elif case in ("gdn_null_beta", "kda_null_beta"):
        p["beta"] = None
    elif case == "gdn_null_dbeta":
        p["dbeta"] = None
    elif case == "gdn_dbeta_overlaps_beta":
        p["dbeta"] = addr(4, 64)
    elif case == "gdn_dbeta_overlaps_dg":
        p["dbeta"] = addr(13, 2)
    elif case == "gdn_z0_given":
        p["z0"] = addr(8)
    elif case == "kath_g_given":
        p["g"] = addr(3)
    elif case == "kath_null_dz0":
        p["dz0"] = None
    elif case == "kath_dz0_overlaps_z0":
        p["dz0"] = addr(8, 64)
    elif case == "gla_z0_given":
        p["z0"] = addr(8)
    assert call_bwd(lib, d, ws, wsb, **p) == expect, case


def test_backward_gdn_accepts_beta(lib):
    """The delta rule's backward takes beta and writes dbeta; with no sequences it enqueues
    nothing, so the call returns LA_OK without a device."""
    d = good("gdn", B=0)
    p = bwd_args()
    p["beta"], p["dbeta"] = addr(4), addr(15)
    assert call_bwd(lib, d, **p) == bd.LA_OK
    d = good("kath", B=0)
    p = bwd_args()
    p["g"], p["dg"], p["dz0"] = None, None, addr(16)
    assert call_bwd(lib, d, **p) == bd.LA_OK


def test_backward_workspace_query(lib):
    n = ctypes.c_size_t(0)
    d = good("ssd", dk=128, dv=64, N=100)
    assert lib.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == bd.LA_OK
    assert n.value > 0
    d = good("gdn")
    assert lib.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == bd.LA_OK
    assert n.value > 0
    d = good("kda")
    assert lib.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == bd.LA_OK
    assert n.value > 0
    d = good("gla", B=0)
    assert call_bwd(lib, d, **bwd_args()) == bd.LA_OK   # no sequences: nothing to do


def test_stream_rmw_rejects(lib):
    """la_stream_rmw validates before any HIP call: n = 0 is a no-op even with NULL; a NULL
    buffer, n not a multiple of 4, or a misaligned buffer is LA_ERR_INVALID."""
    buf = (ctypes.c_float * 16)()
    base = ctypes.addressof(buf)
    assert lib.la_stream_rmw(None, 0, ctypes.c_float(2.0), None) == bd.LA_OK
    assert lib.la_stream_rmw(None, 4, ctypes.c_float(2.0), None) == bd.LA_ERR_INVALID
    aligned = base + (-base) % 16
    assert lib.la_stream_rmw(ctypes.c_void_p(aligned), 6, ctypes.c_float(2.0), None) == bd.LA_ERR_INVALID
    assert lib.la_stream_rmw(ctypes.c_void_p(aligned + 4), 4, ctypes.c_float(2.0), None) == bd.LA_ERR_INVALID
