"""Parity of the selective-scan kernel (Mamba-1) against the fp64 oracle (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import TOL, banner, dev, f64, relerr

pytestmark = pytest.mark.gpu


def case(Bt, T, D, n, io, seed, with_state=True):
    wl = W.SelScan("t", Bt, T, D, n, io, seed)
    return W.make_selscan_inputs(wl, with_state=with_state)


def run_gpu(d, softplus=True, use_skip=True, use_bias=True, h0=None, h_final=None):
    g = {k: dev(v) for k, v in d.items()}
    y, hT = bd.selective_scan(g["dt"], g["A"], g["Bm"], g["Cm"], g["x"],
                              g["Dskip"] if use_skip else None,
                              g["dt_bias"] if use_bias else None, dt_softplus=softplus,
                              h0=g.get("h0") if h0 is None else h0, h_final=h_final)
    torch.cuda.synchronize()
    return y, hT


def run_oracle(e, softplus=True, use_skip=True, use_bias=True, chans=None):
    sel = (lambda a: a) if chans is None else (lambda a: a[..., chans])
    h0 = e.get("h0")
    return oracle.selective_scan(sel(e["dt"]), e["A"] if chans is None else e["A"][chans],
                                 e["Bm"], e["Cm"], sel(e["x"]),
                                 (sel(e["Dskip"]) if use_skip else None),
                                 (sel(e["dt_bias"]) if use_bias else None), softplus,
                                 None if h0 is None else (h0 if chans is None else h0[:, chans]))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n", [16, 32, 64, 128])
@pytest.mark.parametrize("T,D", [(1, 16), (33, 40), (100, 96)])
def test_scan_shapes(io, n, T, D):
    """Tokens across chunk boundaries (32 per chunk) with a ragged tail, channel counts that
    leave a partial block of 16, every supported state size."""
    d, e = case(2, T, D, n, io, seed=T * 7 + D + n)
    banner(f"selscan {io} Bt=2 T={T} D={D} n={n}")
    y, hT = run_gpu(d)
    y_ref, h_ref = run_oracle(e)
    assert relerr(y, y_ref) <= TOL[io], relerr(y, y_ref)
    assert relerr(hT, h_ref) <= TOL["f32"], relerr(hT, h_ref)


@pytest.mark.parametrize("softplus,skip,bias", [(False, True, True), (True, False, False),
                                                (False, False, True)])
def test_scan_options(softplus, skip, bias):
    d, e = case(1, 70, 48, 64, "f32", seed=5)
    if not softplus:   # a raw step must stay positive for a decay
        for k_ in ("dt", "dt_bias"):
            d[k_] = np.abs(d[k_]).astype(np.float32)
            e[k_] = d[k_].astype(np.float64)
    banner(f"selscan options softplus={softplus} skip={skip} bias={bias}")
    y, hT = run_gpu(d, softplus, skip, bias)
    y_ref, h_ref = run_oracle(e, softplus, skip, bias)
    assert relerr(y, y_ref) <= TOL["f32"] and relerr(hT, h_ref) <= TOL["f32"]


def test_scan_no_initial_state():
    d, e = case(2, 45, 32, 32, "bf16", seed=8, with_state=False)
    banner("selscan without h0")
    y, hT = run_gpu(d)
    y_ref, h_ref = run_oracle(e)
    assert relerr(y, y_ref) <= TOL["bf16"] and relerr(hT, h_ref) <= TOL["f32"]


def test_scan_empty_sequence_copies_state():
    d, e = case(2, 0, 24, 16, "f32", seed=9)
    banner("selscan T=0")
    y, hT = run_gpu(d)
    assert torch.equal(hT.cpu(), torch.from_numpy(d["h0"]))


def test_scan_split_and_decode_steps_are_exact():
    """The state carried between calls continues the scan exactly: two calls split at a
    chunk-internal token, and single-token in-place calls (the decode form), give the same
    bits as one call over the whole sequence (per-token arithmetic does not depend on the
    chunking)."""
    d, e = case(2, 80, 40, 128, "bf16", seed=10)
    banner("selscan split / decode steps")
    g = {k: dev(v) for k, v in d.items()}
    y, hT = bd.selective_scan(g["dt"], g["A"], g["Bm"], g["Cm"], g["x"], g["Dskip"], g["dt_bias"],
                              h0=g["h0"])
    sl = lambda t, a, b: t[:, a:b].contiguous()
    cut = 45
    yL, hm = bd.selective_scan(sl(g["dt"], 0, cut), g["A"], sl(g["Bm"], 0, cut), sl(g["Cm"], 0, cut),
                               sl(g["x"], 0, cut), g["Dskip"], g["dt_bias"], h0=g["h0"])
    yR, hR = bd.selective_scan(sl(g["dt"], cut, 80), g["A"], sl(g["Bm"], cut, 80),
                               sl(g["Cm"], cut, 80), sl(g["x"], cut, 80), g["Dskip"], g["dt_bias"],
                               h0=hm)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([yL, yR], 1), y) and torch.equal(hR, hT)
    h = g["h0"].clone()
    ys = []
    for t in range(80):
        yt, h2 = bd.selective_scan(sl(g["dt"], t, t + 1), g["A"], sl(g["Bm"], t, t + 1),
                                   sl(g["Cm"], t, t + 1), sl(g["x"], t, t + 1), g["Dskip"],
                                   g["dt_bias"], h0=h, h_final=h)
        assert h2.data_ptr() == h.data_ptr()
        ys.append(yt)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, 1), y) and torch.equal(h, hT)
    y_ref, h_ref = run_oracle(e)
    assert relerr(y, y_ref) <= TOL["bf16"] and relerr(hT, h_ref) <= TOL["f32"]


@pytest.mark.parametrize("name", list(W.SELSCAN))
def test_scan_full_workload_sampled(name):
    """Full-size run as the benchmark launches it; the oracle checks sampled channels
    (first, last, and some in between, in every batch row) element by element."""
    wl = W.SELSCAN[name]
    d, e = W.make_selscan_inputs(wl)
    banner(f"selscan full workload {name}")
    y, hT = run_gpu(d)
    chans = [0, 1, 15, 16, wl.D // 2 + 3, wl.D - 17, wl.D - 1]
    y_ref, h_ref = run_oracle(e, chans=chans)
    errs = (relerr(y[:, :, chans], y_ref), relerr(hT[:, chans], h_ref))
    print(name, errs, flush=True)
    assert errs[0] <= TOL["bf16"] and errs[1] <= TOL["f32"], errs
    assert torch.isfinite(y.float()).all()
