"""Parity of the decode kernel and the fp32 VALU prefill against the fp64 oracle (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import TOL, banner, dev, f64, inputs_to_device, relerr

pytestmark = pytest.mark.gpu


def run_prefill_case(wl, path="valu", with_state=True, seed=None, check=True):
    inp = W.make_inputs(wl, with_state=with_state, seed=seed)
    d = inputs_to_device(inp)
    banner(f"prefill {wl.variant} {wl.io} B{wl.B} H{wl.H} N{wl.N} dk{wl.dk} dv{wl.dv} "
           f"path={path} gates={wl.gate_kind}")
    o, S, z = bd.prefill(d["q"], d["k"], d["v"], d.get("g"), d.get("beta"), variant=wl.variant,
                         S0=d.get("S0"), z0=d.get("z0"), eps=wl.eps, path=path)
    torch.cuda.synchronize()
    e = inp.exact
    o_ref, S_ref, z_ref = oracle.prefill(wl.variant, e["q"], e["k"], e["v"], e.get("g"),
                                         e.get("beta"), e.get("S0"), e.get("z0"), eps=wl.eps)
    tol = TOL[wl.io]
    errs = {"o": relerr(o, o_ref), "S": relerr(S, S_ref)}
    if wl.variant == "kath":
        errs["z"] = relerr(z, z_ref)
    if check:
        for name, err in errs.items():
            assert err <= tol, f"{name}: {err:.3e} > {tol}"
    return errs


def test_config_kath_f32_n256_d16():
    """The small fp32 normalized-attention workload, full size, tolerance 1e-5."""
    wl = W.WORKLOADS["kath_f32_n256_d16"]
    errs = run_prefill_case(wl, path="auto", with_state=False)
    print(errs)


SHAPES = [(16, 16), (32, 64), (64, 32), (128, 128), (128, 64)]


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", SHAPES)
def test_valu_prefill_shapes(variant, io, dk, dv):
    wl = W.Workload("t", variant, 2, 2, 37, dk, dv, io, io, seed=dk * 7 + dv,
                    qk_scale=(1.0 if variant == "kath" else dk ** -0.5),
                    l2norm_qk=(variant in ("gdn", "kda")))
    run_prefill_case(wl)


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 64, 129])
def test_valu_prefill_lengths(variant, N):
    wl = W.Workload("t", variant, 1, 3, N, 32, 16, "f32", "f32", seed=N,
                    l2norm_qk=(variant in ("gdn", "kda")),
                    gate_kind="slow" if variant != "kath" else "default")
    run_prefill_case(wl)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
@pytest.mark.parametrize("kind", ["default", "ones", "beta0", "beta1", "slow"])
def test_valu_delta_gate_kinds(variant, kind):
    wl = W.Workload("t", variant, 1, 2, 80, 64, 32, "f32", "f32", seed=3, l2norm_qk=True,
                    gate_kind=kind)
    run_prefill_case(wl)


def test_empty_sequence_copies_state():
    banner("prefill N=0")
    B, H, dk, dv = 2, 3, 32, 16
    S0 = torch.randn(B, H, dk, dv, device="cuda")
    z0 = torch.rand(B, H, dk, device="cuda")
    q = torch.empty(B, H, 0, dk, device="cuda")
    v = torch.empty(B, H, 0, dv, device="cuda")
    o, S, z = bd.prefill(q, q, v, variant="kath", S0=S0, z0=z0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0)
    o, S, _ = bd.prefill(q, q, v, torch.empty(B, H, 0, dk, device="cuda"), variant="gla")
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_in_place_state_carry():
    """S_final may be S0: the carried state is updated in place."""
    wl = W.Workload("t", "gdn", 1, 2, 50, 64, 64, "f32", "f32", seed=9, l2norm_qk=True)
    inp = W.make_inputs(wl, with_state=True)
    d = inputs_to_device(inp)
    banner("prefill in-place S0 == S_final")
    S = d["S0"].clone()
    o, S_out, _ = bd.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], variant="gdn", S0=S,
                             S_final=S, path="valu")
    torch.cuda.synchronize()
    e = inp.exact
    o_ref, S_ref, _ = oracle.prefill("gdn", e["q"], e["k"], e["v"], e["g"], e["beta"], e["S0"])
    assert S_out.data_ptr() == S.data_ptr()
    assert relerr(S, S_ref) < 1e-5 and relerr(o, o_ref) < 1e-5


def test_valu_split_carry_matches_whole():
    """Prefill [0, m) then [m, N) with the carried state equals the whole run."""
    wl = W.Workload("t", "gla", 1, 2, 90, 64, 32, "f32", "f32", seed=4, gate_kind="slow")
    inp = W.make_inputs(wl, with_state=False)
    d = inputs_to_device(inp)
    banner("prefill split/carry")
    o, S, _ = bd.prefill(d["q"], d["k"], d["v"], d["g"], variant="gla", path="valu")
    for m in (16, 37):
        sl = lambda t, a, b: t[:, :, a:b].contiguous()
        oL, SL, _ = bd.prefill(sl(d["q"], 0, m), sl(d["k"], 0, m), sl(d["v"], 0, m),
                               sl(d["g"], 0, m), variant="gla", path="valu")
        oR, SR, _ = bd.prefill(sl(d["q"], m, 90), sl(d["k"], m, 90), sl(d["v"], m, 90),
                               sl(d["g"], m, 90), variant="gla", S0=SL, path="valu")
        torch.cuda.synchronize()
        assert relerr(torch.cat([oL, oR], 2), f64(o)) < 1e-6
        assert relerr(SR, f64(S)) < 1e-6
        if m % 16 == 0:   # split at a chunk boundary: identical arithmetic
            assert torch.equal(torch.cat([oL, oR], 2), o) and torch.equal(SR, S)


# ------------------------------------------------------------------------- decode

def decode_case(variant, io, B, H, dk, dv, seed=0, steps=1, gate_kind="default"):
    wl = W.Workload("dec", variant, B, H, 1, dk, dv, io, io, seed=seed, decode=True,
                    qk_scale=(1.0 if variant == "kath" else dk ** -0.5),
                    l2norm_qk=(variant in ("gdn", "kda")), gate_kind=gate_kind)
    rng = np.random.default_rng(seed + 100)
    S64 = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32).astype(np.float64)
    z64 = (np.abs(rng.standard_normal((B, H, dk))) + 1.0).astype(np.float32).astype(np.float64)
    S = torch.from_numpy(S64.astype(np.float32)).cuda()
    z = torch.from_numpy(z64.astype(np.float32)).cuda() if variant == "kath" else None
    S_ref = S64.copy()
    z_ref = z64.copy() if variant == "kath" else None
    banner(f"decode {variant} {io} B{B} H{H} dk{dk} dv{dv} steps={steps}")
    errs = []
    for s in range(steps):
        inp = W.make_inputs(wl, seed=seed * 1000 + s)
        sq = {k: (a.reshape(a.shape[:2] + a.shape[3:]) if a.ndim >= 3 else a)
              for k, a in inp.dev.items()}
        ex = {k: (a.reshape(a.shape[:2] + a.shape[3:]) if a.ndim >= 3 else a)
              for k, a in inp.exact.items()}
        d = {k: dev(a) for k, a in sq.items()}
        o = bd.decode_step(d["q"], d["k"], d["v"], S, d.get("g"), d.get("beta"), variant=variant,
                           z=z, eps=wl.eps)
        o_ref = oracle.decode_step(variant, ex["q"], ex["k"], ex["v"], S_ref, g=ex.get("g"),
                                   beta=ex.get("beta"), z=z_ref, eps=wl.eps)
        torch.cuda.synchronize()
        errs.append((relerr(o, o_ref), relerr(S, S_ref)))
    return errs


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (64, 64), (128, 128)])
def test_decode_shapes(variant, io, dk, dv):
    errs = decode_case(variant, io, 3, 5, dk, dv, seed=dk + dv, steps=3)
    for eo, eS in errs:
        assert eo <= TOL[io] and eS <= 1e-5, errs


@pytest.mark.parametrize("variant", ["gdn", "gla", "kda", "ssd"])
def test_decode_many_steps(variant):
    errs = decode_case(variant, "bf16", 4, 8, 128, 128, seed=5, steps=40, gate_kind="default")
    eo, eS = errs[-1]
    assert max(e[0] for e in errs) <= 2e-2 and max(e[1] for e in errs) <= 1e-5, errs[-1]
