"""Parity of the prefill backward (KATH, GLA, SSD, GDN, KDA) against the fp64 oracle's
reverse-mode gradients (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import TOL, banner, dev, relerr

pytestmark = pytest.mark.gpu


def make_case(variant, B, H, N, dk, dv, io, seed, gate_kind="default", with_state=True,
              with_dsf=True, gate_io=None):
    kw = dict(seed=seed, qk_scale=dk ** -0.5, gate_kind=gate_kind)
    if variant == "gla":
        kw["v_scale"] = dk ** -0.5
    if variant in ("gdn", "kda"):
        kw["l2norm_qk"] = True
    wl = W.Workload("b", variant, B, H, N, dk, dv, io, gate_io or io, **kw)
    inp = W.make_inputs(wl, with_state=with_state)
    rng = np.random.default_rng(seed + 77)
    dO, dO_x = W.round_to(rng.standard_normal((B, H, N, dv)), io)
    dSf = dSf_x = None
    if with_dsf:
        dSf, dSf_x = W.round_to(rng.standard_normal((B, H, dk, dv)) * 0.1, "f32")
        if variant == "kath":   # the normaliser's final gradient rides along with dS_final
            dzf, dzf_x = W.round_to(rng.standard_normal((B, H, dk)) * 0.01, "f32")
            dSf, dSf_x = (dSf, dzf), (dSf_x, dzf_x)
    return inp, dO, dO_x, dSf, dSf_x


def run_both(variant, inp, dO, dO_x, dSf, dSf_x, seqs=None, threads=0, eps=1e-6):
    d = {k: dev(v) for k, v in inp.dev.items()}
    dSf, dzf = dSf if isinstance(dSf, tuple) else (dSf, None)
    dSf_x, dzf_x = dSf_x if isinstance(dSf_x, tuple) else (dSf_x, None)
    gr = bd.prefill_backward(d["q"], d["k"], d["v"], d.get("g"), dev(dO), variant=variant,
                             beta=d.get("beta"), S0=d.get("S0"), z0=d.get("z0"),
                             dS_final=dev(dSf), dz_final=dev(dzf), eps=eps)
    torch.cuda.synchronize()
    e = inp.exact
    sel = (lambda a: a) if seqs is None else \
        (lambda a: None if a is None else a.reshape((-1,) + a.shape[2:])[seqs][None])
    ref = oracle.prefill_backward(variant, sel(e["q"]), sel(e["k"]), sel(e["v"]),
                                  sel(e.get("g")), sel(e.get("beta")), sel(e.get("S0")),
                                  sel(e.get("z0")), sel(dO_x), sel(dSf_x), sel(dzf_x), eps=eps,
                                  threads=threads)
    got = {"dq": gr.dq, "dk": gr.dk, "dv": gr.dv, "dS0": gr.dS0}
    if gr.dg is not None:
        got["dg"] = gr.dg
    if gr.dbeta is not None:
        got["dbeta"] = gr.dbeta
    if gr.dz0 is not None:
        got["dz0"] = gr.dz0
    if seqs is not None:
        got = {k: v.reshape((-1,) + tuple(v.shape[2:]))[seqs][None] for k, v in got.items()}
    return got, ref


def check(got, ref, tol):
    errs = {k: relerr(got[k], ref[k]) for k in got}
    for k, v in errs.items():
        assert v <= tol, f"{k}: {v:.3e} > {tol} ({errs})"
    return errs


@pytest.mark.parametrize("variant", ["kath", "gla", "ssd", "gdn", "kda"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (128, 64)])
def test_backward_shapes(variant, io, dk, dv):
    case = make_case(variant, 2, 2, 37, dk, dv, io, seed=dk + 3 * dv)
    banner(f"backward {variant} {io} dk={dk} dv={dv} N=37")
    check(*run_both(variant, *case), TOL[io])


@pytest.mark.parametrize("variant", ["kath", "gla", "ssd", "gdn", "kda"])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 70])
def test_backward_lengths(variant, N):
    case = make_case(variant, 1, 3, N, 32, 16, "f32", seed=N, gate_kind="slow")
    banner(f"backward {variant} N={N}")
    check(*run_both(variant, *case), TOL["f32"])


@pytest.mark.parametrize("variant,kind", [("gla", "fast"), ("gla", "ones"), ("ssd", "fast"),
                                          ("ssd", "ones"), ("gdn", "default"), ("gdn", "ones"),
                                          ("gdn", "beta0"), ("gdn", "beta1"),
                                          ("kda", "default"), ("kda", "ones"), ("kda", "beta0"),
                                          ("kda", "beta1")])
def test_backward_gate_kinds(variant, kind):
    case = make_case(variant, 1, 2, 50, 64, 32, "f32", seed=9, gate_kind=kind)
    banner(f"backward {variant} gates={kind}")
    check(*run_both(variant, *case), TOL["f32"])


@pytest.mark.parametrize("variant", ["gla", "ssd", "gdn", "kda"])
@pytest.mark.parametrize("io,gate_io", [("f32", "bf16"), ("bf16", "f32")])
def test_backward_mixed_dtypes(variant, io, gate_io):
    """q, k, v, dO in one dtype and the gates (and beta) in the other; every gradient keeps
    its input's dtype."""
    case = make_case(variant, 1, 2, 45, 32, 32, io, seed=31, gate_io=gate_io)
    banner(f"backward {variant} io={io} gates={gate_io}")
    got, ref = run_both(variant, *case)
    assert got["dq"].dtype == (torch.float32 if io == "f32" else torch.bfloat16)
    assert got["dg"].dtype == (torch.float32 if gate_io == "f32" else torch.bfloat16)
    check(got, ref, TOL["bf16"] if "bf16" in (io, gate_io) else TOL["f32"])


def test_backward_without_state_or_final_gradient():
    case = make_case("gla", 1, 2, 40, 64, 32, "bf16", seed=12, with_state=False, with_dsf=False)
    banner("backward gla no S0, no dS_final")
    check(*run_both("gla", *case), TOL["bf16"])


@pytest.mark.parametrize("variant", ["ssd", "gdn", "kda", "kath"])
def test_backward_empty_sequence(variant):
    """N = 0: the initial state's gradient is the final state's."""
    inp, dO, dO_x, dSf, dSf_x = make_case(variant, 2, 3, 0, 32, 16, "f32", seed=3)
    banner(f"backward {variant} N=0")
    got, ref = run_both(variant, inp, dO, dO_x, dSf, dSf_x)
    if variant == "kath":
        assert torch.equal(got["dz0"].cpu(), torch.from_numpy(dSf[1]))
        dSf = dSf[0]
    assert torch.equal(got["dS0"].cpu(), torch.from_numpy(dSf))


@pytest.mark.parametrize("name", ["gla_bf16_b2h8_n2048_d128", "ssd_bf16_b2h32_n4096_dk128_dv64",
                                  "gdn_bf16_b4h16_n8192_d128", "kda_bf16_b4h16_n8192_d128",
                                  "kath_bf16_b1h16_n32768_dk128_dv64"])
@pytest.mark.timeout(300)
def test_backward_full_workload(name):
    """The full-size workload; the oracle's reverse mode runs every sequence (it keeps every
    token state, about 1-2 GB per sequence in flight on each host thread) and every gradient
    is compared on all of them."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(wl.seed + 500)
    dO, dO_x = W.round_to(rng.standard_normal((wl.B, wl.H, wl.N, wl.dv)), wl.io)
    banner(f"backward full workload {name}")
    got, ref = run_both(wl.variant, inp, dO, dO_x, None, None, eps=wl.eps)
    errs = check(got, ref, TOL["bf16"])
    print(name, errs, flush=True)


@pytest.mark.parametrize("variant", ["gla", "gdn", "kda"])
def test_backward_tiny_gates(variant):
    """Gates down to 1e-7 (5% of them): the gate gradient is taken directly from the states,
    so tiny gates cost no accuracy (fp32 bound)."""
    inp, dO, dO_x, dSf, dSf_x = make_case(variant, 1, 2, 60, 64, 32, "f32", seed=21)
    rng = np.random.default_rng(22)
    g = np.where(rng.random(inp.exact["g"].shape) < 0.05, 1e-7, inp.exact["g"])
    inp.dev["g"], inp.exact["g"] = W.round_to(g, "f32")
    banner(f"backward {variant} tiny gates")
    check(*run_both(variant, inp, dO, dO_x, dSf, dSf_x), TOL["f32"])


@pytest.mark.parametrize("N", [64, 200, 257])
def test_backward_ssd_matrix_cores_vs_valu(N):
    """The matrix-core SSD backward (bf16, d_k = 128, d_v = 64, chunk 64) against the oracle
    and against the fp32 VALU backward on the same inputs."""
    inp, dO, dO_x, dSf, dSf_x = make_case("ssd", 2, 3, N, 128, 64, "bf16", seed=N)
    banner(f"backward ssd matrix cores N={N}")
    got, ref = run_both("ssd", inp, dO, dO_x, dSf, dSf_x)
    check(got, ref, TOL["bf16"])
    d = {k: dev(v) for k, v in inp.dev.items()}
    valu = bd.prefill_backward(d["q"], d["k"], d["v"], d["g"], dev(dO), variant="ssd",
                               S0=d.get("S0"), dS_final=dev(dSf), path="valu")
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dS0"):
        assert relerr(got[name], getattr(valu, name).double().cpu().numpy()) <= TOL["bf16"], name


@pytest.mark.parametrize("dv,N,with_state", [(128, 64, True), (128, 200, True), (128, 257, False),
                                            (64, 130, True), (64, 1, True)])
def test_backward_gdn_matrix_cores_vs_valu(dv, N, with_state):
    """The matrix-core GDN backward (bf16, d_k = 128, chunk 64) against the oracle and
    against the fp32 VALU backward on the same inputs: several chunks, ragged tails, one
    token, with and without an initial state."""
    inp, dO, dO_x, dSf, dSf_x = make_case("gdn", 2, 3, N, 128, dv, "bf16", seed=N + dv,
                                          with_state=with_state)
    banner(f"backward gdn matrix cores dv={dv} N={N} S0={with_state}")
    got, ref = run_both("gdn", inp, dO, dO_x, dSf, dSf_x)
    check(got, ref, TOL["bf16"])
    d = {k: dev(v) for k, v in inp.dev.items()}
    valu = bd.prefill_backward(d["q"], d["k"], d["v"], d["g"], dev(dO), variant="gdn",
                               beta=d["beta"], S0=d.get("S0"), dS_final=dev(dSf), path="valu")
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        assert relerr(got[name], getattr(valu, name).double().cpu().numpy()) <= TOL["bf16"], name


@pytest.mark.parametrize("variant,dk,dv,N,path", [
    ("kath", 64, 32, 53, "auto"), ("gla", 64, 32, 53, "auto"), ("ssd", 64, 32, 53, "auto"),
    ("gdn", 64, 32, 53, "auto"), ("kda", 64, 32, 53, "auto"),
    # the matrix-core backwards (bf16, d_k = 128): several chunks and a tail
    ("ssd", 128, 64, 200, "mfma"), ("gdn", 128, 128, 200, "mfma")])
def test_backward_deterministic_and_batch_invariant(variant, dk, dv, N, path):
    """No atomics anywhere: two calls give the same bits, and a sequence's gradients do
    not depend on the other sequences of the batch (the same bits when it runs alone)."""
    inp, dO, dO_x, dSf, dSf_x = make_case(variant, 3, 2, N, dk, dv, "bf16", seed=41)
    banner(f"backward {variant} dk{dk} dv{dv} N{N} path={path} determinism / batch invariance")
    d = {k: dev(v) for k, v in inp.dev.items()}
    dSf0, dzf = dSf if isinstance(dSf, tuple) else (dSf, None)

    def call(sl):
        pick = lambda t: None if t is None else t[sl].contiguous()
        return bd.prefill_backward(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d.get("g")),
                                   pick(dev(dO)), variant=variant, beta=pick(d.get("beta")),
                                   S0=pick(d.get("S0")), z0=pick(d.get("z0")),
                                   dS_final=pick(dev(dSf0)), dz_final=pick(dev(dzf)), path=path)

    full = slice(0, 3)
    a, b = call(full), call(full)
    alone = call(slice(1, 2))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0", "dz0"):
        x, y, z = getattr(a, name), getattr(b, name), getattr(alone, name)
        if x is None:
            continue
        assert torch.equal(x, y), f"{name} differs between two calls"
        assert torch.equal(x[1:2], z), f"{name} of batch row 1 depends on the other rows"
