"""Parity of the bf16 matrix-core prefill kernels against the fp64 oracle, plus the
invariants the chunked method must keep (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import TOL, banner, f64, inputs_to_device, relerr

pytestmark = pytest.mark.gpu


def wl_for(variant, B, H, N, dv, seed, gate_kind="default", dk=128):
    if variant == "gla":
        return W.Workload("t", "gla", B, H, N, dk, dv, "bf16", "bf16", seed=seed,
                          qk_scale=dk ** -0.5, v_scale=dk ** -0.5, gate_kind=gate_kind)
    if variant in ("gdn", "kda"):
        return W.Workload("t", variant, B, H, N, dk, dv, "bf16", "bf16", seed=seed,
                          l2norm_qk=True, gate_kind=gate_kind)
    if variant == "ssd":
        return W.Workload("t", "ssd", B, H, N, dk, dv, "bf16", "bf16", seed=seed,
                          qk_scale=dk ** -0.5, gate_kind=gate_kind)
    return W.Workload("t", "kath", B, H, N, dk, dv, "bf16", "bf16", seed=seed)


def run_gpu(inp, d=None, path="mfma", segments=0, **kw):
    wl = inp.wl
    d = d or inputs_to_device(inp)
    o, S, z = bd.prefill(d["q"], d["k"], d["v"], d.get("g"), d.get("beta"), variant=wl.variant,
                         S0=d.get("S0"), z0=d.get("z0"), eps=wl.eps, path=path,
                         segments=segments, **kw)
    torch.cuda.synchronize()
    return o, S, z


def run_oracle(inp, seqs=None):
    """Oracle on all sequences, or on the flat sequence indices ``seqs``."""
    wl, e = inp.wl, inp.exact
    sel = lambda a: a if (a is None or seqs is None) else a.reshape((-1,) + a.shape[2:])[seqs][None]
    return oracle.prefill(wl.variant, sel(e["q"]), sel(e["k"]), sel(e["v"]), sel(e.get("g")),
                          sel(e.get("beta")), sel(e.get("S0")), sel(e.get("z0")), eps=wl.eps)


def check(inp, got, ref, tol=TOL["bf16"], seqs=None):
    o, S, z = got
    o_ref, S_ref, z_ref = ref
    if seqs is not None:
        flat = lambda t: t.reshape((-1,) + tuple(t.shape[2:]))[seqs][None]
        o, S = flat(o), flat(S)
        z = flat(z) if z is not None else None
    errs = {"o": relerr(o, o_ref), "S": relerr(S, S_ref)}
    if z_ref is not None:
        errs["z"] = relerr(z, z_ref)
    for k_, v_ in errs.items():
        assert v_ <= tol, f"{k_}: {v_:.3e} > {tol} ({errs})"
    return errs


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_mfma_shapes(variant, dv):
    inp = W.make_inputs(wl_for(variant, 2, 3, 200, dv, seed=dv + 1), with_state=True)
    banner(f"mfma {variant} dv={dv} N=200 with S0")
    errs = check(inp, run_gpu(inp), run_oracle(inp))
    print(errs)


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 130, 447])
def test_mfma_lengths(variant, N):
    inp = W.make_inputs(wl_for(variant, 1, 2, N, 64, seed=N), with_state=(N % 2 == 1))
    banner(f"mfma {variant} N={N}")
    check(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("variant", ["kath", "gla"])
@pytest.mark.parametrize("segments", [1, 2, 3, 5, 9])
def test_mfma_segments(variant, segments):
    inp = W.make_inputs(wl_for(variant, 1, 2, 64 * 9 + 5, 32, seed=segments), with_state=True)
    banner(f"mfma {variant} segments={segments}")
    check(inp, run_gpu(inp, segments=segments), run_oracle(inp))


@pytest.mark.parametrize("variant,kind", [("gla", "fast"), ("gla", "ones"), ("gla", "slow"),
                                          ("gdn", "slow"), ("gdn", "ones"), ("gdn", "beta0"),
                                          ("gdn", "beta1"), ("kda", "slow"), ("kda", "ones"),
                                          ("kda", "beta0"), ("kda", "beta1"), ("ssd", "slow"),
                                          ("ssd", "ones"), ("ssd", "fast")])
def test_mfma_gate_kinds(variant, kind):
    inp = W.make_inputs(wl_for(variant, 1, 2, 300, 64, seed=7, gate_kind=kind), with_state=True)
    banner(f"mfma {variant} gates={kind}")
    check(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("variant", ["gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("N", [70, 449])
def test_mfma_fp32_gates(variant, N):
    """bf16 q, k, v with fp32 gates (the other gate storage the ABI accepts)."""
    wl = wl_for(variant, 1, 2, N, 64, seed=N + 1).with_(gate_io="f32")
    inp = W.make_inputs(wl, with_state=True)
    assert inp.dev["g"].dtype == np.float32
    banner(f"mfma {variant} fp32 gates N={N}")
    check(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("segments", [3, 7])
def test_mfma_wide_tiles_segments(variant, segments):
    """d_v = 128 (the widest value tiles) with an explicit segment count and a ragged
    last chunk; GDN ignores the segment count."""
    inp = W.make_inputs(wl_for(variant, 1, 3, 64 * 13 + 9, 128, seed=40 + segments),
                        with_state=True)
    banner(f"mfma {variant} dv=128 segments={segments}")
    check(inp, run_gpu(inp, segments=segments), run_oracle(inp))


def test_gla_tiny_gates_clamped():
    """Gates far below exp(-10) (the matrix-core clamp) still match the oracle."""
    wl = wl_for("gla", 1, 2, 200, 32, seed=3)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(0)
    g = np.where(rng.random(inp.exact["g"].shape) < 0.05, 1e-7, inp.exact["g"])
    inp.dev["g"], inp.exact["g"] = W.round_to(g, "bf16")
    banner("mfma gla tiny gates")
    check(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
def test_mfma_matches_valu_path(variant):
    inp = W.make_inputs(wl_for(variant, 2, 2, 333, 64, seed=11), with_state=True)
    d = inputs_to_device(inp)
    banner(f"mfma vs valu {variant}")
    a = run_gpu(inp, d, path="mfma")
    b = run_gpu(inp, d, path="valu")
    assert relerr(a[0], f64(b[0])) < 2e-2 and relerr(a[1], f64(b[1])) < 2e-2


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
def test_mfma_deterministic_and_batch_invariant(variant):
    inp = W.make_inputs(wl_for(variant, 2, 3, 257, 64, seed=5), with_state=True)
    d = inputs_to_device(inp)
    banner(f"determinism/batch invariance {variant}")
    o1, S1, _ = run_gpu(inp, d, segments=2)
    o2, S2, _ = run_gpu(inp, d, segments=2)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # sequence (1, 2) alone
    one = {k: (v[1:2, 2:3].contiguous() if v is not None else None) for k, v in d.items()}
    o3, S3, _ = run_gpu(inp, one, segments=2)
    assert torch.equal(o3[0, 0], o1[1, 2]) and torch.equal(S3[0, 0], S1[1, 2])


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
def test_mfma_causality(variant):
    inp = W.make_inputs(wl_for(variant, 1, 2, 200, 32, seed=6), with_state=True)
    d = inputs_to_device(inp)
    banner(f"causality {variant}")
    o, _, _ = run_gpu(inp, d, segments=1)
    for tp in (0, 37, 64, 150):
        d2 = {k: (v.clone() if v is not None else None) for k, v in d.items()}
        d2["q"][:, :, tp] += 1
        d2["k"][:, :, tp] -= 1
        d2["v"][:, :, tp] *= -2
        if variant != "kath":
            d2["g"][:, :, tp] *= 0.5
        o2, _, _ = run_gpu(inp, d2, segments=1)
        assert torch.equal(o2[:, :, :tp], o[:, :, :tp]), tp
        assert not torch.equal(o2[:, :, tp], o[:, :, tp])


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
def test_mfma_split_at_chunk_boundary_is_exact(variant):
    inp = W.make_inputs(wl_for(variant, 1, 2, 320, 64, seed=8), with_state=True)
    d = inputs_to_device(inp)
    banner(f"split carry {variant}")
    o, S, z = run_gpu(inp, d, segments=1)
    for m in (128, 100):
        sl = lambda t, a_, b_: t[:, :, a_:b_].contiguous()
        left = {k: (sl(v, 0, m) if k in ("q", "k", "v", "g", "beta") else v) for k, v in d.items()}
        oL, SL, zL = run_gpu(inp, left, segments=1)
        right = {k: (sl(v, m, 320) if k in ("q", "k", "v", "g", "beta") else v) for k, v in d.items()}
        right["S0"] = SL
        if variant == "kath":
            right["z0"] = zL
        oR, SR, zR = run_gpu(inp, right, segments=1)
        if m % 64 == 0:
            assert torch.equal(torch.cat([oL, oR], 2), o) and torch.equal(SR, S)
        else:
            assert relerr(torch.cat([oL, oR], 2), f64(o)) < 2e-2 and relerr(SR, f64(S)) < 1e-2


@pytest.mark.parametrize("variant", ["kath", "gla", "gdn", "kda", "ssd"])
@pytest.mark.parametrize("segments", [1, 5])
def test_mfma_in_place_state(variant, segments):
    """S_final (and z_final) may be the very buffers of S0 (z0), also when the sequence
    is cut into segments that run side by side: the result equals the separate-buffer
    run bit for bit."""
    inp = W.make_inputs(wl_for(variant, 1, 3, 64 * 9 + 17, 64, seed=12), with_state=True)
    d = inputs_to_device(inp)
    banner(f"in-place state {variant} segments={segments}")
    o, S, z = run_gpu(inp, d, segments=segments)
    Sx = d["S0"].clone()
    zx = d["z0"].clone() if variant == "kath" else None
    d2 = dict(d, S0=Sx, z0=zx)
    o2, S2, z2 = run_gpu(inp, d2, segments=segments, S_final=Sx, z_final=zx)
    assert S2.data_ptr() == Sx.data_ptr()
    assert torch.equal(o2, o) and torch.equal(S2, S)
    if variant == "kath":
        assert z2.data_ptr() == zx.data_ptr() and torch.equal(z2, z)
    check(inp, (o2, S2, z2), run_oracle(inp))


@pytest.mark.parametrize("variant", ["gla", "gdn", "kath", "kda", "ssd"])
def test_prefill_then_decode_equals_longer_prefill(variant):
    N, extra = 192, 5
    inp = W.make_inputs(wl_for(variant, 1, 2, N + extra, 64, seed=12))
    d = inputs_to_device(inp)
    banner(f"prefill + decode {variant}")
    o_all, S_all, z_all = run_gpu(inp, d)
    head = {k: (v[:, :, :N].contiguous() if k in ("q", "k", "v", "g", "beta") else v)
            for k, v in d.items()}
    _, S, z = run_gpu(inp, head)
    for t in range(N, N + extra):
        tok = {k: (v[:, :, t].contiguous() if k in ("q", "k", "v", "g", "beta") else None)
               for k, v in d.items()}
        ot = bd.decode_step(tok["q"], tok["k"], tok["v"], S, tok.get("g"), tok.get("beta"),
                            variant=variant, z=z, eps=inp.wl.eps)
        torch.cuda.synchronize()
        assert relerr(ot, f64(o_all[:, :, t])) < 2e-2
    assert relerr(S, f64(S_all)) < 1e-2


# ---------------------------------------------------------------- full-size workloads

FULL = ["gla_bf16_b2h8_n2048_d128", "kath_bf16_b1h16_n32768_dk128_dv64",
        "gdn_bf16_b4h16_n8192_d128", "kda_bf16_b4h16_n8192_d128",
        "ssd_bf16_b2h32_n4096_dk128_dv64"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    """Full-size run in the benchmark's launch configuration; the oracle runs every
    sequence and o, S_final (z_final) are compared element by element on all of them."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl)
    banner(f"full workload {name}")
    got = run_gpu(inp, path="auto")
    ref = run_oracle(inp)
    errs = check(inp, got, ref)
    # the worst single sequence, against its own max|ref| (stricter than the per-tensor bound)
    nseq = wl.B * wl.H
    o = f64(got[0]).reshape(nseq, -1)
    o_ref = ref[0].reshape(nseq, -1)
    per_seq = np.max(np.abs(o - o_ref), axis=1) / np.max(np.abs(o_ref), axis=1)
    print(name, errs, "worst sequence o", float(per_seq.max()), int(per_seq.argmax()), flush=True)
    assert float(per_seq.max()) <= TOL["bf16"]


@pytest.mark.parametrize("N,dv,segments", [(64 * 20 + 3, 128, 2), (64 * 70 + 7, 16, 71),
                                           (64 * 8 + 1, 64, 3)])
def test_gla_segment_counts(N, dv, segments):
    """GLA with long segments (eleven chunks), with many short ones (71 segments, so the
    look-back of the last one reads 70 summaries), and with 64-column tiles."""
    inp = W.make_inputs(wl_for("gla", 1, 2, N, dv, seed=N % 97), with_state=True)
    banner(f"mfma gla N={N} dv={dv} segments={segments}")
    check(inp, run_gpu(inp, segments=segments), run_oracle(inp))
