"""Packed variable-length prefill (la_prefill_varlen) against the oracle per sequence and
against la_prefill on each sequence alone (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import TOL, banner, f64, inputs_to_device, relerr

pytestmark = pytest.mark.gpu

LENGTHS = [130, 0, 1, 64, 63, 257, 7, 192]


def seq_workload(variant, H, n, dk, dv, io, seed):
    kw = dict(seed=seed)
    if variant in ("gla",):
        kw.update(qk_scale=dk ** -0.5, v_scale=dk ** -0.5, gate_kind="slow")
    if variant == "ssd":
        kw.update(qk_scale=dk ** -0.5, v_scale=dk ** -0.5, gate_kind="slow")
    if variant in ("gdn", "kda"):
        kw.update(l2norm_qk=True, gate_kind="slow")
    return W.Workload("v", variant, 1, H, n, dk, dv, io, io, **kw)


def build_case(variant, H, dk, dv, io, lengths, seed=0):
    """Per-sequence inputs (seeded), packed along N, plus per-sequence S0 / z0."""
    seqs = [W.make_inputs(seq_workload(variant, H, n, dk, dv, io, seed + 17 * i), with_state=True)
            for i, n in enumerate(lengths)]
    names = [k for k in ("q", "k", "v", "g", "beta") if k in seqs[0].dev]
    packed_dev = {k: np.concatenate([s.dev[k] for s in seqs], axis=2) for k in names}
    state = {k: np.concatenate([s.dev[k] for s in seqs], axis=0) for k in ("S0", "z0")
             if k in seqs[0].dev}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return seqs, packed_dev, state, cu


@pytest.mark.parametrize("variant,io,path", [
    ("kath", "bf16", "mfma"), ("gla", "bf16", "mfma"), ("gdn", "bf16", "mfma"), ("kda", "bf16", "mfma"),
    ("ssd", "bf16", "mfma"), ("kath", "f32", "valu"), ("gla", "f32", "valu"), ("gdn", "f32", "valu"),
    ("kda", "f32", "valu"), ("ssd", "f32", "valu")])
def test_varlen_matches_each_sequence(variant, io, path):
    H, dk, dv = 2, 128, 64
    seqs, packed, state, cu = build_case(variant, H, dk, dv, io, LENGTHS)
    d = inputs_to_device(type(seqs[0])(seqs[0].wl, {**packed, **state}, {}))
    cu_t = torch.from_numpy(cu).cuda()
    banner(f"varlen {variant} {io} path={path} lengths={LENGTHS}")
    segs = 1 if variant in ("kath", "gla", "ssd") else 0
    o, S, z = bd.prefill_varlen(d["q"], d["k"], d["v"], d.get("g"), d.get("beta"), variant=variant,
                                cu_seqlens=cu_t, max_seqlen=max(LENGTHS), S0=d["S0"],
                                z0=d.get("z0"), path=path, segments=segs)
    torch.cuda.synchronize()
    tol = TOL[io]
    for i, inp in enumerate(seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        e = inp.exact
        o_ref, S_ref, z_ref = oracle.prefill(variant, e["q"], e["k"], e["v"], e.get("g"), e.get("beta"),
                                             e["S0"], e.get("z0"), eps=inp.wl.eps)
        assert relerr(S[i:i + 1], S_ref) <= tol, (i, relerr(S[i:i + 1], S_ref))
        if variant == "kath":
            assert relerr(z[i:i + 1], z_ref) <= tol
        if b > a:
            assert relerr(o[:, :, a:b], o_ref) <= tol, (i, relerr(o[:, :, a:b], o_ref))
        # the same sequence alone through la_prefill: identical arithmetic
        if b > a:
            di = inputs_to_device(inp)
            oi, Si, zi = bd.prefill(di["q"], di["k"], di["v"], di.get("g"), di.get("beta"),
                                    variant=variant, S0=di["S0"], z0=di.get("z0"), path=path,
                                    segments=segs)
            torch.cuda.synchronize()
            assert torch.equal(oi, o[:, :, a:b]), i
            assert torch.equal(Si, S[i:i + 1]), i


@pytest.mark.parametrize("variant", ["kath", "gla", "ssd"])
def test_varlen_segments(variant):
    """Sequences of different lengths cut into several segments each (segments past a
    short sequence's end are identity steps)."""
    H, dk, dv = 2, 128, 64
    lengths = [640, 65, 0, 333]
    seqs, packed, state, cu = build_case(variant, H, dk, dv, "bf16", lengths, seed=5)
    d = inputs_to_device(type(seqs[0])(seqs[0].wl, {**packed, **state}, {}))
    cu_t = torch.from_numpy(cu).cuda()
    banner(f"varlen segments {variant}")
    o, S, z = bd.prefill_varlen(d["q"], d["k"], d["v"], d.get("g"), variant=variant,
                                cu_seqlens=cu_t, max_seqlen=max(lengths), S0=d["S0"],
                                z0=d.get("z0"), path="mfma", segments=5)
    torch.cuda.synchronize()
    for i, inp in enumerate(seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        e = inp.exact
        o_ref, S_ref, z_ref = oracle.prefill(variant, e["q"], e["k"], e["v"], e.get("g"), None,
                                             e["S0"], e.get("z0"), eps=inp.wl.eps)
        assert relerr(S[i:i + 1], S_ref) <= TOL["bf16"]
        if b > a:
            assert relerr(o[:, :, a:b], o_ref) <= TOL["bf16"]


def test_varlen_all_empty_copies_state():
    H, dk, dv = 2, 64, 32
    cu_t = torch.zeros(4, dtype=torch.int32, device="cuda")
    q = torch.randn(1, H, 5, dk, device="cuda")
    v = torch.randn(1, H, 5, dv, device="cuda")
    S0 = torch.randn(3, H, dk, dv, device="cuda")
    banner("varlen all empty")
    o, S, _ = bd.prefill_varlen(q, q, v, torch.rand(1, H, 5, dk, device="cuda"), variant="gla",
                                cu_seqlens=cu_t, max_seqlen=0, S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


@pytest.mark.parametrize("name", list(W.VARLEN))
def test_varlen_workload(name):
    """The benchmark's packed batches at full size; every sequence against the oracle."""
    wl, inp, cu, lengths = W.make_varlen_inputs(name)
    d = inputs_to_device(inp)
    cu_t = torch.from_numpy(cu).cuda()
    banner(f"varlen workload {name}: {len(lengths)} sequences, {int(cu[-1])} tokens")
    o, S, _ = bd.prefill_varlen(d["q"], d["k"], d["v"], d.get("g"), d.get("beta"),
                                variant=wl.variant, cu_seqlens=cu_t, max_seqlen=int(lengths.max()))
    torch.cuda.synchronize()
    e = inp.exact
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        sl = lambda x: None if x is None else x[:, :, a:b]
        o_ref, S_ref, _ = oracle.prefill(wl.variant, sl(e["q"]), sl(e["k"]), sl(e["v"]),
                                         sl(e.get("g")), sl(e.get("beta")), eps=wl.eps)
        eo, eS = relerr(o[:, :, a:b], o_ref), relerr(S[i:i + 1], S_ref)
        print(name, i, b - a, eo, eS, flush=True)
        assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (i, eo, eS)
