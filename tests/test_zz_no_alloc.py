"""la_prefill_noalloc against la_prefill (GPU): the same kernels with the workspace taken
from the library's fixed per-device array instead of a caller buffer. Two calls in a row,
the second smaller, each must equal la_prefill's result bit for bit; a descriptor whose
workspace exceeds the array is rejected before anything runs."""
import ctypes

import pytest
import torch

from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu

P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(lib, wl, d, noalloc):
    io = bd.LA_BF16 if wl.io == "bf16" else bd.LA_F32
    desc = bd.make_desc(wl.variant, wl.B, wl.H, wl.N, wl.dk, wl.dv, io, io, wl.eps)
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    o = torch.full((wl.B, wl.H, wl.N, wl.dv), 7.0, dtype=dt, device="cuda")
    S = torch.full((wl.B, wl.H, wl.dk, wl.dv), 7.0, device="cuda")
    z = torch.full((wl.B, wl.H, wl.dk), 7.0, device="cuda") if wl.variant == "kath" else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (P(d["q"]), P(d["k"]), P(d["v"]), P(d.get("g")), P(d.get("beta")), P(d.get("S0")),
            P(d.get("z0")), P(o), P(S), P(z))
    if noalloc:
        rc = lib.la_prefill_noalloc(ctypes.byref(desc), *args, stream)
    else:
        n = ctypes.c_size_t(0)
        assert lib.la_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n)) == 0
        ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device="cuda")
        rc = lib.la_prefill(ctypes.byref(desc), *args, P(ws) if n.value else None, int(n.value),
                            stream)
    torch.cuda.synchronize()
    assert rc == 0, bd.status_str(rc)
    return o, S, z


@pytest.mark.parametrize("variant", ["gla", "gdn", "kath", "ssd", "kda"])
def test_noalloc_equals_prefill_twice(variant):
    lib = bd.load()
    big = W.Workload("na", variant, 2, 4, 700, 128, 64, "bf16", "bf16", seed=5,
                     qk_scale=(1.0 if variant == "kath" else 128 ** -0.5),
                     l2norm_qk=variant in ("gdn", "kda"))
    small = big.with_(B=1, H=3, N=130, seed=6)
    for wl in (big, small):   # the second call is smaller and reuses the array
        inp = W.make_inputs(wl, with_state=True)
        d = {k: dev(v) for k, v in inp.dev.items()}
        banner(f"noalloc {variant} B{wl.B} H{wl.H} N{wl.N}")
        ref = _call(lib, wl, d, noalloc=False)
        got = _call(lib, wl, d, noalloc=True)
        for a, b in zip(got, ref):
            if a is not None:
                assert torch.equal(a, b)


def test_noalloc_rejects_oversized_workspace():
    """A KDA call whose workspace exceeds the array: LA_ERR_WORKSPACE, outputs untouched."""
    lib = bd.load()
    wl = W.Workload("na", "kda", 4, 16, 2048, 128, 128, "bf16", "bf16", seed=1, l2norm_qk=True)
    desc = bd.make_desc("kda", wl.B, wl.H, wl.N, 128, 128, bd.LA_BF16, bd.LA_BF16)
    n = ctypes.c_size_t(0)
    assert lib.la_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n)) == 0
    limit = 64 << 20
    assert n.value > limit
    q = torch.zeros((wl.B, wl.H, wl.N, 128), dtype=torch.bfloat16, device="cuda")
    k, v, g = torch.zeros_like(q), torch.zeros_like(q), torch.ones_like(q)
    beta = torch.zeros((wl.B, wl.H, wl.N), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    S = torch.full((wl.B, wl.H, 128, 128), 3.0, device="cuda")
    banner("noalloc oversized workspace")
    rc = lib.la_prefill_noalloc(ctypes.byref(desc), P(q), P(k), P(v), P(g), P(beta), None, None,
                                P(o), P(S), None,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == bd.LA_ERR_WORKSPACE
    assert bool((o == 3.0).all()) and bool((S == 3.0).all())
