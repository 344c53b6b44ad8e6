"""Decode at its full configuration, as the benchmark runs it: 8,192 states (256 sequences x
32 heads, d_k = d_v = 128; SSD: 256 x 64 heads, d_k = 128, d_v = 64), fp32 state drawn with
standard deviation 0.02, 1000 in-place la_decode_step calls, step s taking token set s mod 8
of a pool of 8 ("线性注意力与 SSM", section 01: decode carries only the final recurrent state,
so a run of steps is one state updated in place).

The fp64 oracle steps every head through the same 1000 tokens (heads are independent, so it
walks them in blocks of 128 heads, all 1000 steps per block, which keeps a block's states in
the host caches). o and S are compared per tensor on every head after step 1 and after step
1000: o at the bf16 bound (2e-2 of max|ref|), S at the fp32 bound (1e-5), since the state is
fp32 and every step's arithmetic is fp32.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_linear_amd import binding as bd
from gated_delta_rule_linear_amd import workloads as W
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu

STEPS = 1000
BLOCK = 128   # heads per oracle block


class MaxErr:
    """max|gpu - ref| and max|ref| accumulated over blocks of one tensor."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, gpu, ref):
        g = np.asarray(gpu, np.float64)
        assert g.shape == ref.shape, (g.shape, ref.shape)
        assert np.all(np.isfinite(g)), "non-finite GPU output"
        self.num = max(self.num, float(np.max(np.abs(g - ref))))
        self.den = max(self.den, float(np.max(np.abs(ref))))

    @property
    def rel(self):
        return self.num / self.den if self.den > 0 else self.num


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode_gdn_256x32_d128", "decode_gla_256x32_d128",
                                  "decode_kda_256x32_d128", "decode_ssd_256x64_dk128_dv64"])
def test_decode_full_config_1000_steps(name):
    wl = W.WORKLOADS[name]
    banner(f"decode full config {name}: {wl.B}x{wl.H} states, {STEPS} steps")
    S32, S64, sets = W.make_decode_pool(wl)
    nh = wl.B * wl.H
    # GPU: 1000 in-place steps through the C ABI, as the benchmark calls them
    S = torch.from_numpy(S32).cuda()
    del S32
    dsets = [{k: dev(v) for k, v in s.dev.items()} for s in sets]
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=torch.bfloat16, device="cuda")
    desc = bd.make_desc(wl.variant, wl.B, wl.H, 1, wl.dk, wl.dv, bd.LA_BF16, bd.LA_BF16, wl.eps)
    lib = bd.load()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = [(P(d["q"]), P(d["k"]), P(d["v"]), P(d.get("g")), P(d.get("beta")), P(S), None, P(o))
            for d in dsets]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    got = {}
    for s in range(STEPS):
        rc = lib.la_decode_step(ctypes.byref(desc), *args[s % len(args)], stream)
        assert rc == 0, bd.status_str(rc)
        if s == 0 or s == STEPS - 1:
            torch.cuda.synchronize()
            got[s] = (o.float().cpu().numpy().reshape(nh, wl.dv),
                      S.cpu().numpy().reshape(nh, wl.dk, wl.dv))
    del S
    torch.cuda.empty_cache()

    # oracle: all 1000 steps per block of heads
    flat = lambda a: a.reshape((1, nh) + a.shape[2:])
    ex = [{k: flat(v) for k, v in s.exact.items()} for s in sets]
    S64 = S64.reshape(1, nh, wl.dk, wl.dv)
    errs = {(s, t): MaxErr() for s in (0, STEPS - 1) for t in ("o", "S")}
    for h0 in range(0, nh, BLOCK):
        h1 = min(nh, h0 + BLOCK)
        Sb = np.ascontiguousarray(S64[:, h0:h1])
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, h0:h1])
        for s in range(STEPS):
            e = ex[s % len(ex)]
            ob = oracle.decode_step(wl.variant, sl(e["q"]), sl(e["k"]), sl(e["v"]), Sb,
                                    g=sl(e.get("g")), beta=sl(e.get("beta")), eps=wl.eps)
            if s in got:
                go, gS = got[s]
                errs[(s, "o")].add(go[h0:h1], ob[0])
                errs[(s, "S")].add(gS[h0:h1], Sb[0])
    report = {f"step{s + 1}_{t}": round(m.rel, 9) for (s, t), m in errs.items()}
    print(name, report, flush=True)
    for (s, t), m in errs.items():
        bound = 2e-2 if t == "o" else 1e-5
        assert m.rel <= bound, f"{name} step {s + 1} {t}: {m.rel:.3e} > {bound} ({report})"
