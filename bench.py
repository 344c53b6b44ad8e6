#!/usr/bin/env python3
"""Benchmark of the linear-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only WORKLOAD] [--no-cpu] [--no-extras]
(WORKLOAD may be backward_<prefill workload> for the backward of that prefill)

A step is one chunked prefill of the headline workload (GLA, B=2 H=8 N=2048
d_k=d_v=128, bf16 inputs, fp32 state, chunk 64) over one batch of seeded
synthetic inputs already resident in HBM. Eight distinct input sets rotate so
that the 43 MB working set does not sit in the 256 MB last-level cache. Exactly
K steps are timed: HIP graphs of those launches (the same kernels and work as
eager calls, without host launch gaps) replayed K // 8 times, plus a graph of the
K % 8 remaining calls; each graph's output is checked bit for bit against an
eager call first, and the eager time is reported beside it. Events between the
replays give per-step samples: the line reports the mean over the timed region
and the median, 10th and 90th percentiles.

The other workloads (Gated DeltaNet, KDA and Mamba-2 SSD prefill, long
normalized-attention prefill, packed variable-length batches, decode steps, the
backward, the selective scan, the small fp32 case) are timed the same way and
reported under "workloads", each with its roofline. Beside every workload the
fp64 oracle runs on a bounded sample of the same inputs on the host cores (its
rate and core count under "cpu_oracle"); its outputs are the parity reference of
the timed run's outputs on that sample ("parity": max|gpu - ref| / max|ref| per
tensor). One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill Mtok/s & MFMA util (GLA/GDN chunked); decode state-update HBM GB/s"
MAIN = "gla_bf16_b2h8_n2048_d128"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6    # dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
# Selective scan: each state update needs one exponential (v_exp_f32, which takes two issue
# slots: half the fp32 rate on gfx950, as a throughput probe of independent exponentials
# measures) and four other fp32 operations (two multiplies, two fused multiply-adds): six
# slots of a 16-lane SIMD. The chip issues 256 CU x 4 SIMD x 16 lanes x 2.4 GHz = 39.3 T
# fp32 lane operations per second without packed fp32 (157.3 TFLOP/s counts packed
# fused multiply-adds), so at most 39.3 T / 6 = 6.55 T state updates per second.
PEAK_SCAN_UPDATES = 256 * 4 * 16 * 2.4e9 / 6
PROFILES = os.path.join(ROOT, "profiles")
# the kernels one prefill step launches, per variant (the roofline covers the whole step)
STEP_KERNELS = {
    "gla": "gla_prep_kernel + gla_chain_kernel (summary) + gla_chain_kernel (forward)",
    "kath": "kath_chain_kernel (summary) + kath_scan_kernel + kath_chain_kernel",
    "gdn": "gdn_prep_kernel + gdn_fwd_kernel",
    "kda": "kda_prep_kernel + kda_fwd_kernel",
    "ssd": "ssd_chain_kernel (summary) + ssd_chain_kernel (forward; one pass over q, k, v, decays)",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_linear_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(name: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = t.get("workloads", {}).get(name)
    return None if w is None else w.get("hbm_bytes_per_step")


# ---------------------------------------------------------------------------


def to_dev(a, torch, device):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class PrefillCase:
    """Preallocated buffers and a lean ctypes call for repeated prefills."""

    def __init__(self, wl, rotate, torch, bd, W, device):
        import ctypes
        self.wl, self.torch, self.bd = wl, torch, bd
        inp = W.make_inputs(wl)
        self.exact = inp.exact
        base = {k: to_dev(v, torch, device) for k, v in inp.dev.items()}
        self.sets = [base]
        for r in range(1, rotate):   # distinct memory, same value distribution
            self.sets.append({k: torch.roll(v, shifts=97 * r, dims=2).contiguous()
                              for k, v in base.items()})
        io = bd.LA_BF16 if wl.io == "bf16" else bd.LA_F32
        gd = bd.LA_BF16 if wl.gate_io == "bf16" else bd.LA_F32
        self.desc = bd.make_desc(wl.variant, wl.B, wl.H, wl.N, wl.dk, wl.dv, io, gd, wl.eps)
        self.ws_bytes = bd.prefill_workspace_bytes(self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
        self.outs = []
        for _ in self.sets:
            o = torch.empty((wl.B, wl.H, wl.N, wl.dv), dtype=dt, device=device)
            S = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=device)
            z = (torch.empty((wl.B, wl.H, wl.dk), dtype=torch.float32, device=device)
                 if wl.variant == "kath" else None)
            self.outs.append((o, S, z))
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        self.args = []
        for s, (o, S, z) in zip(self.sets, self.outs):
            self.args.append((P(s["q"]), P(s["k"]), P(s["v"]), P(s.get("g")), P(s.get("beta")),
                              None, None, P(o), P(S), P(z),
                              P(self.ws) if self.ws_bytes else None, self.ws_bytes))
        self.lib = bd.load()
        self.pdesc = ctypes.byref(self.desc)
        self.ctypes = ctypes

    def call(self, i, stream):
        a = self.args[i % len(self.args)]
        rc = self.lib.la_prefill(self.pdesc, *a, self.ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise self.bd.LinAttnError(rc, "la_prefill")


def summarize(samples):
    """Median and 10th / 90th percentiles of per-call times (ms)."""
    import numpy as np
    a = np.asarray(samples, dtype=np.float64)
    return {"ms_median": float(np.median(a)), "ms_p10": float(np.percentile(a, 10)),
            "ms_p90": float(np.percentile(a, 90)), "timed_samples": int(a.size)}


def time_calls(fn, n, warmup, torch, stream):
    """n calls on `stream`, an event recorded after each one. Returns (mean ms per call over
    the whole timed region, per-call ms)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[n]) / n, [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def time_graph(case, steps, warmup, torch, stream, per_graph=8):
    """Exactly `steps` calls replayed from HIP graphs: a graph of per_graph consecutive calls
    (rotating input sets) replayed steps // per_graph times, then a graph of the remaining
    steps % per_graph calls. Returns (mean ms per call, per-call ms of each full replay)."""
    per_graph = max(1, min(per_graph, len(case.sets), steps))
    full, rem = divmod(steps, per_graph)
    graphs = []
    for count in (per_graph, rem):
        if count == 0:
            graphs.append(None)
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                case.call(i, stream)
        graphs.append(g)
    for _ in range(max(1, warmup)):
        graphs[0].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(full + 2)]
    ev[0].record(stream)
    for r in range(full):
        graphs[0].replay()
        ev[r + 1].record(stream)
    if graphs[1] is not None:
        graphs[1].replay()
    ev[full + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / per_graph for r in range(full)]
    return ev[0].elapsed_time(ev[full + 1]) / steps, per, graphs


def prefill_record(name, ms, wl, W, chunk=64):
    byts = W.algorithmic_bytes(wl)
    flops = W.algorithmic_flops(wl, chunk=chunk)
    s = ms / 1e3
    gbs = byts / s / 1e9
    tfl = flops / s / 1e12
    return {
        "ms": ms,
        "Mtok_per_s": wl.B * wl.N / s / 1e6,
        "token_heads_per_s": wl.token_heads / s,
        "GB_per_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
        "TFLOP_per_s": tfl, "mfma_frac": tfl / PEAK_BF16_TFLOPS,
        "algorithmic_bytes": byts, "algorithmic_flops": flops,
        "binding_frac": max(byts / (PEAK_HBM_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12)) / s,
    }


def bench_prefill(name, steps, warmup, rotate, torch, bd, W, device, stream, graph=True):
    wl = W.WORKLOADS[name]
    log(f"prefill {name}: generating inputs")
    case = PrefillCase(wl, rotate, torch, bd, W, device)
    fn = lambda i: case.call(i, stream)
    ms_eager, per = time_calls(fn, steps, warmup, torch, stream)
    rec = {"workload": name, "eager_ms": ms_eager, "timed_calls": steps}
    ms = ms_eager
    if graph:
        # eager reference outputs of set 0, then graph replay must reproduce them exactly
        case.call(0, stream)
        torch.cuda.synchronize()
        ref = [t.clone() if t is not None else None for t in case.outs[0]]
        ms_g, per_g, graphs = time_graph(case, steps, warmup, torch, stream)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(case.outs[0], ref) if a is not None)
        rec["graph_replay_matches_eager"] = bool(same)
        if not same:
            log(f"{name}: graph replay differs from eager; reporting eager timing")
        else:
            rec["graph_ms"] = ms = ms_g
            per = per_g
        del graphs
    rec.update(prefill_record(name, ms, wl, W))
    rec.update(summarize(per))
    o = case.outs[0][0]
    rec["finite"] = bool(torch.isfinite(o.float()).all().item())
    return rec, case


def bench_varlen(name, steps, warmup, torch, bd, W, device, stream):
    """Packed variable-length prefill: sum of the sequence lengths per second."""
    import ctypes
    wl, inp, cu, lengths = W.make_varlen_inputs(name)
    log(f"varlen {name}: {len(lengths)} sequences, {int(cu[-1])} tokens per head")
    sets = [{k: to_dev(v, torch, device) for k, v in inp.dev.items()}]
    sets.append({k: torch.roll(v, shifts=97, dims=2).contiguous() for k, v in sets[0].items()})
    cu_t = torch.from_numpy(cu).to(device)
    nseq, maxlen = len(lengths), int(lengths.max())
    io = bd.LA_BF16 if wl.io == "bf16" else bd.LA_F32
    desc = bd.make_desc(wl.variant, 1, wl.H, wl.N, wl.dk, wl.dv, io, io, wl.eps)
    lib = bd.load()
    n = ctypes.c_size_t(0)
    rc = lib.la_prefill_varlen_workspace_size(ctypes.byref(desc), nseq, maxlen, ctypes.byref(n))
    if rc != 0:
        raise bd.LinAttnError(rc, "la_prefill_varlen_workspace_size")
    ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device)
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = []
    for s in sets:
        o = torch.empty((1, wl.H, wl.N, wl.dv), dtype=dt, device=device)
        S = torch.empty((nseq, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=device)
        args.append(((P(s["q"]), P(s["k"]), P(s["v"]), P(s.get("g")), P(s.get("beta")), None, None,
                      P(o), P(S), None, P(ws) if n.value else None, int(n.value)), o, S))
    pd = ctypes.byref(desc)
    sh = ctypes.c_void_p(stream.cuda_stream)
    pcu = P(cu_t)

    def fn(i):
        a = args[i % len(args)][0]
        rc = lib.la_prefill_varlen(pd, nseq, pcu, maxlen, *a, sh)
        if rc != 0:
            raise bd.LinAttnError(rc, "la_prefill_varlen")

    ms, per = time_calls(fn, steps, warmup, torch, stream)
    tokens = int(cu[-1])
    per_tok = W.algorithmic_bytes_per_token_head(wl)
    byts = tokens * wl.H * per_tok + nseq * wl.H * wl.dk * wl.dv * 4
    flops = W.algorithmic_flops(wl)   # the packed layout's token count, B = 1
    s = ms / 1e3
    gbs = byts / s / 1e9
    rec = {"workload": name, "ms": ms, "timed_calls": steps, "sequences": nseq, "tokens": tokens,
           "length_min": int(lengths.min()), "length_max": maxlen,
           "Mtok_per_s": tokens / s / 1e6, "GB_per_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
           "TFLOP_per_s": flops / s / 1e12, "mfma_frac": flops / s / 1e12 / PEAK_BF16_TFLOPS,
           "finite": bool(torch.isfinite(args[0][1].float()).all().item())}
    rec.update(summarize(per))
    out = {"o": args[0][1], "S": args[0][2]}
    return rec, (wl, inp, cu, lengths, out)


def bench_decode(name, steps, warmup, torch, bd, W, device, stream, check_heads=1024):
    """`steps` in-place decode steps (token set s mod 8). After the timed steps, one more
    step runs from a saved copy of the first check_heads states, for the oracle leg to
    compare against (o and S of that step)."""
    import ctypes
    wl = W.WORKLOADS[name]
    log(f"decode {name}: generating state and token pool")
    S32, S64, sets = W.make_decode_pool(wl, with_exact=True)
    del S64
    S = torch.from_numpy(S32).to(device)
    del S32
    dsets = [{k: to_dev(v, torch, device) for k, v in s.dev.items()} for s in sets]
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=torch.bfloat16, device=device)
    desc = bd.make_desc(wl.variant, wl.B, wl.H, 1, wl.dk, wl.dv, bd.LA_BF16, bd.LA_BF16, wl.eps)
    lib = bd.load()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = [(P(d["q"]), P(d["k"]), P(d["v"]), P(d.get("g")), P(d.get("beta")), P(S), None, P(o))
            for d in dsets]
    pd = ctypes.byref(desc)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def fn(i):
        rc = lib.la_decode_step(pd, *args[i % len(args)], sh)
        if rc != 0:
            raise bd.LinAttnError(rc, "la_decode_step")

    ms, per = time_calls(fn, steps, warmup, torch, stream)
    byts = W.algorithmic_bytes(wl)
    flops = W.algorithmic_flops(wl)
    s = ms / 1e3
    gbs = byts / s / 1e9
    rec = {"workload": name, "ms": ms, "us_per_step": ms * 1e3, "GB_per_s": gbs,
           "hbm_frac": gbs / PEAK_HBM_GBS, "TFLOP_per_s": flops / s / 1e12,
           "algorithmic_bytes": byts, "timed_calls": steps,
           "finite": bool(torch.isfinite(S).all().item())}
    rec.update(summarize(per))
    # the ceiling beside it: the plain in-place pass over the same state bytes
    # (la_stream_rmw, x <- 1 x), timed the same way
    sbytes = S.numel() * S.element_size()

    def rmw(i):
        rc = lib.la_stream_rmw(ctypes.c_void_p(S.data_ptr()), S.numel(), ctypes.c_float(1.0), sh)
        if rc != 0:
            raise bd.LinAttnError(rc, "la_stream_rmw")

    ms_c, per_c = time_calls(rmw, steps, warmup, torch, stream)
    rec["ceiling"] = {"kernel": "la_stream_rmw", "bytes": 2 * sbytes, "us_per_step": ms_c * 1e3,
                      "GB_per_s": 2 * sbytes / (ms_c / 1e3) / 1e9,
                      "step_over_ceiling": ms / ms_c, "us_median": summarize(per_c)["ms_median"] * 1e3}
    # the check step: token set j from the current states of the first check_heads heads
    nh = wl.B * wl.H
    hc = min(check_heads, nh)
    S_before = S.reshape(nh, wl.dk, wl.dv)[:hc].double().cpu().numpy()
    j = (warmup + steps) % len(sets)
    fn(j)
    torch.cuda.synchronize()
    chk = {"heads": hc, "set": sets[j], "S_before": S_before,
           "o": o.reshape(nh, wl.dv)[:hc].float().cpu().numpy(),
           "S": S.reshape(nh, wl.dk, wl.dv)[:hc].float().cpu().numpy()}
    return rec, chk


def bench_selscan(name, steps, warmup, torch, bd, W, device, stream, graph=True):
    """Mamba-1 selective scan: state updates (Bt T D n) and tokens per second."""
    import ctypes
    wl = W.SELSCAN[name]
    log(f"selective scan {name}: generating inputs")
    sets, exact0 = [], None
    for r in range(2):
        d, ex = W.make_selscan_inputs(wl, with_state=True, seed=wl.seed + 100 * r)
        sets.append({k: to_dev(v, torch, device) for k, v in d.items()})
        if r == 0:
            exact0 = ex
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    io = bd.LA_BF16 if wl.io == "bf16" else bd.LA_F32
    desc = bd.ScanDesc(wl.Bt, wl.T, wl.D, wl.n, io, 1)
    lib = bd.load()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    outs, args = [], []
    for s_ in sets:
        y = torch.empty((wl.Bt, wl.T, wl.D), dtype=dt, device=device)
        h = torch.empty((wl.Bt, wl.D, wl.n), dtype=torch.float32, device=device)
        outs.append((y, h))
        args.append((P(s_["dt"]), P(s_["A"]), P(s_["Bm"]), P(s_["Cm"]), P(s_["x"]),
                     P(s_["Dskip"]), P(s_["dt_bias"]), P(s_["h0"]), P(y), P(h)))
    pd = ctypes.byref(desc)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def fn(i):
        rc = lib.la_selective_scan(pd, *args[i % len(args)], sh)
        if rc != 0:
            raise bd.LinAttnError(rc, "la_selective_scan")

    ms, per = time_calls(fn, steps, warmup, torch, stream)
    rec = {"workload": name, "eager_ms": ms, "timed_calls": steps}
    if graph:
        fn(0)
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs[0]]

        class _Case:   # the graph helper's view: one call per input set
            def __init__(self):
                self.sets = sets

            def call(self, i, stream_):
                fn(i)

        gms, gper, graphs = time_graph(_Case(), steps, warmup, torch, stream, per_graph=2)
        same = all(torch.equal(a, b) for a, b in zip(outs[0], ref))
        rec["graph_replay_matches_eager"] = bool(same)
        if same:
            rec["graph_ms"] = ms = gms
            per = gper
        del graphs
    s = ms / 1e3
    updates = wl.Bt * wl.T * wl.D * wl.n
    byts = W.selscan_algorithmic_bytes(wl)
    rec.update({"ms": ms, "Mtok_per_s": wl.Bt * wl.T / s / 1e6,
                "G_state_updates_per_s": updates / s / 1e9,
                "alu_frac": updates / s / PEAK_SCAN_UPDATES,
                "GB_per_s": byts / s / 1e9, "hbm_frac": byts / s / 1e9 / PEAK_HBM_GBS,
                "algorithmic_bytes": byts, "state_updates": updates,
                "finite": bool(torch.isfinite(outs[0][0].float()).all().item())})
    rec.update(summarize(per))
    return rec, (wl, exact0, outs[0])


def bench_backward(name, steps, warmup, torch, bd, W, device, stream):
    """Backward of the prefill (the default path: matrix cores for SSD, fp32 VALU for KATH,
    GLA, GDN and KDA):
    tokens per second of the whole backward (every kernel of la_prefill_backward)."""
    import ctypes
    import numpy as np
    wl = W.WORKLOADS[name]
    log(f"backward {name}: generating inputs")
    inp = W.make_inputs(wl)
    d = {k: to_dev(v, torch, device) for k, v in inp.dev.items()}
    rng = np.random.default_rng(wl.seed + 500)
    dO_st, dO_x = W.round_to(rng.standard_normal((wl.B, wl.H, wl.N, wl.dv)), wl.io)
    dO = to_dev(dO_st, torch, device)
    io = bd.LA_BF16 if wl.io == "bf16" else bd.LA_F32
    desc = bd.make_desc(wl.variant, wl.B, wl.H, wl.N, wl.dk, wl.dv, io, io, wl.eps, "auto")
    lib = bd.load()
    n = ctypes.c_size_t(0)
    rc = lib.la_prefill_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != 0:
        raise bd.LinAttnError(rc, "la_prefill_backward_workspace_size")
    ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device)
    outs = [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
            torch.empty_like(d["g"]) if "g" in d else None,
            torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=device),
            torch.empty_like(d["beta"]) if "beta" in d else None,
            torch.empty((wl.B, wl.H, wl.dk), dtype=torch.float32, device=device)
            if wl.variant == "kath" else None]
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = (P(d["q"]), P(d["k"]), P(d["v"]), P(d.get("g")), P(d.get("beta")), None, None,
            P(dO), None, None, P(outs[0]), P(outs[1]), P(outs[2]), P(outs[3]), P(outs[5]),
            P(outs[4]), P(outs[6]), P(ws), int(n.value), ctypes.c_void_p(stream.cuda_stream))
    pd = ctypes.byref(desc)

    def fn(i):
        rc = lib.la_prefill_backward(pd, *args)
        if rc != 0:
            raise bd.LinAttnError(rc, "la_prefill_backward")

    ms, per = time_calls(fn, steps, warmup, torch, stream)
    s = ms / 1e3
    # algorithmic bytes: the forward's inputs and dO read, dq, dk, dv, dg and dS0 written
    per_tok = W.algorithmic_bytes_per_token_head(wl)
    isz = 4 if wl.io == "f32" else 2
    byts = wl.token_heads * (2 * per_tok - wl.dv * isz) + wl.B * wl.H * wl.dk * wl.dv * 4
    rec = {"workload": name + " (backward)", "ms": ms, "timed_calls": steps,
           "Mtok_per_s": wl.B * wl.N / s / 1e6,
           "GB_per_s": byts / s / 1e9, "hbm_frac": byts / s / 1e9 / PEAK_HBM_GBS,
           "algorithmic_bytes": byts, "workspace_bytes": int(n.value),
           "finite": bool(torch.isfinite(outs[0].float()).all().item())}
    rec.update(summarize(per))
    got = {"dq": outs[0], "dk": outs[1], "dv": outs[2], "dS0": outs[4]}
    if outs[3] is not None:
        got["dg"] = outs[3]
    if outs[5] is not None:
        got["dbeta"] = outs[5]
    if outs[6] is not None:
        got["dz0"] = outs[6]
    return rec, (wl, inp.exact, dO_x, got)


def relerr(gpu, ref):
    """max|gpu - ref| / max|ref| over one output tensor (the parity metric of the tests)."""
    import numpy as np
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if hasattr(gpu, "detach") \
        else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(g - r))) if r.size else 0.0
    return num / den if den > 0 else num


def _repeat(call, min_wall_s):
    """Run call() until about min_wall_s of wall time is timed; (reps, seconds, last result)."""
    reps, tk, out = 0, 0.0, None
    while reps == 0 or (tk < min_wall_s and reps < 1000):
        t0 = time.perf_counter()
        out = call()
        tk += time.perf_counter() - t0
        reps += 1
    return reps, tk, out


def cpu_baseline(case, wl, budget_s=8.0, min_wall_s=10.0):
    """Time the fp64 oracle on a bounded sample of the workload's sequences (input set 0 of
    the timed run). When the sample finishes quickly, the same call repeats until about
    min_wall_s of wall time has been timed and the mean rate is reported. The oracle's
    outputs for the sample are the parity reference of the GPU's outputs for that set."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    nseq = wl.B * wl.H
    e = case.exact
    flat = lambda a: None if a is None else a.reshape((-1,) + a.shape[2:])
    fe = {k: flat(v) for k, v in e.items()}
    # one sequence first, single-threaded (a per-core rate), then a batch across cores
    t0 = time.perf_counter()
    sel = lambda a, idx: None if a is None else a[idx][None]
    oracle.prefill(wl.variant, sel(fe["q"], [0]), sel(fe["k"], [0]), sel(fe["v"], [0]),
                   sel(fe.get("g"), [0]), sel(fe.get("beta"), [0]), eps=wl.eps, threads=1)
    t1 = time.perf_counter() - t0
    per_seq = max(t1, 1e-6)
    k = int(min(nseq, max(1, cores * max(1, int(budget_s / per_seq)))))
    k = min(k, nseq)
    idx = list(range(k))
    threads = min(cores, k)
    args = (sel(fe["q"], idx), sel(fe["k"], idx), sel(fe["v"], idx), sel(fe.get("g"), idx),
            sel(fe.get("beta"), idx))
    reps, tk, ref = _repeat(lambda: oracle.prefill(wl.variant, *args, eps=wl.eps,
                                                   threads=threads), min_wall_s)
    tokens = reps * k / wl.H * wl.N   # B*N tokens per repetition = sequences / H * N
    o, S, z = case.outs[0]
    fl = lambda t: t.reshape((-1,) + tuple(t.shape[2:]))[:k][None]
    parity = {"sequences": k, "o": relerr(fl(o), ref[0]), "S_final": relerr(fl(S), ref[1])}
    if z is not None:
        parity["z_final"] = relerr(fl(z), ref[2])
    return {"value": tokens / tk / 1e6, "unit": "Mtok/s", "cores": threads, "kind": "oracle",
            "sample": f"{k} of {nseq} (b,h) sequences x N={wl.N} of {wl.name}, fp64 token "
                      f"recurrence, {threads} OpenMP threads, {reps} repetitions in {tk:.2f} s "
                      f"wall; single-thread one sequence {t1:.3f} s",
            "seconds": tk}, parity


def cpu_baseline_varlen(ctx, budget_s=2.0):
    """The oracle on the first sequences of a packed batch (every head), timed; parity of
    the GPU's o and S_final on them."""
    import numpy as np

    import oracle
    wl, inp, cu, lengths, out = ctx
    cores = len(os.sched_getaffinity(0))
    e = inp.exact
    k, tk, tokens, eo, eS = 0, 0.0, 0, 0.0, 0.0
    while k < len(lengths) and tk < budget_s:
        a, b = int(cu[k]), int(cu[k + 1])
        sl = lambda x: None if x is None else x[:, :, a:b]
        t0 = time.perf_counter()
        o_ref, S_ref, _ = oracle.prefill(wl.variant, sl(e["q"]), sl(e["k"]), sl(e["v"]),
                                         sl(e.get("g")), sl(e.get("beta")), eps=wl.eps,
                                         threads=min(cores, wl.H))
        tk += time.perf_counter() - t0
        tokens += b - a
        eo = max(eo, relerr(out["o"][:, :, a:b], o_ref))
        eS = max(eS, relerr(out["S"][k:k + 1], S_ref))
        k += 1
    cpu = {"value": tokens / tk / 1e6, "unit": "Mtok/s", "cores": min(cores, wl.H),
           "kind": "oracle", "sample": f"first {k} of {len(lengths)} packed sequences "
           f"({tokens} tokens, every head), one oracle call per sequence", "seconds": tk}
    return cpu, {"sequences": k, "o": eo, "S_final": eS}


def cpu_baseline_decode(chk, wl, W, min_wall_s=2.0):
    """One decode step of the oracle on the checked heads from their saved states, timed
    (repeated on copies); parity of the GPU's o and S for that step."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    hc = chk["heads"]
    ex = {k: np.ascontiguousarray(v.reshape((1, -1) + v.shape[2:])[:, :hc])
          for k, v in chk["set"].exact.items()}
    S0 = chk["S_before"].reshape(1, hc, wl.dk, wl.dv)

    def step():
        Sx = S0.copy()
        o = oracle.decode_step(wl.variant, ex["q"], ex["k"], ex["v"], Sx, g=ex.get("g"),
                               beta=ex.get("beta"), eps=wl.eps, threads=cores)
        return o, Sx

    reps, tk, (o_ref, S_ref) = _repeat(step, min_wall_s)
    t_full = tk / reps * (wl.B * wl.H) / hc
    parity = {"heads": hc, "o": relerr(chk["o"], o_ref[0]), "S": relerr(chk["S"], S_ref[0])}
    return {"value": W.algorithmic_bytes(wl) / t_full / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle", "us_per_step": t_full * 1e6,
            "sample": f"one step on {hc} of {wl.B * wl.H} heads (fp64 state copy included), "
                      f"{reps} repetitions in {tk:.2f} s, scaled to all heads",
            "seconds": tk}, parity


def cpu_baseline_backward(ctx, budget_s=3.0):
    """The oracle's reverse mode on a sample of sequences, timed; parity of every gradient
    of the timed GPU call on them."""
    import oracle
    wl, e, dO_x, got = ctx
    cores = len(os.sched_getaffinity(0))
    flat = lambda a: None if a is None else a.reshape((-1,) + a.shape[2:])
    sel = lambda a, idx: None if a is None else flat(a)[idx][None]
    t0 = time.perf_counter()
    oracle.prefill_backward(wl.variant, sel(e["q"], [0]), sel(e["k"], [0]), sel(e["v"], [0]),
                            sel(e.get("g"), [0]), sel(e.get("beta"), [0]), dO=sel(dO_x, [0]),
                            eps=wl.eps, threads=1)
    t1 = max(time.perf_counter() - t0, 1e-6)
    nseq = wl.B * wl.H
    k = min(nseq, cores) if t1 < budget_s else 1
    idx = list(range(k))
    t0 = time.perf_counter()
    ref = oracle.prefill_backward(wl.variant, sel(e["q"], idx), sel(e["k"], idx),
                                  sel(e["v"], idx), sel(e.get("g"), idx), sel(e.get("beta"), idx),
                                  dO=sel(dO_x, idx), eps=wl.eps, threads=min(cores, k))
    tk = time.perf_counter() - t0
    parity = {"sequences": k}
    for name, t in got.items():
        parity[name] = relerr(t.reshape((-1,) + tuple(t.shape[2:]))[:k][None], ref[name])
    return {"value": k / wl.H * wl.N / tk / 1e6, "unit": "Mtok/s", "cores": min(cores, k),
            "kind": "oracle", "sample": f"{k} of {nseq} sequences, one call in {tk:.2f} s; "
            f"single-thread one sequence {t1:.2f} s", "seconds": tk}, parity


def cpu_baseline_selscan(ctx, channels=64):
    """The oracle scan of row 0 on the first `channels` channels, timed; parity of y and the
    final state there."""
    import numpy as np

    import oracle
    wl, ex, (y, h) = ctx
    cores = len(os.sched_getaffinity(0))
    c = min(channels, wl.D)
    pick = lambda a: np.ascontiguousarray(a[:1, :, :c])
    t0 = time.perf_counter()
    y_ref, h_ref = oracle.selective_scan(pick(ex["dt"]), ex["A"][:c], ex["Bm"][:1], ex["Cm"][:1],
                                         pick(ex["x"]), ex["Dskip"][:c], ex["dt_bias"][:c], True,
                                         np.ascontiguousarray(ex["h0"][:1, :c]), threads=cores)
    tk = time.perf_counter() - t0
    frac = c / wl.D / wl.Bt
    parity = {"rows": 1, "channels": c, "y": relerr(y[:1, :, :c], y_ref),
              "h_final": relerr(h[:1, :c], h_ref)}
    return {"value": wl.Bt * wl.T * frac / tk / 1e6, "unit": "Mtok/s (full-width equivalent)",
            "cores": cores, "kind": "oracle",
            "sample": f"row 0, channels 0..{c - 1} of {wl.D} ({wl.T} tokens) in {tk:.2f} s",
            "seconds": tk}, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None, help="time only this workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length lines (they launch the same kernels as "
                         "the dense workloads, which per-kernel counter passes must not mix)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (b, h) sequence is independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_linear_amd import binding as bd
    from gated_delta_rule_linear_amd import workloads as W

    if not os.path.exists(bd.LIB_PATH):
        raise SystemExit(f"{bd.LIB_PATH} missing: run `python -m gated_delta_rule_linear_amd.build`")
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    # all timed work runs on one side stream (default priority); graph capture needs a
    # non-default stream
    stream = torch.cuda.Stream(device)
    torch.cuda.set_stream(stream)
    use_graph = not args.no_graph

    if args.copy_calib:
        n = 512 << 20
        a = torch.empty(n, dtype=torch.uint8, device=device)
        b = torch.empty(n, dtype=torch.uint8, device=device)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 512 MiB device copies")

    results = {}
    main_name = args.only or MAIN
    cpu_on = not args.no_cpu

    def run_one(name, steps, warmup, headline=False):
        """Time one workload on the GPU, then (unless --no-cpu) its oracle leg beside it,
        whose outputs give the parity of the timed run's outputs."""
        cpu = parity = None
        if name.startswith("backward_"):
            rec, ctx = bench_backward(name[len("backward_"):], steps, warmup, torch, bd, W,
                                      device, stream)
            if cpu_on:
                cpu, parity = cpu_baseline_backward(ctx)
        elif name.startswith("decode"):
            rec, ctx = bench_decode(name, steps, warmup, torch, bd, W, device, stream)
            if cpu_on:
                cpu, parity = cpu_baseline_decode(ctx, W.WORKLOADS[name], W)
        elif name.startswith("selscan"):
            rec, ctx = bench_selscan(name, steps, warmup, torch, bd, W, device, stream,
                                     graph=use_graph)
            if cpu_on:
                cpu, parity = cpu_baseline_selscan(ctx)
        elif name in W.VARLEN:
            rec, ctx = bench_varlen(name, steps, warmup, torch, bd, W, device, stream)
            if cpu_on:
                cpu, parity = cpu_baseline_varlen(ctx)
        else:
            rotate = 8 if headline else 2
            rec, ctx = bench_prefill(name, steps, warmup, rotate, torch, bd, W, device, stream,
                                     graph=use_graph)
            if cpu_on:
                if headline:
                    cpu, parity = cpu_baseline(ctx, W.WORKLOADS[name])
                else:
                    cpu, parity = cpu_baseline(ctx, W.WORKLOADS[name], budget_s=1.5,
                                               min_wall_s=2.0)
        if cpu is not None:
            log(f"{name}: oracle {cpu['value']:.4g} {cpu['unit']}; parity {parity}")
        rec["cpu_oracle"] = cpu
        rec["parity"] = parity
        del ctx
        torch.cuda.empty_cache()
        return rec

    rec = run_one(main_name, args.steps, args.warmup, headline=True)
    results[main_name] = rec
    bwd = main_name.startswith("backward_")

    if not args.no_extras and not args.only:
        for name in ("gdn_bf16_b4h16_n8192_d128", "kath_bf16_b1h16_n32768_dk128_dv64",
                     "kath_f32_n256_d16", "kda_bf16_b4h16_n8192_d128",
                     "ssd_bf16_b2h32_n4096_dk128_dv64"):
            results[name] = run_one(name, max(20, args.steps // 8), 5)
        for name in ([] if args.no_varlen else W.VARLEN):
            results[name] = run_one(name, max(20, args.steps // 8), 5)
        for name in ("decode_gdn_256x32_d128", "decode_gla_256x32_d128", "decode_kda_256x32_d128",
                     "decode_ssd_256x64_dk128_dv64"):
            results[name] = run_one(name, 1000, 10)
        for name in ("gla_bf16_b2h8_n2048_d128", "ssd_bf16_b2h32_n4096_dk128_dv64",
                     "gdn_bf16_b4h16_n8192_d128", "kda_bf16_b4h16_n8192_d128",
                     "kath_bf16_b1h16_n32768_dk128_dv64"):
            results["backward_" + name] = run_one("backward_" + name, max(5, args.steps // 80), 2)
        for name in W.SELSCAN:
            results[name] = run_one(name, max(10, args.steps // 40), 3)

    scan = main_name.startswith("selscan")
    wl = W.SELSCAN[main_name] if scan else \
        W.WORKLOADS[main_name[len("backward_"):] if bwd else main_name]
    m = results[main_name]
    if bwd:   # every kernel of la_prefill_backward against the algorithmic bytes
        value, unit = m["Mtok_per_s"], "Mtok/s"
        roof = {"bound": "hbm", "achieved": m["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": m["hbm_frac"], "traffic": None, "kernel": "la_prefill_backward",
                "duration_us": m["ms"] * 1e3}
    elif scan:
        value, unit = m["Mtok_per_s"], "Mtok/s"
        roof = {"bound": "alu", "achieved": m["G_state_updates_per_s"],
                "peak": PEAK_SCAN_UPDATES / 1e9, "unit": "G state updates/s",
                "frac": m["alu_frac"], "traffic": load_traffic(main_name),
                "kernel": "selective_scan_kernel", "duration_us": m["ms"] * 1e3}
    elif main_name.startswith("decode"):
        value, unit = m["GB_per_s"], "GB/s"
        roof = {"bound": "hbm", "achieved": m["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": m["hbm_frac"], "traffic": load_traffic(main_name),
                "kernel": "decode_kernel", "duration_us": m["us_per_step"]}
    else:
        value, unit = m["Mtok_per_s"], "Mtok/s"
        roof = {"bound": "hbm", "achieved": m["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": m["hbm_frac"], "traffic": load_traffic(main_name),
                "kernel": STEP_KERNELS[wl.variant],
                "duration_us": m["ms"] * 1e3,
                "mfma": {"achieved": m["TFLOP_per_s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": m["mfma_frac"]}}
    cpu = m.get("cpu_oracle")
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": m["timed_calls"],
        "warmup": args.warmup, "ms_per_step": m["ms"], "ms_median": m["ms_median"],
        "ms_p10": m["ms_p10"], "ms_p90": m["ms_p90"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.io == "bf16" else "f32",
        "data": "synthetic",
        "config": ({"workload": main_name, "variant": "selective_scan", "Bt": wl.Bt, "T": wl.T,
                    "D": wl.D, "n": wl.n, "state": "fp32", "parallelism": "single GPU"} if scan else
                   {"workload": main_name, "variant": wl.variant, "B": wl.B, "H": wl.H, "N": wl.N,
                    "dk": wl.dk, "dv": wl.dv, "chunk": 64, "state": "fp32",
                    "parallelism": "single GPU"}),
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": m.get("parity"),
        "workloads": results,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
