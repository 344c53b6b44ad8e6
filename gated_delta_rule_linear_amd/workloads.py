"""Seeded synthetic inputs for the linear-attention recurrence.

This module holds input generation only: random draws, the gate
parameterisations that define the input distributions, per-token L2
normalisation of q and k where a workload asks for it, and rounding to the
storage dtype. It contains none of the recurrence's arithmetic, so both the
GPU path's tests and the oracle can take their inputs from here.

Recipe (every workload):
  * numpy ``default_rng(seed)`` (PCG64); arrays are drawn in C order, in the
    order q, k, v, then the gate pre-activations (u, then w for GDN), in fp64;
  * gate transforms and normalisation are done in fp64;
  * values are rounded fp64 -> fp32 (round to nearest even), then, for bf16
    storage, fp32 -> bf16 (round to nearest even on the fp32 bit pattern);
  * the fp64 copies handed to the oracle are the rounded values, exactly.

Gate parameterisations (input distributions, per workload):
  * GLA: g = exp(logsigmoid(u) / 16), u ~ N(0, 1) per (token, key dim)
    (forget gate per key dimension, "Linear / RNN 路线" section 2.2);
  * GDN: alpha = exp(-softplus(u)) = sigmoid(-u), beta = sigmoid(w), u, w ~
    N(0, 1) per (token, head) (scalar gates in (0, 1), "线性注意力与 SSM"
    section GDN);
  * KDA: a retention per (token, key channel) from the bounded log-decay of
    "状态空间与线性注意力" section KDA, alpha = exp(g_min sigmoid(e^A z)) with
    g_min = -5 and A = 0 (the page's own example), z ~ N(0, 1), so alpha lies
    in (e^-5, 1); beta = sigmoid(w), w ~ N(0, 1) per (token, head);
  * SSD (Mamba-2, one decay per token and head, "Linear / RNN 路线" sections 3.6
    and 4.1): a = exp(Delta A_h) with A_h = -(1 + h mod 16) (the page's A =
    -arange(1, ..) initialisation, one value per head) and Delta = softplus(u),
    u ~ N(-3, 1) per (token, head); q = C and k = B ~ N(0, 1/d_k), v = Delta x
    with x ~ N(0, 1) (the step scales the written input), so a lies in about
    (0.4, 1);
  * extra gate kinds for carry-sensitive tests: "slow" (alpha or g =
    exp(logsigmoid(u) / 16), about 0.95; KDA: exp(-5 sigmoid(z - 6)), about
    0.99), "ones" (g = 1 or alpha = 1), "beta0" (beta = 0), "beta1" (beta = 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (storage format: uint16 bit patterns)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to(x64: np.ndarray, dtype: str):
    """Round fp64 values to the storage dtype.

    Returns (stored, exact): ``stored`` is float32 or uint16 bf16 bits,
    ``exact`` the float64 value of what is stored.
    """
    f32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f32, f32.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(f32)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


def _logsigmoid(u):
    # stable: log(sigmoid(u)) = -log1p(exp(-u)) for u >= 0, u - log1p(exp(u)) for u < 0
    return np.where(u >= 0, -np.log1p(np.exp(-np.abs(u))), u - np.log1p(np.exp(-np.abs(u))))


def _sigmoid(u):
    return np.exp(_logsigmoid(u))


# ---------------------------------------------------------------------------
# Workload registry
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str            # "kath" | "gla" | "gdn" | "kda" | "ssd"
    B: int
    H: int
    N: int
    dk: int
    dv: int
    io: str                 # storage dtype of q, k, v, o: "f32" | "bf16"
    gate_io: str            # storage dtype of gates: "f32" | "bf16"
    seed: int
    eps: float = 1e-6
    qk_scale: float = 1.0   # q, k ~ N(0, qk_scale^2)
    v_scale: float = 1.0
    l2norm_qk: bool = False
    gate_kind: str = "default"
    decode: bool = False
    description: str = field(default="", compare=False)

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "kath_f32_n256_d16": Workload(
        "kath_f32_n256_d16", "kath", 1, 1, 256, 16, 16, "f32", "f32", seed=1,
        description="normalized ELU+1 linear attention, 1 head, N=256, d=16, fp32"),
    "gla_bf16_b2h8_n2048_d128": Workload(
        "gla_bf16_b2h8_n2048_d128", "gla", 2, 8, 2048, 128, 128, "bf16", "bf16", seed=2,
        qk_scale=1.0 / np.sqrt(128.0), v_scale=1.0 / np.sqrt(128.0),
        description="GLA per-key-dim gate forward, B=2 H=8 N=2048 d=128, bf16"),
    "kath_bf16_b1h16_n32768_dk128_dv64": Workload(
        "kath_bf16_b1h16_n32768_dk128_dv64", "kath", 1, 16, 32768, 128, 64, "bf16", "bf16",
        seed=3, description="normalized ELU+1 linear attention, B=1 H=16 N=32768 "
                            "dphi=128 dv=64, bf16"),
    "gdn_bf16_b4h16_n8192_d128": Workload(
        "gdn_bf16_b4h16_n8192_d128", "gdn", 4, 16, 8192, 128, 128, "bf16", "bf16", seed=4,
        l2norm_qk=True, description="Gated DeltaNet forward, B=4 H=16 N=8192 d=128, bf16, "
                                    "q/k L2-normalized"),
    "kda_bf16_b4h16_n8192_d128": Workload(
        "kda_bf16_b4h16_n8192_d128", "kda", 4, 16, 8192, 128, 128, "bf16", "bf16", seed=6,
        l2norm_qk=True, description="Kimi Delta Attention forward, B=4 H=16 N=8192 d=128, bf16, "
                                    "q/k L2-normalized, bounded per-channel retention"),
    "ssd_bf16_b2h32_n4096_dk128_dv64": Workload(
        "ssd_bf16_b2h32_n4096_dk128_dv64", "ssd", 2, 32, 4096, 128, 64, "bf16", "bf16", seed=8,
        qk_scale=1.0 / np.sqrt(128.0),
        description="Mamba-2 SSD forward (scalar decay per token and head), B=2 H=32 N=4096 "
                    "d_state=128 head dim 64, bf16"),
    "decode_gdn_256x32_d128": Workload(
        "decode_gdn_256x32_d128", "gdn", 256, 32, 1, 128, 128, "bf16", "bf16", seed=5,
        l2norm_qk=True, decode=True,
        description="GDN decode step, 256 sequences x 32 heads, d=128, fp32 state"),
    "decode_gla_256x32_d128": Workload(
        "decode_gla_256x32_d128", "gla", 256, 32, 1, 128, 128, "bf16", "bf16", seed=5,
        qk_scale=1.0 / np.sqrt(128.0), v_scale=1.0 / np.sqrt(128.0), decode=True,
        description="GLA decode step, 256 sequences x 32 heads, d=128, fp32 state"),
    "decode_kda_256x32_d128": Workload(
        "decode_kda_256x32_d128", "kda", 256, 32, 1, 128, 128, "bf16", "bf16", seed=7,
        l2norm_qk=True, decode=True,
        description="KDA decode step, 256 sequences x 32 heads, d=128, fp32 state"),
    "decode_ssd_256x64_dk128_dv64": Workload(
        "decode_ssd_256x64_dk128_dv64", "ssd", 256, 64, 1, 128, 64, "bf16", "bf16", seed=9,
        qk_scale=1.0 / np.sqrt(128.0), decode=True,
        description="SSD decode step, 256 sequences x 64 heads, d_state=128 head dim 64, "
                    "fp32 state"),
}

SSD_DT_MEAN = -3.0   # Delta = softplus(u), u ~ N(SSD_DT_MEAN, 1)

KDA_LOG_DECAY_MIN = -5.0   # g_min of the bounded log-decay

# Packed variable-length batches: a base workload (its H, d, dtypes and gate recipe),
# the number of sequences, and lengths drawn log-uniformly in [lo, hi] (seeded): a
# serving-like mix of short and long prompts.
VARLEN = {
    "gla_varlen_bf16_h8_d128": dict(base="gla_bf16_b2h8_n2048_d128", nseq=16, lo=64, hi=4096,
                                    seed=21),
    "gdn_varlen_bf16_h16_d128": dict(base="gdn_bf16_b4h16_n8192_d128", nseq=64, lo=256, hi=16384,
                                     seed=22),
}


def varlen_lengths(nseq: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths, log-uniform in [lo, hi] (int32)."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(np.log(lo), np.log(hi), nseq)).astype(np.int32)


def make_varlen_inputs(name: str):
    """(Workload of the packed layout [1, H, total, d], Inputs, cu_seqlens int32, lengths)."""
    spec = VARLEN[name]
    base = WORKLOADS[spec["base"]]
    lengths = varlen_lengths(spec["nseq"], spec["lo"], spec["hi"], spec["seed"])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    wl = base.with_(name=name, B=1, N=int(cu[-1]), seed=spec["seed"])
    return wl, make_inputs(wl), cu, lengths


DECODE_STATE_STD = 0.02   # decode state S ~ N(0, 0.02^2): std 0.02 (torch normal(mean, std))
DECODE_POOL = 8           # distinct token sets cycled through by repeated decode steps


@dataclass
class Inputs:
    """Device-format arrays plus their exact fp64 values.

    ``dev`` maps name -> float32 array or uint16 bf16 bits; ``exact`` maps name
    -> float64 copy of the same values. Names: q, k, v, and g (GLA gate or GDN
    alpha) and beta (GDN), S0 / z0 when present.
    """
    wl: Workload
    dev: dict
    exact: dict


def _draw_gates(rng, wl: Workload, shape_tok):
    """Draw gate pre-activations and transform them (fp64). Returns dict."""
    B, H, N = shape_tok
    out = {}
    kind = wl.gate_kind
    if wl.variant == "gla":
        u = rng.standard_normal((B, H, N, wl.dk))
        if kind in ("default", "slow"):
            g = np.exp(_logsigmoid(u) / 16.0)
        elif kind == "ones":
            g = np.ones_like(u)
        elif kind == "fast":
            g = _sigmoid(u + 1.0)          # strong forgetting, about 0.7 on average
        else:
            raise ValueError(kind)
        out["g"] = g
    elif wl.variant == "gdn":
        u = rng.standard_normal((B, H, N))
        w = rng.standard_normal((B, H, N))
        if kind == "default":
            alpha = _sigmoid(-u)                 # exp(-softplus(u))
            beta = _sigmoid(w)
        elif kind == "slow":
            alpha = np.exp(_logsigmoid(u) / 16.0)
            beta = _sigmoid(w)
        elif kind == "ones":                      # DeltaNet: no decay
            alpha = np.ones_like(u)
            beta = _sigmoid(w)
        elif kind == "beta0":                     # pure decay, no write
            alpha = np.exp(_logsigmoid(u) / 16.0)
            beta = np.zeros_like(w)
        elif kind == "beta1":
            alpha = _sigmoid(-u)
            beta = np.ones_like(w)
        else:
            raise ValueError(kind)
        out["g"] = alpha
        out["beta"] = beta
    elif wl.variant == "kda":
        z = rng.standard_normal((B, H, N, wl.dk))
        w = rng.standard_normal((B, H, N))
        beta = _sigmoid(w)
        if kind == "default":
            alpha = np.exp(KDA_LOG_DECAY_MIN * _sigmoid(z))
        elif kind == "slow":
            alpha = np.exp(KDA_LOG_DECAY_MIN * _sigmoid(z - 6.0))
        elif kind == "ones":
            alpha = np.ones_like(z)
        elif kind == "beta0":
            alpha = np.exp(KDA_LOG_DECAY_MIN * _sigmoid(z - 6.0))
            beta = np.zeros_like(w)
        elif kind == "beta1":
            alpha = np.exp(KDA_LOG_DECAY_MIN * _sigmoid(z))
            beta = np.ones_like(w)
        else:
            raise ValueError(kind)
        out["g"] = alpha
        out["beta"] = beta
    elif wl.variant == "ssd":
        u = rng.standard_normal((B, H, N)) + SSD_DT_MEAN
        delta = np.logaddexp(0.0, u)
        A_h = -(1.0 + (np.arange(H) % 16))[None, :, None]
        if kind == "default":
            a = np.exp(delta * A_h)
        elif kind == "slow":
            a = np.exp(delta * A_h / 16.0)
        elif kind == "ones":
            a = np.ones_like(delta)
        elif kind == "fast":
            a = np.exp(delta * A_h * 16.0)
        else:
            raise ValueError(kind)
        out["g"] = a
        out["_v_step"] = delta   # v = Delta x: the step scales the written input
    return out


def make_inputs(wl: Workload | str, *, with_state: bool = False, state_std: float = 0.5,
                seed: int | None = None, N: int | None = None) -> Inputs:
    """Generate one batch of seeded inputs for a prefill workload.

    ``with_state`` adds a nonzero initial state S0 (and z0 for KATH, drawn
    positive since z accumulates phi(k) > 0). ``seed`` / ``N`` override the
    workload's values.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if N is not None:
        wl = wl.with_(N=N)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, H, N, dk, dv = wl.B, wl.H, wl.N, wl.dk, wl.dv
    q = rng.standard_normal((B, H, N, dk)) * wl.qk_scale
    k = rng.standard_normal((B, H, N, dk)) * wl.qk_scale
    v = rng.standard_normal((B, H, N, dv)) * wl.v_scale
    if wl.l2norm_qk:
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    raw = {"q": q, "k": k, "v": v}
    gates = _draw_gates(rng, wl, (B, H, N))
    if "_v_step" in gates:
        raw["v"] = raw["v"] * gates.pop("_v_step")[..., None]
    dev, exact = {}, {}
    for name, arr in raw.items():
        dev[name], exact[name] = round_to(arr, wl.io)
    for name, arr in gates.items():
        dev[name], exact[name] = round_to(arr, wl.gate_io)
    if with_state:
        S0 = rng.standard_normal((B, H, dk, dv)) * state_std
        dev["S0"], exact["S0"] = round_to(S0, "f32")
        if wl.variant == "kath":
            z0 = np.abs(rng.standard_normal((B, H, dk))) * state_std * 4 + 0.5
            dev["z0"], exact["z0"] = round_to(z0, "f32")
    return Inputs(wl, dev, exact)


def make_decode_pool(wl: Workload | str, *, pool: int = DECODE_POOL, seed: int | None = None,
                     B: int | None = None, with_exact: bool = True):
    """Decode workload: initial state S ~ N(0, 0.02^2) fp32 and a pool of token sets.

    Token set j (q, k, v and gates, each [B, H, d] or [B, H]) is drawn like the
    matching prefill workload with N = 1. Step s of a repeated decode run uses
    token set s mod pool. Returns (S0_f32, S0_exact_or_None, [Inputs] * pool).
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if B is not None:
        wl = wl.with_(B=B)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    S = rng.standard_normal((wl.B, wl.H, wl.dk, wl.dv), dtype=np.float64) * DECODE_STATE_STD
    S32 = S.astype(np.float32)
    del S
    sets = []
    for j in range(pool):
        sub = make_inputs(wl.with_(N=1), seed=(wl.seed if seed is None else seed) * 1000 + 1 + j)
        dev = {k: (a.reshape(a.shape[:2] + a.shape[3:]) if a.ndim >= 3 else a)
               for k, a in sub.dev.items()}
        ex = {k: (a.reshape(a.shape[:2] + a.shape[3:]) if a.ndim >= 3 else a)
              for k, a in sub.exact.items()} if with_exact else {}
        sets.append(Inputs(wl, dev, ex))
    return S32, (S32.astype(np.float64) if with_exact else None), sets


def algorithmic_bytes_per_token_head(wl: Workload) -> int:
    """Bytes one pass must move at minimum: every input read once, every output written once.

    Prefill: q, k, v (+ gates) read, o written, in their storage dtypes.
    S_final (and z_final) are counted separately per sequence (see
    ``algorithmic_bytes``). Decode: the fp32 state read and written once per
    head plus the token's q, k, v, gates and o.
    """
    isz = 4 if wl.io == "f32" else 2
    gsz = 4 if wl.gate_io == "f32" else 2
    b = (2 * wl.dk + wl.dv) * isz + wl.dv * isz
    if wl.variant == "gla":
        b += wl.dk * gsz
    elif wl.variant == "gdn":
        b += 2 * gsz
    elif wl.variant == "kda":
        b += wl.dk * gsz + gsz
    elif wl.variant == "ssd":
        b += gsz
    return b


def algorithmic_bytes(wl: Workload) -> int:
    per = algorithmic_bytes_per_token_head(wl)
    seqs = wl.B * wl.H
    if wl.decode:
        state = wl.dk * wl.dv * 4 * 2 + (wl.dk * 4 * 2 if wl.variant == "kath" else 0)
        return seqs * (per + state)
    state_out = wl.dk * wl.dv * 4 + (wl.dk * 4 if wl.variant == "kath" else 0)
    return wl.token_heads * per + seqs * state_out


def algorithmic_flops(wl: Workload, chunk: int = 64) -> int:
    """Flops of the chunked method with full C x C tiles (C = chunk), per pass.

    Per token-head: 2*C*d per C x C contraction and 2*dk*dv per state
    contraction. KATH/GLA: Q K^T (2*C*dk), P V (2*C*dv), Q S and K^T V
    (2 x 2*dk*dv); KATH adds the normaliser column (2*C + 2*dk for P 1, phi(q) z,
    and dk for z += phi(k)). GDN: K K^T, Q K^T (2 x 2*C*dk), T (beta gamma K)
    (2*C*dk), T (beta V) and P U (2 x 2*C*dv), Q S, W S and K^T U
    (3 x 2*dk*dv) and the triangular inverse (C^2/3 per token). KDA counts as GDN
    (its decay sits inside the same products).
    Decode: 2*dk*dv per state read or write product (GLA 5, GDN 7, KATH 4 dk*dv).
    """
    dk, dv, C = wl.dk, wl.dv, chunk
    if wl.decode:
        per = {"gla": 5, "gdn": 7, "kda": 7, "kath": 4, "ssd": 5}[wl.variant] * dk * dv
        return wl.B * wl.H * per
    if wl.variant in ("gla", "ssd"):
        per = 2 * C * dk + 2 * C * dv + 4 * dk * dv
    elif wl.variant == "kath":
        per = 2 * C * dk + 2 * C * (dv + 1) + 4 * dk * dv + 3 * dk
    else:
        per = 6 * C * dk + 4 * C * dv + 6 * dk * dv + (C * C) // 3
    return wl.token_heads * per


# ---------------------------------------------------------------------------
# Selective scan (Mamba-1)
# ---------------------------------------------------------------------------
# Recipe ("Linear / RNN 路线" section 3.6, the simplified block's parameters):
#   * A = -arange(1, n + 1) for every channel (the block's initialisation, fp32);
#   * dt ~ N(0, 0.5^2) per (token, channel) and dt_bias ~ U(-1, 1) per channel, the
#     step being Delta = softplus(dt + dt_bias) inside the scan (the block's dt_proj
#     output with its bias split off);
#   * B, C ~ N(0, 1) per (token, state entry), x ~ N(0, 1) per (token, channel);
#   * D = 1 per channel (the skip at its usual initialisation);
#   * drawn in the order dt, dt_bias, B, C, x (then h0 ~ N(0, 0.5^2) when asked for),
#     rounded like the other inputs: dt, B, C, x to the storage dtype, A, D, dt_bias
#     and h0 to fp32.


@dataclass(frozen=True)
class SelScan:
    name: str
    Bt: int       # batch rows
    T: int        # tokens per row
    D: int        # channels (the block's inner width)
    n: int        # state entries per channel
    io: str       # storage dtype of dt, B, C, x, y
    seed: int
    description: str = field(default="", compare=False)

    def with_(self, **kw) -> "SelScan":
        return replace(self, **kw)


SELSCAN = {
    "selscan_bf16_b2_t4096_d2048_n128": SelScan(
        "selscan_bf16_b2_t4096_d2048_n128", 2, 4096, 2048, 128, "bf16", seed=11,
        description="Mamba-1 selective scan, 2 rows x 4096 tokens, 2048 channels, "
                    "128 state entries per channel, bf16 inputs, fp32 state"),
    "selscan_bf16_b2_t4096_d2048_n16": SelScan(
        "selscan_bf16_b2_t4096_d2048_n16", 2, 4096, 2048, 16, "bf16", seed=12,
        description="Mamba-1 selective scan with 16 state entries per channel"),
}


def make_selscan_inputs(wl: SelScan | str, *, with_state: bool = False, seed: int | None = None,
                        T: int | None = None):
    """(dev, exact) dicts for a selective-scan workload: dt, dt_bias, A, Bm, Cm, x, Dskip
    (and h0). ``dev`` holds the stored arrays (bf16 bits or fp32), ``exact`` their fp64
    values."""
    if isinstance(wl, str):
        wl = SELSCAN[wl]
    if T is not None:
        wl = wl.with_(T=T)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    Bt, T, D, n = wl.Bt, wl.T, wl.D, wl.n
    raw_io = {"dt": rng.normal(0.0, 0.5, (Bt, T, D))}
    raw_f32 = {"dt_bias": rng.uniform(-1.0, 1.0, D)}
    raw_io["Bm"] = rng.standard_normal((Bt, T, n))
    raw_io["Cm"] = rng.standard_normal((Bt, T, n))
    raw_io["x"] = rng.standard_normal((Bt, T, D))
    raw_f32["A"] = -np.broadcast_to(np.arange(1.0, n + 1.0), (D, n)).copy()
    raw_f32["Dskip"] = np.ones(D)
    if with_state:
        raw_f32["h0"] = rng.normal(0.0, 0.5, (Bt, D, n))
    dev, exact = {}, {}
    for k_, a in raw_io.items():
        dev[k_], exact[k_] = round_to(a, wl.io)
    for k_, a in raw_f32.items():
        dev[k_], exact[k_] = round_to(a, "f32")
    return dev, exact


def selscan_algorithmic_bytes(wl: SelScan) -> int:
    """Minimum bytes of one scan: dt, x read and y written per (token, channel), B and C
    per (token, state entry), A, D and dt_bias once, the final state written once."""
    isz = 4 if wl.io == "f32" else 2
    return (wl.Bt * wl.T * (3 * wl.D + 2 * wl.n) * isz + wl.D * (wl.n + 2) * 4
            + wl.Bt * wl.D * wl.n * 4)
