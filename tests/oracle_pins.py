"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle library at
``lib`` (a path, or None for the built one) disagrees with a fact that does
not come from the oracle itself:

  * explicit masked quadratic (semiseparable) forms built without any
    recurrence ("状态空间与线性注意力", section State Space Duality, the
    matrix M_{j,i} = C_j^T A_j ... A_{i+1} B_i; and the validation matrix's
    "explicit lower-triangular matrix" row);
  * split / carry invariance ("状态空间与线性注意力", minimal semantic
    implementation: split anywhere, carry the state, equal the whole scan);
  * the gated delta rule written in its value-major matrix form
    ("线性注意力与 SSM", section GDN) and the KDA recurrence with a broadcast
    gate ("状态空间与线性注意力", section KDA); KDA's expanded transition
    (I - b k k^T) Diag(a), its reduction to the gated delta rule, and its
    per-channel closed form;
  * the worked delta-rule example (golden fixture);
  * the single-head hand count (golden fixture);
  * closed forms for constant inputs; special cases that reduce to known
    forms (plain causal linear attention, RetNet's decayed parallel form,
    DeltaNet, pure decay); causality; linearity in V.

The functions are shared by ``test_oracle_pins.py`` (against the built
oracle) and the mutation tests (against deliberately broken copies of the
oracle source, which must fail at least one pin).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def phi_lib(x: np.ndarray) -> np.ndarray:
    """ELU (alpha = 1) plus one, from torch's ELU in float64."""
    return (torch.nn.functional.elu(torch.from_numpy(np.asarray(x, np.float64))) + 1.0).numpy()


def rand_case(variant, B=1, H=2, N=12, dk=5, dv=4, seed=0, with_state=True, unit_keys=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = beta = None
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    if variant == "gla":
        g = rng.uniform(0.5, 1.0, (B, H, N, dk))
    elif variant == "gdn":
        g = rng.uniform(0.5, 1.0, (B, H, N))
        beta = rng.uniform(0.05, 0.95, (B, H, N))
    elif variant == "kda":
        g = rng.uniform(0.5, 1.0, (B, H, N, dk))
        beta = rng.uniform(0.05, 0.95, (B, H, N))
    elif variant == "ssd":
        g = rng.uniform(0.5, 1.0, (B, H, N))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.7 if with_state else None
    z0 = (rng.uniform(0.5, 2.0, (B, H, dk)) if (with_state and variant == "kath") else None)
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, z0=z0)


def run(variant, case, lib=None, eps=1e-6, **kw):
    return oracle.prefill(variant, case["q"], case["k"], case["v"], case["g"], case["beta"],
                          case["S0"], case["z0"], eps=eps, lib_path=lib, **kw)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# explicit quadratic forms (no recurrence), one head at a time
# ---------------------------------------------------------------------------

def quad_kath(q, k, v, S0, z0, eps):
    T = q.shape[0]
    fq, fk = phi_lib(q), phi_lib(k)
    A = np.tril(fq @ fk.T)
    num = A @ v + fq @ S0
    den = A @ np.ones(T) + fq @ z0 + eps
    O = num / den[:, None]
    return O, S0 + fk.T @ v, z0 + fk.sum(axis=0)


def quad_gla(q, k, v, g, S0):
    T, dk = q.shape
    M = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            w = np.prod(g[s + 1:t + 1], axis=0) if t > s else np.ones(dk)
            M[t, s] = np.sum(q[t] * k[s] * w)
    pref = np.array([np.prod(g[:t + 1], axis=0) for t in range(T)])  # prod_{r<=t} g_r
    O = M @ v + (q * pref) @ S0
    S = pref[-1][:, None] * S0
    for s in range(T):
        w = np.prod(g[s + 1:], axis=0) if s < T - 1 else np.ones(dk)
        S = S + np.outer(w * k[s], v[s])
    return O, S


def quad_gdn(q, k, v, alpha, beta, S0):
    """Key-major state; F_t = alpha_t (I - beta_t k_t k_t^T), later factors on the left."""
    T, dk = q.shape
    I = np.eye(dk)
    F = [alpha[t] * (I - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    return _quad_delta(q, k, v, beta, S0, F)


def quad_kda(q, k, v, alpha, beta, S0):
    """KDA's expanded transition F_t = (I - beta_t k_t k_t^T) Diag(alpha_t) ("状态空间与线性
    注意力", section KDA, the second form), later factors on the left."""
    T, dk = q.shape
    I = np.eye(dk)
    F = [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t]) for t in range(T)]
    return _quad_delta(q, k, v, beta, S0, F)


def _quad_delta(q, k, v, beta, S0, F):
    """S_t = F_t S_{t-1} + beta_t k_t v_t^T unrolled into products of the F's."""
    T, dk = q.shape
    I = np.eye(dk)

    def chain(t, s):  # F_t F_{t-1} ... F_{s+1}   (identity when t == s)
        P = I.copy()
        for r in range(s + 1, t + 1):
            P = F[r] @ P
        return P

    M = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            M[t, s] = beta[s] * q[t] @ chain(t, s) @ k[s]
    O = M @ v + np.array([q[t] @ (chain(t, -1) @ S0) for t in range(T)])
    S = chain(T - 1, -1) @ S0
    for s in range(T):
        S = S + chain(T - 1, s) @ np.outer(beta[s] * k[s], v[s])
    return O, S


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_quadratic_form(lib=None):
    for variant, dk, dv in (("kath", 5, 3), ("gla", 5, 3), ("gdn", 4, 6), ("gdn", 6, 4),
                            ("kda", 5, 3), ("kda", 3, 6), ("ssd", 5, 3)):
        case = rand_case(variant, B=2, H=1, N=11, dk=dk, dv=dv, seed=7, with_state=True)
        eps = 0.3 if variant == "kath" else 1e-6
        o, S, z = run(variant, case, lib, eps=eps)
        for b in range(2):
            sl = (b, 0)
            if variant == "kath":
                O_ref, S_ref, z_ref = quad_kath(case["q"][sl], case["k"][sl], case["v"][sl],
                                                case["S0"][sl], case["z0"][sl], eps)
                assert rel(z[sl], z_ref) < 1e-12, "KATH z vs quadratic form"
            elif variant == "gla":
                O_ref, S_ref = quad_gla(case["q"][sl], case["k"][sl], case["v"][sl],
                                        case["g"][sl], case["S0"][sl])
            elif variant == "ssd":   # the semiseparable form with a scalar decay per token
                O_ref, S_ref = quad_gla(case["q"][sl], case["k"][sl], case["v"][sl],
                                        np.repeat(case["g"][sl][:, None], dk, axis=1),
                                        case["S0"][sl])
            elif variant == "gdn":
                O_ref, S_ref = quad_gdn(case["q"][sl], case["k"][sl], case["v"][sl],
                                        case["g"][sl], case["beta"][sl], case["S0"][sl])
            else:
                O_ref, S_ref = quad_kda(case["q"][sl], case["k"][sl], case["v"][sl],
                                        case["g"][sl], case["beta"][sl], case["S0"][sl])
            assert rel(o[sl], O_ref) < 1e-12, f"{variant} o vs quadratic form: {rel(o[sl], O_ref)}"
            assert rel(S[sl], S_ref) < 1e-12, f"{variant} S vs quadratic form"


def pin_split_invariance(lib=None):
    for variant in ("kath", "gla", "gdn", "kda", "ssd"):
        case = rand_case(variant, B=1, H=3, N=23, dk=6, dv=5, seed=11, with_state=True)
        o, S, z = run(variant, case, lib)
        for m in (1, 7, 16, 22):
            left = {kk: (vv[:, :, :m] if (vv is not None and kk in ("q", "k", "v", "g", "beta"))
                         else vv) for kk, vv in case.items()}
            oL, SL, zL = run(variant, left, lib)
            right = {kk: (vv[:, :, m:] if (vv is not None and kk in ("q", "k", "v", "g", "beta"))
                          else vv) for kk, vv in case.items()}
            right["S0"], right["z0"] = SL, zL
            oR, SR, zR = run(variant, right, lib)
            assert np.array_equal(np.concatenate([oL, oR], axis=2), o), f"{variant} split o m={m}"
            assert np.array_equal(SR, S), f"{variant} split S m={m}"
            if variant == "kath":
                assert np.array_equal(zR, z), f"{variant} split z m={m}"


def pin_gdn_page_forms(lib=None):
    """Value-major matrix form and the KDA recurrence with alpha broadcast, step by step."""
    case = rand_case("gdn", B=1, H=1, N=9, dk=5, dv=3, seed=5, with_state=True, unit_keys=True)
    q, k, v = case["q"][0, 0], case["k"][0, 0], case["v"][0, 0]
    a, b = case["g"][0, 0], case["beta"][0, 0]
    o, S, _ = run("gdn", case, lib)
    Sv = case["S0"][0, 0].T.copy()          # value-major d_v x d_k
    Sk = case["S0"][0, 0].copy()            # key-major for the KDA form
    I = np.eye(5)
    for t in range(9):
        Sv = a[t] * Sv @ (I - b[t] * np.outer(k[t], k[t])) + b[t] * np.outer(v[t], k[t])
        Sbar = (a[t] * np.ones(5))[:, None] * Sk
        Sk = Sbar + b[t] * np.outer(k[t], v[t] - k[t] @ Sbar)
        assert rel(o[0, 0, t], Sv @ q[t]) < 1e-12, "GDN o vs value-major form"
        assert rel(o[0, 0, t], Sk.T @ q[t]) < 1e-12, "GDN o vs KDA form"
    assert rel(S[0, 0], Sv.T) < 1e-12 and rel(S[0, 0], Sk) < 1e-12


def pin_kda_forms(lib=None):
    """KDA: decay-then-correct and the expanded (I - b k k^T) Diag(a) S + b k v^T form agree
    with the oracle at every step; with the retention broadcast over the key channels KDA
    is the gated delta rule (pinned on its own above); a channel the keys never touch
    only decays."""
    case = rand_case("kda", B=1, H=1, N=9, dk=5, dv=3, seed=15, with_state=True, unit_keys=True)
    q, k, v = case["q"][0, 0], case["k"][0, 0], case["v"][0, 0]
    a, b = case["g"][0, 0], case["beta"][0, 0]
    o, S, _ = run("kda", case, lib)
    Sx = case["S0"][0, 0].copy()
    I = np.eye(5)
    for t in range(9):
        Sx = (I - b[t] * np.outer(k[t], k[t])) @ np.diag(a[t]) @ Sx + b[t] * np.outer(k[t], v[t])
        assert rel(o[0, 0, t], Sx.T @ q[t]) < 1e-12, "KDA o vs expanded form"
    assert rel(S[0, 0], Sx) < 1e-12
    # broadcast retention: equal to GDN with the scalar alpha
    g_case = rand_case("gdn", B=1, H=2, N=12, dk=4, dv=3, seed=16, with_state=True)
    k_case = dict(g_case)
    k_case["g"] = np.repeat(g_case["g"][..., None], 4, axis=-1)
    og, Sg, _ = run("gdn", g_case, lib)
    ok, Sk, _ = run("kda", k_case, lib)
    assert rel(ok, og) < 1e-12 and rel(Sk, Sg) < 1e-12, "KDA with broadcast retention vs GDN"
    # keys confined to channels 0..2: rows 3, 4 of S0 decay by the product of their
    # retentions and never mix with the others
    case = rand_case("kda", B=1, H=1, N=10, dk=5, dv=3, seed=18, with_state=True)
    case["k"][..., 3:] = 0.0
    o, S, _ = run("kda", case, lib)
    pref = np.prod(case["g"][0, 0], axis=0)
    assert rel(S[0, 0, 3:], pref[3:, None] * case["S0"][0, 0, 3:]) < 1e-13, "KDA idle channels"


def pin_delta_identity(lib=None):
    """S_t - a_t S_{t-1} = b_t k_t (v_t - a_t S_{t-1}^T k_t)^T at every step (decode steps)."""
    case = rand_case("gdn", B=1, H=2, N=8, dk=4, dv=3, seed=9, with_state=True)
    S = case["S0"].copy()
    for t in range(8):
        prev = S.copy()
        oracle.decode_step("gdn", case["q"][:, :, t], case["k"][:, :, t], case["v"][:, :, t], S,
                           g=case["g"][:, :, t], beta=case["beta"][:, :, t], lib_path=lib)
        for h in range(2):
            kk, vv = case["k"][0, h, t], case["v"][0, h, t]
            a, b = case["g"][0, h, t], case["beta"][0, h, t]
            lhs = S[0, h] - a * prev[0, h]
            rhs = b * np.outer(kk, vv - a * prev[0, h].T @ kk)
            assert rel(lhs, rhs) < 1e-12, "delta-rule identity"


def pin_worked_example(lib=None):
    with open(os.path.join(GOLDEN, "delta_rule_worked_example.json")) as f:
        ex = json.load(f)
    keys = np.array(ex["keys"])
    values = np.array(ex["values"])
    beta = np.array(ex["beta"])
    T, dk = keys.shape
    dv = values.shape[1]
    sh = lambda a: a.reshape((1, 1) + a.shape)
    # GDN with alpha = 1 and beta = 1; queries = keys so the post-write read recalls the value
    o, S, _ = oracle.prefill("gdn", sh(keys), sh(keys), sh(values), sh(np.ones(T)), sh(beta),
                             lib_path=lib)
    assert np.array_equal(keys @ S[0, 0], np.array(ex["final_state_times_keys"])), "keys @ S"
    assert np.array_equal(o[0, 0], values), "post-write recall"
    # reads before each write: S_{t-1}^T k_t from the state after the prefix
    state = np.zeros((1, 1, dk, dv))
    reads = []
    for t in range(T):
        reads.append(state[0, 0].T @ keys[t])
        oracle.decode_step("gdn", sh(keys[t]), sh(keys[t]), sh(values[t]), state,
                           g=np.ones((1, 1)), beta=np.full((1, 1), beta[t]), lib_path=lib)
    assert np.array_equal(np.array(reads), np.array(ex["reads_before_write"]))


def pin_hand_count(lib=None):
    with open(os.path.join(GOLDEN, "hand_count_single_head.json")) as f:
        hc = json.load(f)
    N, dk, dv = hc["N"], hc["d_phi"], hc["d_v"]
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, N, dk)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((1, 1, N, dk)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((1, 1, N, dv)).astype(np.float32).astype(np.float64)
    o, S, z, c = oracle.prefill("kath", q, k, v, with_counts=True, lib_path=lib)
    assert S[0, 0].size == hc["state_elements"] and z[0, 0].size == hc["z_elements"]
    assert c.state_update_macs == hc["main_term_macs"], c
    assert c.state_read_macs == hc["main_term_macs"], c
    assert abs(c.state_update_macs - hc["main_term_macs_rounded"]) / hc["main_term_macs_rounded"] < 5e-4
    assert c.tokens == N and c.norm_update_adds == N * dk and c.norm_read_macs == N * dk
    assert N * N == hc["full_attention_scores"]


def pin_closed_forms(lib=None):
    T, eps = 40, 0.25
    # KATH, constant tokens: S_t = t phi(k) v^T, z_t = t phi(k), o_t = v * t a / (t a + eps)
    qv = np.array([-1.0, 0.0, 0.5, 2.0, -0.3])
    kv = np.array([0.7, -2.0, 0.0, 1.5, -0.1])
    vv = np.array([1.0, -2.0, 0.5])
    fq = np.array([np.exp(-1.0), 1.0, 1.5, 3.0, np.exp(-0.3)])      # ELU(x)+1 by its definition
    fk = np.array([1.7, np.exp(-2.0), 1.0, 2.5, np.exp(-0.1)])
    assert rel(phi_lib(qv), fq) < 1e-15 and rel(phi_lib(kv), fk) < 1e-15
    tile = lambda x: np.broadcast_to(x, (1, 1, T, x.size)).copy()
    o, S, z = oracle.prefill("kath", tile(qv), tile(kv), tile(vv), eps=eps, lib_path=lib)
    a = fq @ fk
    t = np.arange(1, T + 1)[:, None]
    assert rel(o[0, 0], vv[None, :] * (t * a) / (t * a + eps)) < 1e-13, "KATH closed form"
    assert rel(S[0, 0], T * np.outer(fk, vv)) < 1e-13 and rel(z[0, 0], T * fk) < 1e-13
    # GLA, constant tokens and gate: S_t = diag((1 - g^t) / (1 - g)) k v^T
    gv = np.array([0.9, 0.5, 0.99, 0.7, 0.3])
    o, S, _ = oracle.prefill("gla", tile(qv), tile(kv), tile(vv), g=tile(gv), lib_path=lib)
    for tt in (1, 2, 17, T):
        St = np.outer((1 - gv ** tt) / (1 - gv) * kv, vv)
        assert rel(o[0, 0, tt - 1], St.T @ qv) < 1e-13, "GLA closed form o"
    assert rel(S[0, 0], np.outer((1 - gv ** T) / (1 - gv) * kv, vv)) < 1e-13
    # GDN, constant tokens with |k| = 1: S_t = k p_t^T, p_t = beta v (1 - rho^t) / (1 - rho)
    ku = kv / np.linalg.norm(kv)
    al, be = 0.8, 0.6
    rho = al * (1 - be)
    o, S, _ = oracle.prefill("gdn", tile(qv), tile(ku), tile(vv), g=np.full((1, 1, T), al),
                             beta=np.full((1, 1, T), be), lib_path=lib)
    for tt in (1, 2, 9, T):
        p = be * vv * (1 - rho ** tt) / (1 - rho)
        assert rel(o[0, 0, tt - 1], (ku @ qv) * p) < 1e-13, "GDN closed form o"
    assert rel(S[0, 0], np.outer(ku, be * vv * (1 - rho ** T) / (1 - rho))) < 1e-13
    # KDA, constant tokens with k = e_0 and a constant retention per channel: row 0 of the
    # state follows r_t = rho r_{t-1} + beta v with rho = a_0 (1 - beta); the other rows
    # only decay, row i by a_i^t
    e0 = np.array([1.0, 0.0, 0.0, 0.0, 0.0])
    av = np.array([0.9, 0.5, 0.99, 0.7, 0.3])
    be = 0.35
    rho = av[0] * (1 - be)
    S0 = np.arange(15, dtype=np.float64).reshape(1, 1, 5, 3) / 7.0 - 1.0
    o, S, _ = oracle.prefill("kda", tile(qv), tile(e0), tile(vv), g=tile(av),
                             beta=np.full((1, 1, T), be), S0=S0, lib_path=lib)
    for tt in (1, 2, 9, T):
        St = (av[:, None] ** tt) * S0[0, 0]
        St[0] = rho ** tt * S0[0, 0, 0] + be * vv * (1 - rho ** tt) / (1 - rho)
        assert rel(o[0, 0, tt - 1], St.T @ qv) < 1e-13, "KDA closed form o"
    assert rel(S[0, 0], St) < 1e-13


def pin_special_cases(lib=None):
    # GDN beta = 0: pure decay of S0
    case = rand_case("gdn", B=1, H=2, N=10, dk=4, dv=3, seed=3, with_state=True)
    case["beta"] = np.zeros_like(case["beta"])
    o, S, _ = run("gdn", case, lib)
    pref = np.cumprod(case["g"], axis=2)
    for h in range(2):
        for t in range(10):
            ref = pref[0, h, t] * case["S0"][0, h].T @ case["q"][0, h, t]
            assert rel(o[0, h, t], ref) < 1e-13, "GDN beta=0"
        assert rel(S[0, h], pref[0, h, -1] * case["S0"][0, h]) < 1e-13
    # GDN alpha = 1: DeltaNet, S_t = S_{t-1} + beta k (v - S_{t-1}^T k)^T
    case = rand_case("gdn", B=1, H=1, N=10, dk=4, dv=3, seed=4, with_state=True)
    case["g"] = np.ones_like(case["g"])
    o, S, _ = run("gdn", case, lib)
    St = case["S0"][0, 0].copy()
    for t in range(10):
        kk = case["k"][0, 0, t]
        St = St + case["beta"][0, 0, t] * np.outer(kk, case["v"][0, 0, t] - St.T @ kk)
        assert rel(o[0, 0, t], St.T @ case["q"][0, 0, t]) < 1e-12, "DeltaNet"
    # GLA g = 1: plain causal linear attention, O = tril(Q K^T) V + Q S0
    case = rand_case("gla", B=1, H=1, N=13, dk=5, dv=4, seed=5, with_state=True)
    case["g"] = np.ones_like(case["g"])
    o, S, _ = run("gla", case, lib)
    Q, K, V = case["q"][0, 0], case["k"][0, 0], case["v"][0, 0]
    assert rel(o[0, 0], np.tril(Q @ K.T) @ V + Q @ case["S0"][0, 0]) < 1e-12, "GLA g=1"
    assert rel(S[0, 0], case["S0"][0, 0] + K.T @ V) < 1e-12
    # GLA with one scalar gate for all key dims: RetNet parallel form with D_ts = gamma^(t-s)
    case = rand_case("gla", B=1, H=1, N=13, dk=5, dv=4, seed=6, with_state=False)
    gam = 0.83
    case["g"] = np.full_like(case["g"], gam)
    o, S, _ = run("gla", case, lib)
    Q, K, V = case["q"][0, 0], case["k"][0, 0], case["v"][0, 0]
    tt = np.arange(13)
    D = np.where(tt[:, None] >= tt[None, :], gam ** (tt[:, None] - tt[None, :]).clip(0), 0.0)
    assert rel(o[0, 0], ((Q @ K.T) * D) @ V) < 1e-12, "RetNet form"
    # SSD with a constant decay: the same parallel form (Mamba-2's 1-semiseparable mask)
    case = rand_case("ssd", B=1, H=1, N=13, dk=5, dv=4, seed=6, with_state=False)
    case["g"] = np.full_like(case["g"], gam)
    o, S, _ = run("ssd", case, lib)
    assert rel(o[0, 0], ((Q @ K.T) * D) @ V) < 1e-12, "SSD constant decay vs RetNet form"
    # SSD with its decay broadcast over the key dims is GLA, operation for operation
    case = rand_case("ssd", B=1, H=2, N=17, dk=4, dv=3, seed=23, with_state=True)
    o, S, _ = run("ssd", case, lib)
    g_case = dict(case)
    g_case["g"] = np.repeat(case["g"][..., None], 4, axis=-1)
    og, Sg, _ = run("gla", g_case, lib)
    assert np.array_equal(o, og) and np.array_equal(S, Sg), "SSD vs GLA with a broadcast gate"
    # KDA beta = 0: every channel of S0 decays by its own retention, nothing is written
    case = rand_case("kda", B=1, H=2, N=10, dk=4, dv=3, seed=19, with_state=True)
    case["beta"] = np.zeros_like(case["beta"])
    o, S, _ = run("kda", case, lib)
    pref = np.cumprod(case["g"], axis=2)
    for h in range(2):
        for t in range(10):
            ref = (pref[0, h, t][:, None] * case["S0"][0, h]).T @ case["q"][0, h, t]
            assert rel(o[0, h, t], ref) < 1e-13, "KDA beta=0"
    # KDA retention 1: DeltaNet
    case = rand_case("kda", B=1, H=1, N=10, dk=4, dv=3, seed=20, with_state=True)
    case["g"] = np.ones_like(case["g"])
    o, S, _ = run("kda", case, lib)
    St = case["S0"][0, 0].copy()
    for t in range(10):
        kk = case["k"][0, 0, t]
        St = St + case["beta"][0, 0, t] * np.outer(kk, case["v"][0, 0, t] - St.T @ kk)
        assert rel(o[0, 0, t], St.T @ case["q"][0, 0, t]) < 1e-12, "KDA retention 1 (DeltaNet)"


def pin_causality(lib=None):
    for variant in ("kath", "gla", "gdn", "kda", "ssd"):
        case = rand_case(variant, B=1, H=2, N=16, dk=4, dv=3, seed=13, with_state=True)
        o, _, _ = run(variant, case, lib)
        for tp in (0, 5, 15):
            c2 = {kk: (None if vv is None else vv.copy()) for kk, vv in case.items()}
            c2["q"][:, :, tp] += 1.5
            c2["k"][:, :, tp] -= 0.75
            c2["v"][:, :, tp] *= -3.0
            if c2["g"] is not None:
                c2["g"][:, :, tp] *= 0.5
            o2, _, _ = run(variant, c2, lib)
            assert np.array_equal(o2[:, :, :tp], o[:, :, :tp]), f"{variant} causality t'={tp}"
            assert not np.array_equal(o2[:, :, tp], o[:, :, tp])


def pin_linearity(lib=None):
    for variant in ("gla", "gdn", "kda", "ssd"):
        case = rand_case(variant, B=1, H=2, N=14, dk=5, dv=4, seed=17, with_state=False)
        rng = np.random.default_rng(1)
        v1, v2 = rng.standard_normal(case["v"].shape), rng.standard_normal(case["v"].shape)
        a, b = 1.7, -0.4
        outs = []
        for vv in (v1, v2, a * v1 + b * v2):
            c2 = dict(case)
            c2["v"] = vv
            outs.append(run(variant, c2, lib))
        assert rel(outs[2][0], a * outs[0][0] + b * outs[1][0]) < 1e-12, f"{variant} linear in V"
        assert rel(outs[2][1], a * outs[0][1] + b * outs[1][1]) < 1e-12


def pin_decode_matches_prefill(lib=None):
    for variant in ("kath", "gla", "gdn", "kda", "ssd"):
        case = rand_case(variant, B=2, H=2, N=6, dk=4, dv=3, seed=21, with_state=True)
        o, S, z = run(variant, case, lib)
        St = case["S0"].copy()
        zt = case["z0"].copy() if variant == "kath" else None
        for t in range(6):
            ot = oracle.decode_step(
                variant, case["q"][:, :, t], case["k"][:, :, t], case["v"][:, :, t], St,
                g=None if case["g"] is None else case["g"][:, :, t],
                beta=None if case["beta"] is None else case["beta"][:, :, t], z=zt, lib_path=lib)
            assert np.array_equal(ot, o[:, :, t]), f"{variant} decode step {t}"
        assert np.array_equal(St, S)
        if variant == "kath":
            assert np.array_equal(zt, z)


def pin_ssd_selective_ssm(lib=None):
    """SSD against the selective state space model it is ("Linear / RNN 路线", sections 3.6 and
    4.1; "状态空间与线性注意力", the Mamba section): every channel p of the head input x runs its
    own diagonal SSM with state h_p in R^n, h_p <- exp(dt*A) h_p + dt * B x_p, y_p = C . h_p,
    with one scalar A per head (Mamba-2).  Written here as P independent scalar-input recurrences,
    it must equal the oracle's SSD with q = C, k = B, v = dt*x and decay exp(dt*A): this fixes
    which axis of S is the state and which is the channel, and that the output reads S after
    the write."""
    rng = np.random.default_rng(41)
    T, n, P = 19, 6, 3
    A = -rng.uniform(1.0, 4.0)
    dt = np.log1p(np.exp(rng.normal(-1.0, 1.0, T)))           # softplus, positive steps
    Bm, Cm, x = rng.normal(size=(T, n)), rng.normal(size=(T, n)), rng.normal(size=(T, P))
    h0 = rng.normal(size=(P, n))
    y, h_end = np.zeros((T, P)), np.zeros((P, n))
    for p in range(P):                                          # one scalar-input SSM per channel
        h = h0[p].copy()
        for t in range(T):
            h = np.exp(dt[t] * A) * h + dt[t] * Bm[t] * x[t, p]
            y[t, p] = Cm[t] @ h
        h_end[p] = h
    case = {"q": Cm[None, None], "k": Bm[None, None], "v": (dt[:, None] * x)[None, None],
            "g": np.exp(dt * A)[None, None], "beta": None, "S0": h0.T[None, None].copy(),
            "z0": None}
    o, S, _ = run("ssd", case, lib)
    assert rel(o[0, 0], y) < 1e-12, "SSD output vs per-channel selective SSM"
    assert rel(S[0, 0], h_end.T) < 1e-12, "SSD state vs per-channel selective SSM"


# ---------------------------------------------------------------------------
# Selective scan (Mamba-1)
# ---------------------------------------------------------------------------

def ss_case(Bt=2, T=11, D=3, n=4, seed=0, with_state=True, softplus=True):
    """Random selective-scan inputs: A < 0 per (channel, state), raw steps around softplus(-1)."""
    rng = np.random.default_rng(seed)
    return dict(dt=rng.normal(-1.0, 1.0, (Bt, T, D)),
                A=-rng.uniform(0.5, 4.0, (D, n)),
                Bm=rng.standard_normal((Bt, T, n)), Cm=rng.standard_normal((Bt, T, n)),
                x=rng.standard_normal((Bt, T, D)), Dskip=rng.standard_normal(D),
                dt_bias=rng.normal(0.0, 0.5, D), dt_softplus=softplus,
                h0=rng.standard_normal((Bt, D, n)) if with_state else None)


def ss_run(case, lib=None, **over):
    c = dict(case, **over)
    return oracle.selective_scan(c["dt"], c["A"], c["Bm"], c["Cm"], c["x"], c["Dskip"],
                                 c["dt_bias"], c["dt_softplus"], c["h0"], lib_path=lib)


def _softplus(u):
    return np.logaddexp(0.0, u)


def pin_selective_scan_unrolled(lib=None):
    """The selective scan against its unrolled sum ("Linear / RNN 路线" section 4.1, with the
    discretisation of section 3.5): h_t = (prod_{0<i<=t} Abar_i) h_0
    + sum_{tau<=t} (prod_{tau<i<=t} Abar_i) Bbar_tau x_tau, per channel and state entry, with
    Abar = exp(Delta A), Bbar = Delta B and Delta = softplus(dt + bias); y_t = C_t . h_t + D x_t
    ("状态空间与线性注意力", section 卷积与递推的等价, for the skip). Every token has its own step."""
    case = ss_case(Bt=2, T=9, D=3, n=4, seed=31)
    y, hT = ss_run(case, lib)
    Bt, T, D = case["x"].shape
    n = case["A"].shape[1]
    delta = _softplus(case["dt"] + case["dt_bias"])                       # [Bt,T,D]
    for b in range(Bt):
        for d in range(D):
            abar = np.exp(delta[b, :, d, None] * case["A"][d][None, :])    # [T,n]
            bbar = delta[b, :, d, None] * case["Bm"][b]                    # [T,n]
            for t in range(T):
                h = np.prod(abar[:t + 1], axis=0) * case["h0"][b, d]
                for tau in range(t + 1):
                    h = h + np.prod(abar[tau + 1:t + 1], axis=0) * bbar[tau] * case["x"][b, tau, d]
                want = case["Cm"][b, t] @ h + case["Dskip"][d] * case["x"][b, t, d]
                assert abs(y[b, t, d] - want) <= 1e-12 * (1 + abs(want)), "unrolled output"
            assert rel(hT[b, d], h) < 1e-12, "unrolled final state"
    # without softplus the step is the raw value itself, bias included
    case["dt"] = np.abs(case["dt"])
    case["dt_bias"] = np.zeros(D)
    y1, _ = ss_run(case, lib, dt_softplus=False)
    y2, _ = ss_run(case, lib, dt=np.log(np.expm1(case["dt"])), dt_softplus=True)
    assert rel(y1, y2) < 1e-10, "softplus off: the raw step is Delta"


def pin_selective_scan_convolution(lib=None):
    """Time-invariant parameters turn the scan into a causal convolution ("状态空间与线性注意力",
    section 卷积与递推的等价): with one Delta, B, C for all tokens, y_t = sum_{i<=t} K_{t-i} x_i
    + D x_t with the kernel K_j = C . (Abar^j Bbar) per channel."""
    rng = np.random.default_rng(32)
    Bt, T, D, n = 1, 15, 3, 5
    A = -rng.uniform(0.2, 2.0, (D, n))
    delta = rng.uniform(0.05, 0.6, D)
    Bv, Cv = rng.standard_normal(n), rng.standard_normal(n)
    x = rng.standard_normal((Bt, T, D))
    Dskip = rng.standard_normal(D)
    y, _ = oracle.selective_scan(np.broadcast_to(delta, (Bt, T, D)), A,
                                 np.broadcast_to(Bv, (Bt, T, n)), np.broadcast_to(Cv, (Bt, T, n)),
                                 x, Dskip, None, False, None, lib_path=lib)
    for d in range(D):
        abar, bbar = np.exp(delta[d] * A[d]), delta[d] * Bv
        K = np.array([Cv @ (abar ** j * bbar) for j in range(T)])
        want = np.convolve(x[0, :, d], K)[:T] + Dskip[d] * x[0, :, d]
        assert rel(y[0, :, d], want) < 1e-12, "convolution form"


def pin_selective_scan_split(lib=None):
    """Split anywhere, carry the state, and the pieces equal the whole scan ("状态空间与线性注意力",
    the split check under its minimal selective_scan): bit for bit, at every split point."""
    case = ss_case(Bt=2, T=7, D=4, n=4, seed=0)
    y, hT = ss_run(case, lib)
    for cut in range(0, 8):
        left = dict(case, dt=case["dt"][:, :cut], Bm=case["Bm"][:, :cut], Cm=case["Cm"][:, :cut],
                    x=case["x"][:, :cut])
        yl, hm = ss_run(left, lib)
        right = dict(case, dt=case["dt"][:, cut:], Bm=case["Bm"][:, cut:], Cm=case["Cm"][:, cut:],
                     x=case["x"][:, cut:], h0=hm)
        yr, hr = ss_run(right, lib)
        assert np.array_equal(np.concatenate([yl, yr], axis=1), y), "split outputs"
        assert np.array_equal(hr, hT), "split final state"


def pin_selective_scan_special_cases(lib=None):
    """Degenerate cases with exact answers, and the pages' minimal elementwise scan."""
    case = ss_case(Bt=2, T=6, D=3, n=4, seed=33)
    # a zero step keeps the state (Abar = 1, Bbar = 0): y = C h0 + D x, h_T = h0 exactly
    y, hT = ss_run(case, lib, dt=np.zeros_like(case["dt"]), dt_bias=None, dt_softplus=False)
    assert np.array_equal(hT, case["h0"]), "zero step keeps the state"
    want = np.einsum("btn,bdn->btd", case["Cm"], case["h0"]) + case["Dskip"] * case["x"]
    assert rel(y, want) < 1e-13, "zero step output"
    # C = 0 and no initial state: only the skip remains
    y, _ = ss_run(case, lib, Cm=np.zeros_like(case["Cm"]))
    assert np.array_equal(y, case["Dskip"] * case["x"]), "C = 0 leaves D x"
    # one state entry: the minimal elementwise scan of the pages, state = a state + b x,
    # out = c state, with a = exp(Delta A), b = Delta B, c = C per channel
    case = ss_case(Bt=1, T=8, D=5, n=1, seed=34)
    y, hT = ss_run(case, lib, Dskip=None)
    delta = _softplus(case["dt"][0] + case["dt_bias"])                    # [T,D]
    a = np.exp(delta * case["A"][:, 0])
    b = delta * case["Bm"][0]                                             # [T,1] broadcast
    c = np.broadcast_to(case["Cm"][0], a.shape)
    state = case["h0"][0, :, 0].copy()
    for t in range(8):
        state = a[t] * state + b[t] * case["x"][0, t]
        assert rel(y[0, t], c[t] * state) < 1e-13, "elementwise scan output"
    assert rel(hT[0, :, 0], state) < 1e-13


def pin_selective_scan_is_ssd(lib=None):
    """Mamba-1 with one A per head (equal over the state entries) and one step per head and token
    is the SSD recurrence ("Linear / RNN 路线", section 4.1): per head, k = B, v = Delta x, q = C
    and the scalar decay exp(Delta A); the head's channel block of h is S^T."""
    rng = np.random.default_rng(35)
    Bt, T, Hh, P, n = 2, 10, 3, 2, 4
    D = Hh * P
    A_h = -rng.uniform(0.5, 3.0, Hh)
    delta_h = rng.uniform(0.05, 0.8, (Bt, T, Hh))
    A = np.repeat(A_h, P)[:, None] * np.ones((1, n))
    dt = np.repeat(delta_h, P, axis=2)
    Bm, Cm = rng.standard_normal((Bt, T, n)), rng.standard_normal((Bt, T, n))
    x = rng.standard_normal((Bt, T, D))
    h0 = rng.standard_normal((Bt, D, n))
    y, hT = oracle.selective_scan(dt, A, Bm, Cm, x, None, None, False, h0, lib_path=lib)
    q = np.repeat(Cm[:, None], Hh, axis=1)
    k = np.repeat(Bm[:, None], Hh, axis=1)
    xv = x.reshape(Bt, T, Hh, P).transpose(0, 2, 1, 3)
    v = delta_h.transpose(0, 2, 1)[..., None] * xv
    g = np.exp(delta_h.transpose(0, 2, 1) * A_h[None, :, None])
    S0 = h0.reshape(Bt, Hh, P, n).transpose(0, 1, 3, 2)
    o, S, _ = oracle.prefill("ssd", q, k, v, g, None, S0, None, lib_path=lib)
    assert rel(y, o.transpose(0, 2, 1, 3).reshape(Bt, T, D)) < 1e-12, "selective scan vs SSD"
    assert rel(hT, S.transpose(0, 1, 3, 2).reshape(Bt, D, n)) < 1e-12


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _loss(variant, case, dO, dSf, dzf, lib):
    """L = <dO, o> + <dS_final, S_final> (+ <dz_final, z_final>): its gradients are what the
    backward returns for that (dO, dS_final, dz_final)."""
    o, S, z = run(variant, case, lib)
    L = float(np.sum(dO * o) + np.sum(dSf * S))
    if variant == "kath":
        L += float(np.sum(dzf * z))
    return L


def _bwd_case(variant, seed):
    case = rand_case(variant, B=1, H=2, N=6, dk=3, dv=2, seed=seed, with_state=True)
    rng = np.random.default_rng(seed + 1000)
    dO = rng.standard_normal(case["v"].shape)
    dSf = rng.standard_normal(case["S0"].shape)
    dzf = rng.standard_normal(case["z0"].shape) if variant == "kath" else None
    return case, dO, dSf, dzf


def _bwd(variant, case, dO, dSf, dzf, lib):
    return oracle.prefill_backward(variant, case["q"], case["k"], case["v"], case["g"],
                                   case["beta"], case["S0"], case["z0"], dO, dSf, dzf,
                                   lib_path=lib)


def pin_backward_finite_differences(lib=None):
    """Every gradient of every variant against central finite differences of the forward
    (the definition of the derivative): h = 1e-5 in fp64, agreement to 1e-6 of the largest
    gradient entry. The forward itself is pinned above."""
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0",
             "z0": "dz0"}
    for variant in ("kath", "gla", "gdn", "kda", "ssd"):
        case, dO, dSf, dzf = _bwd_case(variant, seed=51)
        grads = _bwd(variant, case, dO, dSf, dzf, lib)
        for arg, gname in names.items():
            if case.get(arg) is None:
                continue
            x = case[arg]
            fd = np.zeros_like(x)
            h = 1e-5
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = _loss(variant, case, dO, dSf, dzf, lib)
                x[idx] = old - h
                lm = _loss(variant, case, dO, dSf, dzf, lib)
                x[idx] = old
                fd[idx] = (lp - lm) / (2 * h)
            got = grads[gname]
            assert got is not None and got.shape == x.shape, (variant, gname)
            err = np.max(np.abs(got - fd)) / max(np.max(np.abs(fd)), 1e-12)
            assert err < 1e-6, f"{variant} {gname} vs finite differences: {err:.2e}"


def pin_backward_closed_form(lib=None):
    """Ungated causal linear attention O = tril(Q K^T) V (GLA with g = 1, no initial state,
    no final-state gradient): dQ = tril(dO V^T) K, dK = tril(dO V^T)^T Q,
    dV = tril(Q K^T)^T dO."""
    case = rand_case("gla", B=1, H=1, N=9, dk=4, dv=3, seed=52, with_state=False)
    case["g"] = np.ones_like(case["g"])
    rng = np.random.default_rng(53)
    dO = rng.standard_normal(case["v"].shape)
    grads = _bwd("gla", case, dO, None, None, lib)
    Q, K, V, G = case["q"][0, 0], case["k"][0, 0], case["v"][0, 0], dO[0, 0]
    M = np.tril(np.ones((9, 9)))
    A = (G @ V.T) * M
    assert rel(grads["dq"][0, 0], A @ K) < 1e-13, "dQ closed form"
    assert rel(grads["dk"][0, 0], A.T @ Q) < 1e-13, "dK closed form"
    assert rel(grads["dv"][0, 0], ((Q @ K.T) * M).T @ G) < 1e-13, "dV closed form"
    assert rel(grads["dS0"][0, 0], Q.T @ G) < 1e-13, "dS0 closed form (the zero state's gradient)"


def pin_backward_log_gate_identity(lib=None):
    """For a diagonal transition, o_t depends on the gates only through q_t exp(B_t) and
    k_s exp(-B_s) with B_t the cumulative log gate, and S_final through exp(B_N); so
    g_s dL/dg_s = sum_{t >= s} (q_t dq_t - k_t dk_t) + (dS_final * S_final) summed over the
    value dim (per key dim for GLA; also over the key dims for SSD). The oracle's gate
    gradient comes from the per-token state products instead."""
    for variant in ("gla", "ssd"):
        case, dO, dSf, _ = _bwd_case(variant, seed=54)
        grads = _bwd(variant, case, dO, dSf, None, lib)
        _, S, _ = run(variant, case, lib)
        c = case["q"] * grads["dq"] - case["k"] * grads["dk"]           # [B,H,N,dk]
        rev = np.flip(np.cumsum(np.flip(c, axis=2), axis=2), axis=2)
        fin = np.sum(dSf * S, axis=-1)[:, :, None, :]                    # [B,H,1,dk]
        want = rev + fin
        if variant == "ssd":
            want = want.sum(axis=-1)
        assert rel(case["g"] * grads["dg"], want) < 1e-12, f"{variant} log-gate identity"


def pin_backward_split(lib=None):
    """The chain rule across a split: the backward of the second part with dS_final gives
    the gradient of its initial state, which is the first part's dS_final; together the two
    backwards equal the backward of the whole sequence."""
    for variant in ("kath", "gla", "gdn", "kda", "ssd"):
        case, dO, dSf, dzf = _bwd_case(variant, seed=55)
        whole = _bwd(variant, case, dO, dSf, dzf, lib)
        m = 2
        left = {kk: (vv[:, :, :m] if (vv is not None and kk in ("q", "k", "v", "g", "beta"))
                     else vv) for kk, vv in case.items()}
        _, Sm, zm = run(variant, left, lib)
        right = {kk: (vv[:, :, m:] if (vv is not None and kk in ("q", "k", "v", "g", "beta"))
                      else vv) for kk, vv in case.items()}
        right["S0"], right["z0"] = Sm, zm
        gr = _bwd(variant, right, dO[:, :, m:], dSf, dzf, lib)
        gl = _bwd(variant, left, dO[:, :, :m], gr["dS0"], gr["dz0"], lib)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            if whole[name] is None:
                continue
            cat = np.concatenate([gl[name], gr[name]], axis=2)
            assert rel(cat, whole[name]) < 1e-12, f"{variant} {name} split"
        assert rel(gl["dS0"], whole["dS0"]) < 1e-12, f"{variant} dS0 split"


ALL_PINS = [pin_quadratic_form, pin_split_invariance, pin_gdn_page_forms, pin_kda_forms,
            pin_ssd_selective_ssm, pin_delta_identity,
            pin_worked_example, pin_closed_forms, pin_special_cases, pin_causality,
            pin_linearity, pin_decode_matches_prefill,
            pin_selective_scan_unrolled, pin_selective_scan_convolution, pin_selective_scan_split,
            pin_selective_scan_special_cases, pin_selective_scan_is_ssd,
            pin_backward_finite_differences, pin_backward_closed_form,
            pin_backward_log_gate_identity, pin_backward_split]
