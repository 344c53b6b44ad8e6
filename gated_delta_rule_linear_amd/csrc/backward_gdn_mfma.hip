// Backward of the chunked Gated DeltaNet prefill on bf16 MFMA ("线性注意力与 SSM", section
// GDN: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t, the
// state key-major), d_k = 128, d_v = 64 or 128, chunk C = 64, bf16 q, k, v and dO.
//
// One chunk, rows r, s, t, x = 0..63, c_r the cumulative base-2 log gate from the chunk start,
// eg_r = 2^c_r, el_r = 2^(c_last - c_r), gm_t = 2^c_{t-1} (1 for t = 0), D_rs = 2^(c_r - c_s)
// for s <= r and Dm_ts = 2^(c_{t-1} - c_s) for s < t (0 elsewhere; every factor at most 1),
// S_in the state entering the chunk and dS_out the gradient of the state leaving it:
//   L_rs = beta_r D_rs k_r.k_s (s < r),  T = (I + L)^-1,  P_rs = D_rs q_r.k_s (s <= r)
//   X = diag(beta) (V - diag(eg) K S_in),   U = T X                      (the forward's U)
//   R = diag(el) K dS_out + P^T dO,          dU = T^T R                   (du of every row)
//   S_out = eg_last S_in + K^T diag(el) U
//   dS_in = eg_last dS_out + Q^T diag(eg) dO - K^T diag(beta eg) dU
// and, with A = dO U^T and B = dU U^T (value columns summed),
//   dv = diag(beta) dU
//   dq = diag(eg) dO S_in^T + (D o A) K
//   dk = diag(el) U dS_out^T - diag(beta eg) dU S_in^T + (D o A)^T Q - (Mb + Mb^T) K,
//        Mb_ts = beta_t D_ts B_ts (s < t)
//   dbeta_t = dU_t.v_t - eg_t mu_t - sum_{s<t} D_ts (k_t.k_s) B_ts
//   dalpha_t = sum_{x<t} el_t Dm_tx kap_x + sum_{x>=t} D_xt (gm_t rho_x + Z1_xt)
//              - sum_{x>t} D_xt beta_x (gm_t mu_x + Z2_xt) + el_t gm_t <dS_out, S_in>
//              - beta_t (gm_t mu_t + sum_{s<t} Dm_ts (k_t.k_s) B_ts)
// where kap_x = (K dS_out)_x.U_x, rho_x = (Q S_in)_x.dO_x, mu_x = (K S_in)_x.dU_x, Z1 =
// ((Q K^T) o A) Dm^T and Z2 = ((K K^T) o B) Dm^T. These are the token-form gradients of the
// delta rule (u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t), du_t = G_t^T k_t, dalpha_t =
// <G_t, S_{t-1}> - beta_t du_t . S_{t-1}^T k_t, ...) summed over the chunk. The gate gradient
// is taken directly, never as a reverse sum of dL/dlog alpha divided by alpha.
//
// Three launches:
//   prep    per (sequence, chunk): K K^T and Q K^T on the matrix cores, T = (I + L)^-1 by
//           fp32 forward substitution (one column per lane), T and P stored in bf16;
//   chains  per (sequence, 32 value columns, direction), both directions in one launch:
//           the state (or its gradient) in fp32 accumulators through the chunks; the
//           forward chain stores S_in of every chunk, the reverse chain dS_out of every
//           chunk (bf16, transposed: [column][key]) and dS0;
//   grads   per (sequence, chunk), the value columns in halves of 64: every gradient.
// The workspace (bf16 S_in, dS_out, T, P per chunk) is 0.63 GiB for 64 sequences of 8,192
// tokens at d_k = d_v = 128.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;   // 64
constexpr int NT = 256;
constexpr int HV = 64;          // value columns per half in the grads kernel
constexpr int VT = 32;          // value columns per chain workgroup
constexpr int PQ = DK + 8;      // pitch of [*][128] bf16 tiles
constexpr int PC = C + 8;       // pitch of [*][64] bf16 tiles
constexpr int PV = VT + 8;      // pitch of [*][32] bf16 tiles
static_assert(HV == C, "the half tiles share the [*][64] pitch");

struct GbArgs {
    const uint16_t *q, *k, *v, *dO;
    const void *g, *beta;
    const float *S0, *dSf;
    uint16_t *dq, *dk, *dv;
    void *dg, *dbeta;
    float* dS0;
    uint16_t *Sck, *dSck;   // [nseq][nch][dv][DK]: S_in^T and dS_out^T of every chunk
    uint16_t *Tck, *Pck;    // [nseq][nch][C][C]: T and P of every chunk
    int N, nseq, nch;
};

template <bool GB>
__device__ __forceinline__ float gate_at(const void* p, size_t i) {
    return GB ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
template <bool GB>
__device__ __forceinline__ void store_gate(void* p, size_t i, float x) {
    if (GB) static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
    else static_cast<float*>(p)[i] = x;
}

// A thread's 16-byte pieces of an [R][W] bf16 block: fetched into registers first and
// written to LDS later, so that a chunk's loads are all in flight together.
template <int R, int W>
struct Blk {
    static constexpr int PPR = W / 8, NP = R * PPR / NT;
    static_assert(R * PPR % NT == 0, "whole pieces per thread");
    uint4 w[NP];
    __device__ static int row(int x) { return (int(threadIdx.x) + NT * x) / PPR; }
    __device__ static int col(int x) { return ((int(threadIdx.x) + NT * x) % PPR) * 8; }
};
// through a buffer resource whose rows are pitch_bytes apart (reads past its end are zero)
template <int R, int W>
__device__ __forceinline__ void blk_fetch(Blk<R, W>& b, rsrc_t rs, uint32_t pitch_bytes) {
#pragma unroll
    for (int x = 0; x < Blk<R, W>::NP; ++x)
        b.w[x] = buf_ld16(rs, uint32_t(Blk<R, W>::row(x)) * pitch_bytes +
                                  uint32_t(Blk<R, W>::col(x)) * 2u);
}
template <int R, int W, int P>
__device__ __forceinline__ void blk_stage(uint16_t* dst, const Blk<R, W>& b) {
#pragma unroll
    for (int x = 0; x < Blk<R, W>::NP; ++x)
        *reinterpret_cast<uint4*>(dst + Blk<R, W>::row(x) * P + Blk<R, W>::col(x)) = b.w[x];
}
template <int R, int W, int P, typename F>
__device__ __forceinline__ void blk_stage_scaled(uint16_t* dst, const Blk<R, W>& b, F scale) {
#pragma unroll
    for (int x = 0; x < Blk<R, W>::NP; ++x) {
        float y[8];
        unpack8(b.w[x], y);
        const float f = scale(Blk<R, W>::row(x));
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= f;
        *reinterpret_cast<uint4*>(dst + Blk<R, W>::row(x) * P + Blk<R, W>::col(x)) = pack8(y);
    }
}

// Sum over the 16 lanes of each lane group (a D tile's column index).
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<0xB1, 0xf, 0xf>(v);
    v += dpp_f<0x4E, 0xf, 0xf>(v);
    v += dpp_f<0x141, 0xf, 0xf>(v);
    v += dpp_f<0x140, 0xf, 0xf>(v);
    return v;
}

// ---------------------------------------------------------------------------- prep
struct __align__(16) PrepSmem {
    union {
        struct {
            __align__(16) uint16_t q[C * PQ];
            __align__(16) uint16_t k[C * PQ];
        } in;
        __align__(16) float L[C][C + 4];   // after the products; rows 16-byte aligned
    };
    float c[C], b[C];
};

template <bool GB>
__global__ __launch_bounds__(NT) void gdn_bwd_prep_mfma(GbArgs a) {
    __shared__ PrepSmem sm;
    const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 4, jl = lane & 15;
    const int ch = int(blockIdx.x % unsigned(a.nch));
    const size_t seq = blockIdx.x / unsigned(a.nch);
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok = seq * size_t(a.N) + t0;
    Blk<C, DK> qb, kb;
    const uint32_t rows = uint32_t(n) * DK * 2u;
    blk_fetch(qb, make_rsrc(a.q + tok * DK, rows), DK * 2u);
    blk_fetch(kb, make_rsrc(a.k + tok * DK, rows), DK * 2u);
    if (threadIdx.x < C) {
        const int r = threadIdx.x;
        float lg = 0.f, bt = 0.f;
        if (r < n) {
            lg = __builtin_amdgcn_logf(gate_at<GB>(a.g, tok + r));
            bt = gate_at<GB>(a.beta, tok + r);
        }
        sm.c[r] = wave_inclusive_scan(lg);
        sm.b[r] = bt;
    }
    blk_stage<C, DK, PQ>(sm.in.q, qb);
    blk_stage<C, DK, PQ>(sm.in.k, kb);
    __syncthreads();
    f32x4_t kk[4], qk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) kk[nt] = qk[nt] = zero4();
#pragma unroll
    for (int kc = 0; kc < DK / 32; ++kc) {
        const bf16x8_t ak = frag_kc(sm.in.k, PQ, 16 * w, 32 * kc, lane);
        const bf16x8_t aq = frag_kc(sm.in.q, PQ, 16 * w, 32 * kc, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const bf16x8_t bk = frag_kc(sm.in.k, PQ, 16 * nt, 32 * kc, lane);
            kk[nt] = mfma16(ak, bk, kk[nt]);
            qk[nt] = mfma16(aq, bk, qk[nt]);
        }
    }
    __syncthreads();   // the q, k tiles are read; L takes their place
    uint16_t* Pg = a.Pck + (seq * a.nch + ch) * size_t(C * C);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * w + 4 * g + e, s = 16 * nt + jl;
            const float d = s <= r ? __builtin_amdgcn_exp2f(sm.c[r] - sm.c[s]) : 0.f;
            sm.L[r][s] = s < r ? sm.b[r] * d * kk[nt][e] : 0.f;
            Pg[r * C + s] = f32_to_bf16(d * qk[nt][e]);
        }
    }
    __syncthreads();
    if (w == 0) {
        // T = (I + L)^-1, column j = lane: x_r = delta_rj - sum_{s<r} L_rs x_s, four partial
        // sums per row
        const int j = lane;
        uint16_t* Tg = a.Tck + (seq * a.nch + ch) * size_t(C * C);
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float p[4] = {r == j ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < (r & ~3); s += 4) {
                const float4 l4 = *reinterpret_cast<const float4*>(&sm.L[r][s]);
                p[0] -= l4.x * x[s];
                p[1] -= l4.y * x[s + 1];
                p[2] -= l4.z * x[s + 2];
                p[3] -= l4.w * x[s + 3];
            }
#pragma unroll
            for (int s = r & ~3; s < r; ++s) p[s & 3] -= sm.L[r][s] * x[s];
            x[r] = (p[0] + p[1]) + (p[2] + p[3]);
            Tg[r * C + j] = f32_to_bf16(x[r]);
        }
    }
}

// ---------------------------------------------------------------------------- chains
struct __align__(16) ChainSmem {
    __align__(16) uint16_t k[C * PQ];    // K [token][key]
    __align__(16) uint16_t q[C * PQ];    // reverse: diag(eg) Q
    __align__(16) uint16_t st[VT * PQ];  // the state (or gradient) tile, transposed [column][key]
    __align__(16) uint16_t x[C * PV];    // V (forward) or dO (reverse) tile [token][column]
    __align__(16) uint16_t y[VT * PC];   // X^T or R^T [column][token]
    __align__(16) uint16_t z[VT * PC];   // (diag(el) U)^T or (-diag(beta eg) dU)^T
    __align__(16) uint16_t t[C * PC];    // T [r][s]
    __align__(16) uint16_t p[C * PC];    // reverse: P [r][s]
    float c[2][C], b[2][C];              // gates of the current and the next chunk
};

// One chain: wave w carries key rows 32 w .. 32 w + 31 of the tile (two row tiles) and its
// VT = 32 columns (two column tiles) in fp32 accumulators.
template <bool GB, int DV, bool REV>
__device__ __forceinline__ void chain_walk(const GbArgs& a, ChainSmem& sm, size_t seq, int c0) {
    const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 4, jl = lane & 15;
    f32x4_t S[2][2];
    const float* init = REV ? a.dSf : a.S0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t i = size_t(32 * w + 16 * rt + 4 * g + e);
                S[rt][ct][e] = init ? init[(seq * DK + i) * DV + c0 + 16 * ct + jl] : 0.f;
            }
    uint16_t* ck = (REV ? a.dSck : a.Sck) + seq * size_t(a.nch) * DV * DK;
    const uint16_t* xsrc = REV ? a.dO : a.v;
    Blk<C, DK> kb, qb;
    Blk<C, VT> xb;
    Blk<C, C> tb, pb;
    uint32_t graw = 0, braw = 0;
    auto fetch = [&](int ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
        const size_t tok = seq * size_t(a.N) + t0;
        constexpr uint32_t gs = GB ? 2u : 4u;
        // the gates first: wave 0 waits on them before the rest has arrived
        graw = buf_ld_gate<GB>(make_rsrc(static_cast<const char*>(a.g) + tok * gs, uint32_t(n) * gs), uint32_t(lane));
        braw = buf_ld_gate<GB>(make_rsrc(static_cast<const char*>(a.beta) + tok * gs, uint32_t(n) * gs), uint32_t(lane));
        const uint32_t rows = uint32_t(n) * DK * 2u;
        blk_fetch(kb, make_rsrc(a.k + tok * DK, rows), DK * 2u);
        if (REV) blk_fetch(qb, make_rsrc(a.q + tok * DK, rows), DK * 2u);
        blk_fetch(xb, make_rsrc(xsrc + tok * DV + c0, uint32_t(n - 1) * DV * 2u + VT * 2u), DV * 2u);
        const size_t cb = (seq * a.nch + ch) * size_t(C * C);
        blk_fetch(tb, make_rsrc(a.Tck + cb, C * C * 2u), C * 2u);
        if (REV) blk_fetch(pb, make_rsrc(a.Pck + cb, C * C * 2u), C * 2u);
    };
    auto gates = [&](int ch, int buf) {   // wave 0: cumulative log gates and beta of a chunk
        if (w == 0) {
            const int n = min(C, a.N - ch * C);
            const float lg = lane < n ? __builtin_amdgcn_logf(gate_val<GB>(graw)) : 0.f;
            sm.c[buf][lane] = wave_inclusive_scan(lg);
            sm.b[buf][lane] = lane < n ? gate_val<GB>(braw) : 0.f;
        }
    };
    const int first = REV ? a.nch - 1 : 0;
    fetch(first);
    gates(first, 0);
    for (int it = 0; it < a.nch; ++it) {
        const int ch = REV ? a.nch - 1 - it : it, cur = it & 1;
        const float* cc = sm.c[cur];
        const float* bb = sm.b[cur];
        lds_barrier();   // the last chunk's readers are done; this chunk's gates are in LDS
        uint16_t* ckc = ck + size_t(ch) * DV * DK;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const uint2 pk = make_uint2(pack_bf16x2(S[rt][ct][0], S[rt][ct][1]),
                                            pack_bf16x2(S[rt][ct][2], S[rt][ct][3]));
                const int i = 32 * w + 16 * rt + 4 * g, j = 16 * ct + jl;
                *reinterpret_cast<uint2*>(sm.st + j * PQ + i) = pk;
                *reinterpret_cast<uint2*>(ckc + size_t(c0 + j) * DK + i) = pk;
            }
        blk_stage<C, DK, PQ>(sm.k, kb);
        if (REV) blk_stage_scaled<C, DK, PQ>(sm.q, qb, [&](int r) { return __builtin_amdgcn_exp2f(cc[r]); });
        blk_stage<C, VT, PV>(sm.x, xb);
        blk_stage<C, C, PC>(sm.t, tb);
        if (REV) blk_stage<C, C, PC>(sm.p, pb);
        const bool more = it + 1 < a.nch;
        const int nxt = REV ? ch - 1 : ch + 1;
        if (more) fetch(nxt);
        lds_barrier();
        const float cl = cc[C - 1];
        {   // K S (forward) or K dS and P^T dO (reverse), rows 16 w ..
            f32x4_t ks[2] = {zero4(), zero4()}, pd[2] = {zero4(), zero4()};
#pragma unroll
            for (int kc = 0; kc < DK / 32; ++kc) {
                const bf16x8_t ak = frag_kc(sm.k, PQ, 16 * w, 32 * kc, lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    ks[ct] = mfma16(ak, frag_kc(sm.st, PQ, 16 * ct, 32 * kc, lane), ks[ct]);
            }
            if (REV) {
#pragma unroll
                for (int kc = 0; kc < C / 32; ++kc) {
                    const bf16x8_t ap = frag_kr(sm.p, PC, 32 * kc, 16 * w, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        pd[ct] = mfma16(ap, frag_kr(sm.x, PV, 32 * kc, 16 * ct, lane), pd[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * g + e;
                    if (REV)
                        y[e] = __builtin_amdgcn_exp2f(cl - cc[r]) * ks[ct][e] + pd[ct][e];
                    else
                        y[e] = bb[r] * (bf16_to_f32(sm.x[r * PV + 16 * ct + jl]) -
                                        __builtin_amdgcn_exp2f(cc[r]) * ks[ct][e]);
                }
                store_dT(sm.y, PC, 16 * w, 16 * ct, y, lane);
            }
        }
        lds_barrier();
        {   // U = T X or dU = T^T R, rows 16 w ..
            f32x4_t u[2] = {zero4(), zero4()};
#pragma unroll
            for (int kc = 0; kc < C / 32; ++kc) {
                const bf16x8_t at = REV ? frag_kr(sm.t, PC, 32 * kc, 16 * w, lane)
                                        : frag_kc(sm.t, PC, 16 * w, 32 * kc, lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    u[ct] = mfma16(at, frag_kc(sm.y, PC, 16 * ct, 32 * kc, lane), u[ct]);
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * g + e;
                    u[ct][e] *= REV ? -bb[r] * __builtin_amdgcn_exp2f(cc[r])
                                    : __builtin_amdgcn_exp2f(cl - cc[r]);
                }
                store_dT(sm.z, PC, 16 * w, 16 * ct, u[ct], lane);
            }
        }
        if (more) gates(nxt, cur ^ 1);
        lds_barrier();
        {   // the update of this wave's key rows
            const float el = __builtin_amdgcn_exp2f(cl);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) S[rt][ct] *= el;
#pragma unroll
            for (int kc = 0; kc < C / 32; ++kc) {
                bf16x8_t bz[2], bx[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    bz[ct] = frag_kc(sm.z, PC, 16 * ct, 32 * kc, lane);
                    if (REV) bx[ct] = frag_kr(sm.x, PV, 32 * kc, 16 * ct, lane);
                }
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const bf16x8_t ak = frag_kr(sm.k, PQ, 32 * kc, 32 * w + 16 * rt, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) S[rt][ct] = mfma16(ak, bz[ct], S[rt][ct]);
                    if (REV) {
                        const bf16x8_t aq = frag_kr(sm.q, PQ, 32 * kc, 32 * w + 16 * rt, lane);
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) S[rt][ct] = mfma16(aq, bx[ct], S[rt][ct]);
                    }
                }
            }
        }
    }
    if (REV) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t i = size_t(32 * w + 16 * rt + 4 * g + e);
                    a.dS0[(seq * DK + i) * DV + c0 + 16 * ct + jl] = S[rt][ct][e];
                }
    }
}

template <bool GB, int DV>
__global__ __launch_bounds__(NT) void gdn_bwd_chain_mfma(GbArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainSmem& sm = *reinterpret_cast<ChainSmem*>(smem_raw);
    constexpr int NTL = DV / VT;
    const int nfw = a.nseq * NTL;
    const bool rev = int(blockIdx.x) >= nfw;
    const int unit = rev ? int(blockIdx.x) - nfw : int(blockIdx.x);
    const size_t seq = size_t(unit / NTL);
    const int c0 = (unit % NTL) * VT;
    if (rev) chain_walk<GB, DV, true>(a, sm, seq, c0);
    else chain_walk<GB, DV, false>(a, sm, seq, c0);
}

// ---------------------------------------------------------------------------- grads
struct __align__(16) GradSmem {
    __align__(16) uint16_t q[C * PQ], k[C * PQ];
    __align__(16) uint16_t t[C * PC];    // T [r][s]
    __align__(16) uint16_t pt[C * PC];   // P^T [s][r]
    union {
        struct {   // one half of the value columns
            __align__(16) uint16_t v[C * PC], dO[C * PC];      // [token][column]
            __align__(16) uint16_t s0[HV * PQ], ds[HV * PQ];   // S_in^T, dS_out^T [column][key]
            __align__(16) uint16_t xu[HV * PC], rd[HV * PC];   // X^T then U^T, R^T then dU^T
            __align__(16) uint16_t us[HV * PC], dus[HV * PC];  // (diag(el) U)^T, (-diag(beta eg) dU)^T
        } h;
        struct {   // after both halves
            __align__(16) uint16_t adT[C * PC];   // (D o A)^T [s][t]
            __align__(16) uint16_t mbT[C * PC];   // -Mb^T [s][t]
            __align__(16) uint16_t h1T[C * PC];   // ((Q K^T) o A)^T [s][x]
            __align__(16) uint16_t h2T[C * PC];   // ((K K^T) o B)^T [s][x]
            __align__(16) uint16_t dm[C * PC];    // Dm [t][s]
        } f;
    };
    float c[C], b[C];
    float kap[C], rho[C], mu[C], vdu[C], dbp[C], dup[C];
    float zw[NT / 64][C];   // per-wave partials of the Z terms, summed in wave order
    float sig[NT / 64];
};

template <bool GB, int DV>
__global__ __launch_bounds__(NT) void gdn_bwd_grads_mfma(GbArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    GradSmem& sm = *reinterpret_cast<GradSmem*>(smem_raw);
    constexpr int NH = DV / HV;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4, jl = lane & 15;
    const int ch = int(blockIdx.x % unsigned(a.nch));
    const size_t seq = blockIdx.x / unsigned(a.nch);
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok = seq * size_t(a.N) + t0;
    const size_t cb = seq * a.nch + ch;
    const uint32_t rows = uint32_t(n) * DK * 2u;
    Blk<C, DK> qb, kb;
    Blk<C, C> tb;
    Blk<C, HV> vb, ob;
    Blk<HV, DK> sb, db;
    blk_fetch(qb, make_rsrc(a.q + tok * DK, rows), DK * 2u);
    blk_fetch(kb, make_rsrc(a.k + tok * DK, rows), DK * 2u);
    blk_fetch(tb, make_rsrc(a.Tck + cb * C * C, C * C * 2u), C * 2u);
    auto fetch_half = [&](int h) {
        const uint32_t vrows = uint32_t(n - 1) * DV * 2u + HV * 2u;
        blk_fetch(vb, make_rsrc(a.v + tok * DV + h * HV, vrows), DV * 2u);
        blk_fetch(ob, make_rsrc(a.dO + tok * DV + h * HV, vrows), DV * 2u);
        const size_t so = (cb * DV + size_t(h) * HV) * DK;
        blk_fetch(sb, make_rsrc(a.Sck + so, HV * DK * 2u), DK * 2u);
        blk_fetch(db, make_rsrc(a.dSck + so, HV * DK * 2u), DK * 2u);
    };
    fetch_half(0);
    if (tid < C) {
        const int r = tid;
        float lg = 0.f, bt = 0.f;
        if (r < n) {
            lg = __builtin_amdgcn_logf(gate_at<GB>(a.g, tok + r));
            bt = gate_at<GB>(a.beta, tok + r);
        }
        sm.c[r] = wave_inclusive_scan(lg);
        sm.b[r] = bt;
    }
    blk_stage<C, DK, PQ>(sm.q, qb);
    blk_stage<C, DK, PQ>(sm.k, kb);
    blk_stage<C, C, PC>(sm.t, tb);
    __syncthreads();
    // Q K^T, rows 16 w ..; P^T to LDS
    f32x4_t qk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) qk[nt] = zero4();
#pragma unroll
    for (int kc = 0; kc < DK / 32; ++kc) {
        const bf16x8_t aq = frag_kc(sm.q, PQ, 16 * w, 32 * kc, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            qk[nt] = mfma16(aq, frag_kc(sm.k, PQ, 16 * nt, 32 * kc, lane), qk[nt]);
    }
    const float* cc = sm.c;
    const float* bb = sm.b;
    // The lane's gate factors, read once before any LDS write: LDS reads issued after an LDS
    // write the compiler cannot tell apart wait for it, one round trip each. Rows r = 16 w +
    // 4 g + e (the result-tile rows), columns s = 16 nt + j.
    const float cl = cc[C - 1];
    float cr[4], br[4], cmr[4], egr[4], elr[4], cs4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * g + e;
        cr[e] = cc[r];
        br[e] = bb[r];
        cmr[e] = r > 0 ? cc[r - 1] : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) cs4[nt] = cc[16 * nt + jl];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        egr[e] = __builtin_amdgcn_exp2f(cr[e]);
        elr[e] = __builtin_amdgcn_exp2f(cl - cr[e]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        f32x4_t pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * w + 4 * g + e, s = 16 * nt + jl;
            pv[e] = s <= r ? __builtin_amdgcn_exp2f(cr[e] - cs4[nt]) * qk[nt][e] : 0.f;
        }
        store_dT(sm.pt, PC, 16 * w, 16 * nt, pv, lane);
    }
    f32x4_t dq[8], dk1[8], A[4], Bm[4];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) dq[nt] = dk1[nt] = zero4();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) A[nt] = Bm[nt] = zero4();
    float kap[4] = {}, rho[4] = {}, mu[4] = {}, vdu[4] = {};
    float sig = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        // this half's v, dO, S_in^T, dS_out^T, and <dS_out, S_in> over its pieces
        blk_stage<C, HV, PC>(sm.h.v, vb);
        blk_stage<C, HV, PC>(sm.h.dO, ob);
        blk_stage<HV, DK, PQ>(sm.h.s0, sb);
        blk_stage<HV, DK, PQ>(sm.h.ds, db);
#pragma unroll
        for (int x = 0; x < Blk<HV, DK>::NP; ++x) {
            float s8[8], d8[8];
            unpack8(sb.w[x], s8);
            unpack8(db.w[x], d8);
#pragma unroll
            for (int e = 0; e < 8; ++e) sig += s8[e] * d8[e];
        }
        if (h + 1 < NH) fetch_half(h + 1);
        lds_barrier();
        {   // K S_in, K dS_out, Q S_in and P^T dO; X and R to LDS
            f32x4_t ks[4], kd[4], qs[4], pd[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ks[ct] = kd[ct] = qs[ct] = pd[ct] = zero4();
#pragma unroll
            for (int kc = 0; kc < DK / 32; ++kc) {
                const bf16x8_t ak = frag_kc(sm.k, PQ, 16 * w, 32 * kc, lane);
                const bf16x8_t aq = frag_kc(sm.q, PQ, 16 * w, 32 * kc, lane);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8_t bs = frag_kc(sm.h.s0, PQ, 16 * ct, 32 * kc, lane);
                    const bf16x8_t bd = frag_kc(sm.h.ds, PQ, 16 * ct, 32 * kc, lane);
                    ks[ct] = mfma16(ak, bs, ks[ct]);
                    kd[ct] = mfma16(ak, bd, kd[ct]);
                    qs[ct] = mfma16(aq, bs, qs[ct]);
                }
            }
#pragma unroll
            for (int kc = 0; kc < C / 32; ++kc) {
                const bf16x8_t ap = frag_kc(sm.pt, PC, 16 * w, 32 * kc, lane);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    pd[ct] = mfma16(ap, frag_kr(sm.h.dO, PC, 32 * kc, 16 * ct, lane), pd[ct]);
            }
            float vv[4][4], dd[4][4];   // v and dO of the lane's tile entries, read first
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * g + e, j = 16 * ct + jl;
                    vv[ct][e] = bf16_to_f32(sm.h.v[r * PC + j]);
                    dd[ct][e] = bf16_to_f32(sm.h.dO[r * PC + j]);
                }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4_t xv, rv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rho[e] += qs[ct][e] * dd[ct][e];
                    xv[e] = br[e] * (vv[ct][e] - egr[e] * ks[ct][e]);
                    rv[e] = elr[e] * kd[ct][e] + pd[ct][e];
                }
                store_dT(sm.h.xu, PC, 16 * w, 16 * ct, xv, lane);
                store_dT(sm.h.rd, PC, 16 * w, 16 * ct, rv, lane);
            }
            lds_barrier();
            // U = T X, dU = T^T R
            f32x4_t u[4], du[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) u[ct] = du[ct] = zero4();
#pragma unroll
            for (int kc = 0; kc < C / 32; ++kc) {
                const bf16x8_t at = frag_kc(sm.t, PC, 16 * w, 32 * kc, lane);
                const bf16x8_t att = frag_kr(sm.t, PC, 32 * kc, 16 * w, lane);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    u[ct] = mfma16(at, frag_kc(sm.h.xu, PC, 16 * ct, 32 * kc, lane), u[ct]);
                    du[ct] = mfma16(att, frag_kc(sm.h.rd, PC, 16 * ct, 32 * kc, lane), du[ct]);
                }
            }
            // dv rows past the sequence's end fall outside the resource and are dropped
            const rsrc_t rdv = make_rsrc(a.dv + tok * DV + h * HV, uint32_t((n - 1) * DV + HV) * 2u);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * g + e, j = 16 * ct + jl;
                    kap[e] += kd[ct][e] * u[ct][e];
                    mu[e] += ks[ct][e] * du[ct][e];
                    vdu[e] += vv[ct][e] * du[ct][e];
                    buf_st2(rdv, uint32_t(r * DV + j) * 2u, f32_to_bf16(br[e] * du[ct][e]));
                }
            }
            lds_barrier();   // X^T and R^T are read; U^T and dU^T take their place
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                store_dT(sm.h.xu, PC, 16 * w, 16 * ct, u[ct], lane);
                store_dT(sm.h.rd, PC, 16 * w, 16 * ct, du[ct], lane);
                f32x4_t us_, dus_;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    us_[e] = elr[e] * u[ct][e];
                    dus_[e] = -br[e] * egr[e] * du[ct][e];
                }
                store_dT(sm.h.us, PC, 16 * w, 16 * ct, us_, lane);
                store_dT(sm.h.dus, PC, 16 * w, 16 * ct, dus_, lane);
            }
        }
        lds_barrier();
        // A += dO U^T, B += dU U^T, and the value-column sums of dq and dk
#pragma unroll
        for (int kc = 0; kc < HV / 32; ++kc) {
            const bf16x8_t ado = frag_kc(sm.h.dO, PC, 16 * w, 32 * kc, lane);
            const bf16x8_t adu = frag_kr(sm.h.rd, PC, 32 * kc, 16 * w, lane);
            const bf16x8_t aus = frag_kr(sm.h.us, PC, 32 * kc, 16 * w, lane);
            const bf16x8_t adus = frag_kr(sm.h.dus, PC, 32 * kc, 16 * w, lane);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8_t bu = frag_kr(sm.h.xu, PC, 32 * kc, 16 * nt, lane);
                A[nt] = mfma16(ado, bu, A[nt]);
                Bm[nt] = mfma16(adu, bu, Bm[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const bf16x8_t bs = frag_kr(sm.h.s0, PQ, 32 * kc, 16 * nt, lane);
                const bf16x8_t bd = frag_kr(sm.h.ds, PQ, 32 * kc, 16 * nt, lane);
                dq[nt] = mfma16(ado, bs, dq[nt]);
                dk1[nt] = mfma16(aus, bd, dk1[nt]);
                dk1[nt] = mfma16(adus, bs, dk1[nt]);
            }
        }
        lds_barrier();   // the half's tiles are read
    }
    // row sums of the per-lane partials, and the chunk's matrices for the last products
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float k1 = sum16(kap[e]), r1 = sum16(rho[e]), m1 = sum16(mu[e]), v1 = sum16(vdu[e]);
        if (jl == 0) {
            const int r = 16 * w + 4 * g + e;
            sm.kap[r] = k1;
            sm.rho[r] = r1;
            sm.mu[r] = m1;
            sm.vdu[r] = v1;
        }
    }
    sig = wave_sum(sig);
    if (lane == 0) sm.sig[w] = sig;
    {
        // Q K^T and K K^T of the wave's rows again (q and k are still in LDS): formed anew
        // here rather than held in registers through the halves
        f32x4_t qk[4], kk[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) qk[nt] = kk[nt] = zero4();
#pragma unroll
        for (int kc = 0; kc < DK / 32; ++kc) {
            const bf16x8_t ak = frag_kc(sm.k, PQ, 16 * w, 32 * kc, lane);
            const bf16x8_t aq = frag_kc(sm.q, PQ, 16 * w, 32 * kc, lane);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8_t bk = frag_kc(sm.k, PQ, 16 * nt, 32 * kc, lane);
                kk[nt] = mfma16(ak, bk, kk[nt]);
                qk[nt] = mfma16(aq, bk, qk[nt]);
            }
        }
        float dbp[4] = {}, dupp[4] = {};
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4_t ad, mb, h1, h2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * w + 4 * g + e, s = 16 * nt + jl;
                const float d = s <= t ? __builtin_amdgcn_exp2f(cr[e] - cs4[nt]) : 0.f;
                const float dmv = s < t ? __builtin_amdgcn_exp2f(cmr[e] - cs4[nt]) : 0.f;
                const float kb2 = kk[nt][e] * Bm[nt][e];
                ad[e] = d * A[nt][e];
                mb[e] = s < t ? -br[e] * d * Bm[nt][e] : 0.f;
                if (s < t) dbp[e] += d * kb2;
                dupp[e] += dmv * kb2;
                h1[e] = qk[nt][e] * A[nt][e];
                h2[e] = kb2;
            }
            store_dT(sm.f.adT, PC, 16 * w, 16 * nt, ad, lane);
            store_dT(sm.f.mbT, PC, 16 * w, 16 * nt, mb, lane);
            store_dT(sm.f.h1T, PC, 16 * w, 16 * nt, h1, lane);
            store_dT(sm.f.h2T, PC, 16 * w, 16 * nt, h2, lane);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = sum16(dbp[e]), y = sum16(dupp[e]);
            if (jl == 0) {
                sm.dbp[16 * w + 4 * g + e] = x;
                sm.dup[16 * w + 4 * g + e] = y;
            }
        }
        {   // Dm: thread tid fills column s = tid mod C of rows tid / C + 4 i (every read first)
            static_assert(NT % C == 0, "whole rows per pass");
            constexpr int NI = C * C / NT;
            const int s = tid % C, t0r = tid / C;
            const float csv = cc[s];
            float cmv[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int t = t0r + (NT / C) * i;
                cmv[i] = t > 0 ? cc[t - 1] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int t = t0r + (NT / C) * i;
                sm.f.dm[t * PC + s] = f32_to_bf16(s < t ? __builtin_amdgcn_exp2f(cmv[i] - csv) : 0.f);
            }
        }
    }
    lds_barrier();
    // dq = diag(eg) (dO S_in^T) + (D o A) K; dk = diag(el) (U dS_out^T) - diag(beta eg)
    // (dU S_in^T) + (D o A)^T Q - Mb K - Mb^T K (rows 16 w ..)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[nt][e] *= egr[e];   // dk1 took its row factors on the way in
#pragma unroll
    for (int kc = 0; kc < C / 32; ++kc) {
        const bf16x8_t aad = frag_kr(sm.f.adT, PC, 32 * kc, 16 * w, lane);
        const bf16x8_t aadt = frag_kc(sm.f.adT, PC, 16 * w, 32 * kc, lane);
        const bf16x8_t amb = frag_kr(sm.f.mbT, PC, 32 * kc, 16 * w, lane);
        const bf16x8_t ambt = frag_kc(sm.f.mbT, PC, 16 * w, 32 * kc, lane);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8_t bk = frag_kr(sm.k, PQ, 32 * kc, 16 * nt, lane);
            const bf16x8_t bq = frag_kr(sm.q, PQ, 32 * kc, 16 * nt, lane);
            dq[nt] = mfma16(aad, bk, dq[nt]);
            dk1[nt] = mfma16(aadt, bq, dk1[nt]);
            dk1[nt] = mfma16(amb, bk, dk1[nt]);
            dk1[nt] = mfma16(ambt, bk, dk1[nt]);
        }
    }
    {   // rows past the sequence's end fall outside the resources and are dropped
        const rsrc_t rdq = make_rsrc(a.dq + tok * DK, uint32_t(n) * DK * 2u);
        const rsrc_t rdk = make_rsrc(a.dk + tok * DK, uint32_t(n) * DK * 2u);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t o = uint32_t((16 * w + 4 * g + e) * DK + 16 * nt + jl) * 2u;
                buf_st2(rdq, o, f32_to_bf16(dq[nt][e]));
                buf_st2(rdk, o, f32_to_bf16(dk1[nt][e]));
            }
        }
    }
    {   // Z1 = H1 Dm^T, Z2 = H2 Dm^T (rows x = 16 w ..), weighted and summed over x
        f32x4_t z1[4], z2[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) z1[nt] = z2[nt] = zero4();
#pragma unroll
        for (int kc = 0; kc < C / 32; ++kc) {
            const bf16x8_t ah1 = frag_kr(sm.f.h1T, PC, 32 * kc, 16 * w, lane);
            const bf16x8_t ah2 = frag_kr(sm.f.h2T, PC, 32 * kc, 16 * w, lane);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8_t bdm = frag_kc(sm.f.dm, PC, 16 * nt, 32 * kc, lane);
                z1[nt] = mfma16(ah1, bdm, z1[nt]);
                z2[nt] = mfma16(ah2, bdm, z2[nt]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int t = 16 * nt + jl;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = 16 * w + 4 * g + e;
                if (x >= t) {
                    const float d = __builtin_amdgcn_exp2f(cr[e] - cs4[nt]);
                    part += d * z1[nt][e];
                    if (x > t) part -= d * br[e] * z2[nt][e];
                }
            }
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (g == 0) sm.zw[w][t] = part;
        }
    }
    lds_barrier();
    if (tid < n) {
        const int t = tid;
        const float ct = cc[t], cm = t > 0 ? cc[t - 1] : 0.f;
        const float gm = __builtin_amdgcn_exp2f(cm), el = __builtin_amdgcn_exp2f(cl - ct);
        // s1 = sum_{x<t} 2^(c_{t-1} - c_x) kap_x and s2 = sum_{x>=t} 2^(c_x - c_t) (rho_x -
        // [x > t] beta_x mu_x), in increasing x, as one unrolled pass of 16-byte broadcast
        // reads (a loop with a data-dependent trip count waits on every read)
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int x4 = 0; x4 < C; x4 += 4) {
            const float4 c4 = *reinterpret_cast<const float4*>(cc + x4);
            const float4 k4 = *reinterpret_cast<const float4*>(sm.kap + x4);
            const float4 r4 = *reinterpret_cast<const float4*>(sm.rho + x4);
            const float4 m4 = *reinterpret_cast<const float4*>(sm.mu + x4);
            const float4 b4 = *reinterpret_cast<const float4*>(bb + x4);
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w},
                        rv[4] = {r4.x, r4.y, r4.z, r4.w}, mv[4] = {m4.x, m4.y, m4.z, m4.w},
                        bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = x4 + i;
                const float d = __builtin_amdgcn_exp2f(x < t ? cm - cv[i] : cv[i] - ct);
                if (x < t) s1 += d * kv[i];
                else s2 += d * (rv[i] - (x > t ? bv[i] * mv[i] : 0.f));
            }
        }
        static_assert(NT == 256, "four waves");
        const float zt = ((sm.zw[0][t] + sm.zw[1][t]) + sm.zw[2][t]) + sm.zw[3][t];
        const float sg = ((sm.sig[0] + sm.sig[1]) + sm.sig[2]) + sm.sig[3];
        const float da = el * s1 + gm * s2 + zt + el * gm * sg - bb[t] * (gm * sm.mu[t] + sm.dup[t]);
        const float db = sm.vdu[t] - __builtin_amdgcn_exp2f(ct) * sm.mu[t] - sm.dbp[t];
        store_gate<GB>(a.dg, tok + t, da);
        store_gate<GB>(a.dbeta, tok + t, db);
    }
}

struct GbLayout {
    size_t S, dS, T, P, total;
};
GbLayout gb_layout(const Problem& p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t nseq = size_t(p.B) * p.H, nch = size_t((p.N + C - 1) / C);
    GbLayout L{};
    size_t off = 0;
    L.S = off; off += al(nseq * nch * size_t(p.dv) * DK * 2);
    L.dS = off; off += al(nseq * nch * size_t(p.dv) * DK * 2);
    L.T = off; off += al(nseq * nch * C * C * 2);
    L.P = off; off += al(nseq * nch * C * C * 2);
    L.total = off;
    return L;
}

template <bool GB, int DV>
hipError_t launch_gdv(const Problem& p, const GbArgs& a) {
    const unsigned units = unsigned(size_t(a.nseq) * a.nch);
    gdn_bwd_prep_mfma<GB><<<dim3(units), dim3(NT), 0, p.stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_bwd_chain_mfma<GB, DV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(ChainSmem)));
    if (e != hipSuccess) return e;
    const unsigned chains = unsigned(2 * a.nseq * (DV / VT));
    gdn_bwd_chain_mfma<GB, DV><<<dim3(chains), dim3(NT), sizeof(ChainSmem), p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_bwd_grads_mfma<GB, DV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(GradSmem)));
    if (e != hipSuccess) return e;
    gdn_bwd_grads_mfma<GB, DV><<<dim3(units), dim3(NT), sizeof(GradSmem), p.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool gdn_backward_mfma_supported(const Problem& p) {
    return p.variant == LA_GDN && p.io_bf16 && p.dk == DK && (p.dv == 64 || p.dv == 128);
}

size_t gdn_backward_mfma_workspace_bytes(const Problem& p) {
    if (p.N == 0 || p.B == 0 || p.H == 0) return 0;
    return gb_layout(p).total;
}

hipError_t launch_backward_gdn_mfma(const BwdProblem& bp) {
    const Problem& p = bp.p;
    const size_t nseq = size_t(p.B) * p.H, nch = size_t((p.N + C - 1) / C);
    if (nseq * nch > 0x7fffffffull || 2 * nseq * size_t(p.dv / VT) > 0x7fffffffull)
        return hipErrorInvalidValue;
    const GbLayout L = gb_layout(p);
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    GbArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dO = static_cast<const uint16_t*>(bp.dO);
    a.g = p.g;
    a.beta = p.beta;
    a.S0 = p.S0;
    a.dSf = bp.dS_final;
    a.dq = static_cast<uint16_t*>(bp.dq);
    a.dk = static_cast<uint16_t*>(bp.dk);
    a.dv = static_cast<uint16_t*>(bp.dv);
    a.dg = bp.dg;
    a.dbeta = bp.dbeta;
    a.dS0 = bp.dS0;
    a.Sck = reinterpret_cast<uint16_t*>(ws + L.S);
    a.dSck = reinterpret_cast<uint16_t*>(ws + L.dS);
    a.Tck = reinterpret_cast<uint16_t*>(ws + L.T);
    a.Pck = reinterpret_cast<uint16_t*>(ws + L.P);
    a.N = p.N;
    a.nseq = int(nseq);
    a.nch = int(nch);
    if (p.dv == 128) return p.gate_bf16 ? launch_gdv<true, 128>(p, a) : launch_gdv<false, 128>(p, a);
    return p.gate_bf16 ? launch_gdv<true, 64>(p, a) : launch_gdv<false, 64>(p, a);
}

}  // namespace la
