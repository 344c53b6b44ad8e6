// Backward of the chunked Gated DeltaNet prefill ("线性注意力与 SSM", section GDN: the
// gated delta rule S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t =
// S_t^T q_t, key-major), in fp32 on the vector ALUs with chunk C = 16.
//
// Token form. With u_t = beta_t (v_t - alpha_t p_t), p_t = S_{t-1}^T k_t, and G_t the
// gradient of the loss with respect to S_t (everything downstream of token t, o_t included):
//   du_t = G_t^T k_t,  dv_t = beta_t du_t,  dbeta_t = du_t . (v_t - alpha_t p_t),
//   dq_t = S_t do_t,   dk_t = G_t u_t - alpha_t beta_t S_{t-1} du_t,
//   dalpha_t = <G_t, S_{t-1}> - beta_t du_t . p_t,
//   G_{t-1} = alpha_t (G_t - beta_t k_t du_t^T) + q_{t-1} do_{t-1}^T.
// The gate gradient is taken in this direct form. The log-domain alternative (a reverse
// cumulative sum of dL/dlog alpha, divided by alpha) cancels down to O(alpha) and loses
// fp32 accuracy by 1/alpha.
//
// Chunk form. Inside a chunk with cumulative log gates c_r (base 2 here), D_rs = 2^(c_r -
// c_s) for s <= r, L_rs = beta_r D_rs k_r.k_s (s < r), P_rs = D_rs q_r.k_s (s <= r),
// entering state S0 and leaving-state gradient dS':
//   U  = (I + L)^-1 X,     X_r = beta_r (v_r - 2^c_r S0^T k_r)          (the forward's U)
//   dU = (I + L)^-T R,     R_s = 2^(c_last - c_s) dS'^T k_s + sum_{r>=s} P_rs do_r
// (dU is du of every token: the unrolled G_t, dotted with k_t, is this triangular system),
//   S_t = 2^c_t S0 + sum_{s<=t} D_ts k_s u_s^T,
//   G_t = 2^(c_last-c_t) dS' + sum_{r>=t} D_rt q_r do_r^T - sum_{s>t} D_st beta_s k_s du_s^T.
// Substituting these into the token form turns every gradient into sums, with weights
// that are products of decays (all <= 1), over the chunk's rows of the value-column dot
// products A_rs = do_r.u_s, B_rs = du_r.u_s, kappa_s = (dS'^T k_s).u_s, rho_r = (S0^T
// q_r).do_r, mu_s = (S0^T k_s).du_s, sigma = <dS', S0>, and of d_k-vectors such as S0 do_t.
//
// Kernels: a prep kernel forms every chunk's T = (I + L)^-1 and P in parallel; then one
// launch runs both chains, each workgroup one (sequence, value tile of up to 64 columns),
// with U = T X and dU = T^T R as small products (value columns never mix in either
// recurrence): the forward chain writes the state entering every chunk, the reverse chain
// the gradient leaving it (dS_in = 2^c_last dS' + sum_r 2^c_r q_r do_r^T - sum_s beta_s
// 2^c_s k_s du_s^T), and dS0. Then the grads kernel takes every (sequence, chunk) in
// parallel, loops over 16-column value tiles accumulating the column sums, and writes
// final dq, dk, dv, dalpha and dbeta.
//
// KDA ("状态空间与线性注意力", section KDA: the decay Diag(alpha_t) applied first, then
// the delta write, with alpha_t per key dim) takes the same route with per-key-dim
// cumulative logs b_r[i]: every decay factor 2^(c_x - c_y) becomes the vector 2^(b_x - b_y)
// inside the key-dim sums (L_rs = beta_r sum_i k_ri k_si 2^(b_ri - b_si), X_r = beta_r (v_r
// - S0^T (k_r 2^b_r)), the state update Diag(2^b_last) S + sum_s (k_s 2^(b_last - b_s))
// u_s^T, and so on), p_t = S-bar_t^T k_t with S-bar_t = Diag(alpha_t) S_{t-1}, dk_t = G_t
// u_t - beta_t S-bar_t du_t, and the gate gradient per key dim, dalpha_t[i] = sum_j
// G_t[i,j] S_{t-1}[i,j] - beta_t k_t[i] (S_{t-1} du_t)[i], whose chunk form needs the
// d_k x C matrices S0 dO^T, dS' U^T and S0 dU^T besides A and B.
#include "common.hpp"
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int C = kValuChunk;  // 16
constexpr int VT = 16;         // value columns per tile
constexpr int NT = 256;        // = C * VT = C * C
static_assert(C * VT == NT && C * C == NT, "thread maps assume 16 x 16");

struct GdnBwdArgs {
    const void *q, *k, *v, *g, *beta, *dO;
    const float *S0, *dSf;
    void *dq, *dk, *dv, *dg, *dbeta;
    float* dS0;
    float* Sck;    // [nseq][nchunks][DK][DV] state entering each chunk
    float* dSck;   // [nseq][nchunks][DK][DV] gradient of the state leaving each chunk
    float* Tck;    // [nseq][nchunks][C][C] T = (I + L)^-1 of each chunk
    float* Pck;    // [nseq][nchunks][C][C] P of each chunk (lower triangle with diagonal)
    int N, nseq, ntiles, nchunks;
    int io_bf16, gate_bf16;
};

// The rows of one chunk shared by both kernels: k (and q), the cumulative base-2 log gate,
// beta and the decay factors. Rows past the end are zero with gate 1 and beta 0, which
// makes them identity steps.
template <int DK>
struct Rows {
    alignas(16) float q[C][DK + 4];
    alignas(16) float k[C][DK + 4];
    float c[C], b[C];
    float eg[C];    // 2^c_r (decay from the chunk start through row r)
    float el[C];    // 2^(c_last - c_r) (decay after row r to the chunk end)
};

template <int DK, bool WQ>
__device__ __forceinline__ void load_rows(Rows<DK>& sm, const GdnBwdArgs& a, size_t tok, int n) {
    const int tid = threadIdx.x;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        const size_t e = (tok + r) * DK + i;
        sm.k[r][i] = r < n ? load_elem(a.k, e, iob) : 0.f;
        if (WQ) sm.q[r][i] = r < n ? load_elem(a.q, e, iob) : 0.f;
    }
    if (tid < kWave) {   // one wave: the log gates, their prefix sums, beta
        const int r = tid;
        float lg = 0.f, bt = 0.f;
        if (r < n) {
            lg = __builtin_amdgcn_logf(load_elem(a.g, tok + r, gb));
            bt = load_elem(a.beta, tok + r, gb);
        }
        const float cs = wave_inclusive_scan(r < C ? lg : 0.f);
        const float cl = __shfl(cs, C - 1);
        if (r < C) {
            sm.c[r] = cs;
            sm.b[r] = bt;
            sm.eg[r] = __builtin_amdgcn_exp2f(cs);
            sm.el[r] = __builtin_amdgcn_exp2f(cl - cs);
        }
    }
}


// Triangular solves for one value column, the solved rows kept in registers (an LDS round
// trip per step would put its latency on every row): forward substitution (I + L) u = x
// and back substitution (I + L)^T u = x, L strictly lower with row pitch C + 1.
__device__ __forceinline__ void solve_lower(const float (*L)[C + 1], const float (*x)[VT],
                                            float (*u)[VT], int j) {
    float w[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
        float acc = x[r][j];
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= L[r][s] * w[s];
        w[r] = acc;
        u[r][j] = acc;
    }
}
__device__ __forceinline__ void solve_upper_t(const float (*L)[C + 1], const float (*x)[VT],
                                              float (*u)[VT], int j) {
    float w[C];
#pragma unroll
    for (int s = C - 1; s >= 0; --s) {
        float acc = x[s][j];
#pragma unroll
        for (int r = s + 1; r < C; ++r) acc -= L[r][s] * w[r];
        w[s] = acc;
        u[s][j] = acc;
    }
}


// ---------------------------------------------------------------------------- prep
// T = (I + L)^-1 (unit lower triangular) by forward substitution on the unit vectors, one
// column per thread, and P, for every (sequence, chunk) in parallel.
__device__ __forceinline__ void store_t_and_p(const float (*L)[C + 1], float p, float* Tg,
                                              float* Pg) {
    const int tid = threadIdx.x;
    Pg[tid] = p;   // thread (r, s) = (tid / C, tid % C)
    if (tid < C) {
        const int j = tid;
        float w[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float acc = r == j ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) acc -= L[r][s2] * w[s2];
            w[r] = acc;
            Tg[r * C + j] = acc;
        }
    }
}

template <int DK>
struct PrepSmem {
    Rows<DK> rw;
    float L[C][C + 1];
};

template <int DK>
__global__ __launch_bounds__(NT) void gdn_bwd_prep_kernel(GdnBwdArgs a) {
    __shared__ PrepSmem<DK> sm;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0);
    load_rows<DK, true>(sm.rw, a, seq * size_t(a.N) + t0, n);
    __syncthreads();
    const int r = threadIdx.x / C, s2 = threadIdx.x % C;
    float kk = 0.f, qk = 0.f;
    for (int i = 0; i < DK; ++i) {
        kk += sm.rw.k[r][i] * sm.rw.k[s2][i];
        qk += sm.rw.q[r][i] * sm.rw.k[s2][i];
    }
    const float d = s2 <= r ? __builtin_amdgcn_exp2f(sm.rw.c[r] - sm.rw.c[s2]) : 0.f;
    sm.L[r][s2] = s2 < r ? sm.rw.b[r] * d * kk : 0.f;
    __syncthreads();
    const size_t off = (seq * a.nchunks + ch) * size_t(C * C);
    store_t_and_p(sm.L, d * qk, a.Tck + off, a.Pck + off);
}

// ---------------------------------------------------------------------------- chains
// Both chains of GDN and KDA. Each workgroup walks one (sequence, CT-column value tile) in
// order (CT = 32 where d_v allows: one chunk's keys and queries then serve 32 columns; at
// most 128 registers, so two such workgroups share a CU and every chain stays resident), forward for the states entering the chunks or in reverse for the gradients leaving
// them. The tile stays in registers: thread (g, j) holds rows g*RG .. g*RG+RG-1 of column j.
// Per chunk: the rows' partial dot products with the chunk's (decayed) keys go through a
// padded LDS buffer to give k_t . S[:, j]; then the right-hand side, U = T X (or dU = T^T R),
// and the update of the thread's own rows from the keys (and queries) read as broadcast rows.
template <int VAR, int DK, int CT>
struct ChainSmem {
    static constexpr bool PK = VAR == LA_KDA;   // a decay per key dim
    static constexpr int KP = DK + 4;           // row pitch: 16-byte aligned rows
    float k[C][KP];   // GDN k; KDA k 2^b (after the table step)
    float q[C][KP];   // reverse: GDN q; KDA q 2^b
    float kt[PK ? C : 1][PK ? KP : 1];   // KDA: k 2^(b_last - b)
    union {
        float bq[PK ? C : 1][PK ? KP : 1];   // KDA: cumulative base-2 log gates
        float red[C][16 * CT + 32];          // partials over the 16 row groups (padded rows)
    } w;
    float T[C][C + 1], P[C][C + 1];
    float x[C][CT], rhs[C][CT], u[C][CT];
    float eg[C], el[C], b[C];   // GDN 2^c_r, 2^(c_last - c_r); beta
    float dl[PK ? DK : 1];      // KDA 2^b_last per key dim
};

template <int VAR, int DK, int DV, int CT>
__global__ __launch_bounds__(16 * CT, CT >= 32 ? 4 : 2) void bwd_chains_kernel(GdnBwdArgs a) {
    constexpr bool PK = VAR == LA_KDA;
    constexpr int RG = DK / 16;   // rows per thread
    constexpr int NTC = 16 * CT;  // threads: 16 row groups x CT columns
    static_assert(DK % 16 == 0 && DV % CT == 0 && NTC >= C * C, "16 row groups");
    __shared__ ChainSmem<VAR, DK, CT> sm;
    const int tid = threadIdx.x;
    constexpr int ntiles = DV / CT;
    const int nfw = a.nseq * ntiles;
    const bool rev = int(blockIdx.x) >= nfw;
    const int unit = rev ? int(blockIdx.x) - nfw : int(blockIdx.x);
    const size_t seq = size_t(unit / ntiles);
    const int c0 = (unit % ntiles) * CT;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    const int grp = tid / CT, j = tid % CT, i0 = grp * RG;   // this thread's rows and column
    const int t_me = tid / CT;                                // row of the (t, j) maps
    const size_t sbase = seq * DK * DV;
    const float* init = rev ? a.dSf : a.S0;
    float S[RG];
#pragma unroll
    for (int m = 0; m < RG; ++m) S[m] = init ? init[sbase + size_t(i0 + m) * DV + c0 + j] : 0.f;
    float* ck = (rev ? a.dSck : a.Sck) + seq * size_t(a.nchunks) * DK * DV;
    // A chunk's inputs are fetched into registers one chunk ahead (storage types fixed once,
    // rows past the end read as the last row and zeroed when staged), so the chain waits on
    // them only while the previous chunk computes.
    constexpr int NLK = (C * DK + NTC - 1) / NTC;
    float rk[NLK] = {}, rq[NLK] = {}, rg[NLK] = {};
    float rlg = 1.f, rbt = 0.f, rx = 0.f, rT = 0.f, rP = 0.f;
    auto fetch = [&](int ch) {
        const int nl = min(C, a.N - ch * C) - 1;   // >= 0
        const size_t tok = seq * size_t(a.N) + size_t(ch) * C;
        auto io = [&](auto tag, auto rv) {
            using T = decltype(tag);
            constexpr bool R = decltype(rv)::value;
#pragma unroll
            for (int m = 0; m < NLK; ++m) {
                const int idx = tid + NTC * m;
                if (idx < C * DK) {
                    const size_t e = (tok + min(idx / DK, nl)) * DK + idx % DK;
                    rk[m] = ld<T>(a.k, e);
                    if (R) rq[m] = ld<T>(a.q, e);
                }
            }
            rx = ld<T>(R ? a.dO : a.v, (tok + min(t_me, nl)) * DV + c0 + j);
        };
        auto gates = [&](auto tag) {
            using T = decltype(tag);
            if (PK) {
#pragma unroll
                for (int m = 0; m < NLK; ++m) {
                    const int idx = tid + NTC * m;
                    if (idx < C * DK) rg[m] = ld<T>(a.g, (tok + min(idx / DK, nl)) * DK + idx % DK);
                }
            } else if (tid < C) {
                rlg = ld<T>(a.g, tok + min(tid, nl));
            }
            if (tid < C) rbt = ld<T>(a.beta, tok + min(tid, nl));
        };
        if (iob) {
            if (rev) io(uint16_t{}, std::true_type{});
            else io(uint16_t{}, std::false_type{});
        } else {
            if (rev) io(float{}, std::true_type{});
            else io(float{}, std::false_type{});
        }
        if (gb) gates(uint16_t{});
        else gates(float{});
        if (tid < C * C) {
            const size_t off = (seq * a.nchunks + ch) * size_t(C * C);
            rT = a.Tck[off + tid];
            if (rev) rP = a.Pck[off + tid];
        }
    };
    fetch(rev ? a.nchunks - 1 : 0);
    for (int it = 0; it < a.nchunks; ++it) {
        const int ch = rev ? a.nchunks - 1 - it : it;
        const int t0 = ch * C, n = min(C, a.N - t0);
        __syncthreads();   // the previous chunk's readers are done
        float* ckc = ck + size_t(ch) * DK * DV;
#pragma unroll
        for (int m = 0; m < RG; ++m) ckc[size_t(i0 + m) * DV + c0 + j] = S[m];
#pragma unroll
        for (int m = 0; m < NLK; ++m) {
            const int idx = tid + NTC * m;
            if (idx < C * DK) {
                const int r = idx / DK, i = idx % DK;
                const bool in = r < n;
                sm.k[r][i] = in ? rk[m] : 0.f;
                if (rev) sm.q[r][i] = in ? rq[m] : 0.f;
                if (PK) sm.w.bq[r][i] = in ? __builtin_amdgcn_logf(rg[m]) : 0.f;
            }
        }
        if (!PK) {
            if (tid < kWave) {   // one wave: log gates, their prefix sums, beta
                const int r = tid;
                float lg = 0.f, bt = 0.f;
                if (r < n) {
                    lg = __builtin_amdgcn_logf(rlg);
                    bt = rbt;
                }
                const float cs = wave_inclusive_scan(r < C ? lg : 0.f);
                const float cl = __shfl(cs, C - 1);
                if (r < C) {
                    sm.b[r] = bt;
                    sm.eg[r] = __builtin_amdgcn_exp2f(cs);
                    sm.el[r] = __builtin_amdgcn_exp2f(cl - cs);
                }
            }
        } else if (tid < C) {
            sm.b[tid] = tid < n ? rbt : 0.f;
        }
        sm.x[t_me][j] = t_me < n ? rx : 0.f;
        if (tid < C * C) {
            sm.T[tid / C][tid % C] = rT;
            if (rev) sm.P[tid / C][tid % C] = rP;
        }
        if (it + 1 < a.nchunks) fetch(rev ? ch - 1 : ch + 1);
        __syncthreads();
        if (PK) {   // prefix sums per key dim, then the decayed key (and query) rows
            for (int i = tid; i < DK; i += NTC) {
                float acc = 0.f;
                for (int r = 0; r < C; ++r) {
                    acc += sm.w.bq[r][i];
                    sm.w.bq[r][i] = acc;
                }
                sm.dl[i] = __builtin_amdgcn_exp2f(acc);
            }
            __syncthreads();
            for (int idx = tid; idx < C * DK; idx += NTC) {   // each element owned by one thread
                const int r = idx / DK, i = idx % DK;
                const float br = sm.w.bq[r][i], eb = __builtin_amdgcn_exp2f(br);
                const float kv = sm.k[r][i];
                sm.kt[r][i] = kv * __builtin_amdgcn_exp2f(sm.w.bq[C - 1][i] - br);
                sm.k[r][i] = kv * eb;
                if (rev) sm.q[r][i] *= eb;
            }
            __syncthreads();
        }
        {   // partial k_t . S[:, j] over this thread's rows, for every row t of the chunk
            constexpr int KP = ChainSmem<VAR, DK, CT>::KP;
            const float* kk = (PK && rev) ? &sm.kt[0][0] : &sm.k[0][0];
#pragma unroll
            for (int t = 0; t < C; ++t) {
                float p = 0.f;
#pragma unroll
                for (int m = 0; m < RG; ++m) p += kk[t * KP + i0 + m] * S[m];
                sm.w.red[t][grp * CT + j] = p;
            }
        }
        __syncthreads();
        {   // thread (t, j): the right-hand side
            const int t = t_me;
            float ks = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < 16; ++g2) ks += sm.w.red[t][g2 * CT + j];
            float rhs;
            if (!rev) {
                rhs = sm.b[t] * (sm.x[t][j] - (PK ? ks : sm.eg[t] * ks));
            } else {
                rhs = PK ? ks : sm.el[t] * ks;
                for (int r = t; r < C; ++r) rhs += sm.P[r][t] * sm.x[r][j];
            }
            sm.rhs[t][j] = rhs;
        }
        __syncthreads();
        {   // U = T X (forward) or dU = T^T R (reverse)
            const int t = t_me;
            float acc = 0.f;
            if (!rev) {
                for (int s2 = 0; s2 <= t; ++s2) acc += sm.T[t][s2] * sm.rhs[s2][j];
            } else {
                for (int r = t; r < C; ++r) acc += sm.T[r][t] * sm.rhs[r][j];
            }
            sm.u[t][j] = acc;
        }
        __syncthreads();
        {   // the update of this thread's rows
            float acc[RG];
#pragma unroll
            for (int m = 0; m < RG; ++m) acc[m] = 0.f;
            if (!rev) {
#pragma unroll 4
                for (int s2 = 0; s2 < C; ++s2) {
                    const float us = PK ? sm.u[s2][j] : sm.u[s2][j] * sm.el[s2];
#pragma unroll
                    for (int m = 0; m < RG; ++m) acc[m] += (PK ? sm.kt[s2][i0 + m] : sm.k[s2][i0 + m]) * us;
                }
            } else {
#pragma unroll 4
                for (int r = 0; r < C; ++r) {
                    const float xs = PK ? sm.x[r][j] : sm.x[r][j] * sm.eg[r];
                    const float us = PK ? sm.b[r] * sm.u[r][j] : sm.b[r] * sm.eg[r] * sm.u[r][j];
#pragma unroll
                    for (int m = 0; m < RG; ++m) acc[m] += sm.q[r][i0 + m] * xs - sm.k[r][i0 + m] * us;
                }
            }
#pragma unroll
            for (int m = 0; m < RG; ++m) S[m] = (PK ? sm.dl[i0 + m] : sm.eg[C - 1]) * S[m] + acc[m];
        }
    }
    if (rev) {
#pragma unroll
        for (int m = 0; m < RG; ++m) a.dS0[sbase + size_t(i0 + m) * DV + c0 + j] = S[m];
    }
}

// ---------------------------------------------------------------------------- grads
template <int DK>
struct GradSmem {
    Rows<DK> rw;
    float gm[C];                 // 2^c_{t-1} (1 for the first row)
    float D[C][C + 1];           // 2^(c_r - c_s), s <= r; 0 above
    float Dm[C][C + 1];          // 2^(c_{t-1} - c_s), s < t; 0 elsewhere
    float KK[C][C + 1], QK[C][C + 1], L[C][C + 1];
    alignas(16) float S0[DK][VT + 4];   // 16-byte aligned rows
    alignas(16) float dS[DK][VT + 4];
    alignas(16) float v[C][VT];
    alignas(16) float dO[C][VT];
    alignas(16) float U[C][VT];
    alignas(16) float dU[C][VT];
    // K dS_out and Q S_in land in X and R: thread (t, j) reads its own element of each
    // into a register before it writes X[t][j] and R[t][j], and nothing reads them later
    float KS[C][VT], X[C][VT], R[C][VT];
    float A[C][C + 1], Bm[C][C + 1];
    float kap[C], rho[C], mu[C], dup[C];
    float sig[NT / kWave];
};

// Dot product of two 16-float LDS rows (16-byte aligned) read as float4.
__device__ __forceinline__ float dot16(const float* x, const float* y) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
        const float4 a = *reinterpret_cast<const float4*>(x + c);
        const float4 b = *reinterpret_cast<const float4*>(y + c);
        acc += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
    }
    return acc;
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1, 0xf, 0xf>(v);
    v += dpp_f<0x4E, 0xf, 0xf>(v);
    v += dpp_f<0x141, 0xf, 0xf>(v);
    v += dpp_f<0x140, 0xf, 0xf>(v);
    return v;
}

template <int DK, int DV>
__global__ __launch_bounds__(NT, 3) void gdn_bwd_grads_kernel(GdnBwdArgs a) {
    constexpr int MQ = C * DK / NT;   // (row, key dim) pairs per thread
    static_assert(MQ >= 1 && (C * DK) % NT == 0, "d_k >= 16");
    __shared__ GradSmem<DK> sm;
    const int tid = threadIdx.x;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok = seq * size_t(a.N) + t0;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    const int r_me = tid / C, x_me = tid % C;   // (row, column) of the 16 x 16 maps
    load_rows<DK, true>(sm.rw, a, tok, n);
    __syncthreads();
    {
        const int r = r_me, s = x_me;
        float kk = 0.f, qk = 0.f;
        for (int i = 0; i < DK; ++i) {
            kk += sm.rw.k[r][i] * sm.rw.k[s][i];
            qk += sm.rw.q[r][i] * sm.rw.k[s][i];
        }
        const float d = s <= r ? __builtin_amdgcn_exp2f(sm.rw.c[r] - sm.rw.c[s]) : 0.f;
        const float cm = r > 0 ? sm.rw.c[r - 1] : 0.f;
        sm.D[r][s] = d;
        sm.Dm[r][s] = s < r ? __builtin_amdgcn_exp2f(cm - sm.rw.c[s]) : 0.f;
        sm.KK[r][s] = kk;
        sm.QK[r][s] = qk;
        sm.L[r][s] = s < r ? sm.rw.b[r] * d * kk : 0.f;
        if (s == 0) sm.gm[r] = r > 0 ? sm.rw.eg[r - 1] : 1.f;
    }
    float accq[MQ], acck[MQ];
#pragma unroll
    for (int m = 0; m < MQ; ++m) accq[m] = acck[m] = 0.f;
    float A_acc = 0.f, B_acc = 0.f;                            // (r_me, x_me)
    float kap = 0.f, rho = 0.f, mu = 0.f, dbt = 0.f, dup = 0.f;  // row r_me (lane x_me == 0)
    float sig = 0.f;
    const size_t ckoff = (seq * a.nchunks + ch) * size_t(DK) * DV;
    // the next tile's state tiles, v and dO are loaded into registers while this one works
    constexpr int MS = DK * VT / NT;
    float pS0[MS], pdS[MS], pv, pdO;
    auto fetch = [&](int tile) {
        const int c0 = tile * VT;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = tid + NT * m, i = idx / VT, j = idx % VT;
            const size_t e = ckoff + size_t(i) * DV + c0 + j;
            pS0[m] = a.Sck[e];
            pdS[m] = a.dSck[e];
        }
        const size_t e = (tok + r_me) * DV + c0 + x_me;
        pv = r_me < n ? load_elem(a.v, e, iob) : 0.f;
        pdO = r_me < n ? load_elem(a.dO, e, iob) : 0.f;
    };
    fetch(0);
    for (int tile = 0; tile < a.ntiles; ++tile) {
        const int c0 = tile * VT;
        lds_barrier();   // the previous tile's readers are done (loads stay in flight)
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = tid + NT * m, i = idx / VT, j = idx % VT;
            sm.S0[i][j] = pS0[m];
            sm.dS[i][j] = pdS[m];
            sig += pS0[m] * pdS[m];
        }
        sm.v[r_me][x_me] = pv;
        sm.dO[r_me][x_me] = pdO;
        if (tile + 1 < a.ntiles) fetch(tile + 1);
        lds_barrier();
        {
            // K S_in, K dS_out and Q S_in (16 x d_k by d_k x 16) on the fp32 matrix cores,
            // one product per wave, two interleaved accumulators. Lane layout of the
            // 16x16x4 fp32 MFMA (g = lane / 16, jl = lane % 16): A (16 x 4) row jl, k = g;
            // B (4 x 16) column jl, k = g; D (16 x 16) column jl, rows 4g .. 4g + 3.
            const int w = tid / kWave, l = tid % kWave, g = l >> 4, jl = l & 15;
            if (w < 3) {
                const float* Ar = w == 2 ? &sm.rw.q[jl][0] : &sm.rw.k[jl][0];
                const float(*Bt)[VT + 4] = w == 1 ? sm.dS : sm.S0;
                f32x4_t c0v = {0.f, 0.f, 0.f, 0.f}, c1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
                for (int kk = 0; kk < DK; kk += 8) {
                    c0v = __builtin_amdgcn_mfma_f32_16x16x4f32(Ar[kk + g], Bt[kk + g][jl], c0v, 0, 0, 0);
                    c1v = __builtin_amdgcn_mfma_f32_16x16x4f32(Ar[kk + 4 + g], Bt[kk + 4 + g][jl],
                                                                c1v, 0, 0, 0);
                }
                float(*Out)[VT] = w == 0 ? sm.KS : (w == 1 ? sm.X : sm.R);   // KS, K dS_out, Q S_in
#pragma unroll
                for (int r = 0; r < 4; ++r) Out[4 * g + r][jl] = c0v[r] + c1v[r];
            }
        }
        lds_barrier();
        const int t = r_me, j = x_me;
        const float ks = sm.KS[t][j], kds = sm.X[t][j], qs = sm.R[t][j];
        {
            float r_ = sm.rw.el[t] * kds;
            for (int r = t; r < C; ++r) r_ += sm.D[r][t] * sm.QK[r][t] * sm.dO[r][j];
            sm.X[t][j] = sm.rw.b[t] * (sm.v[t][j] - sm.rw.eg[t] * ks);
            sm.R[t][j] = r_;
        }
        lds_barrier();
        if (tid < VT) solve_lower(sm.L, sm.X, sm.U, tid);   // U, one column per thread
        else if (tid >= kWave && tid < kWave + VT)          // dU, on another wave
            solve_upper_t(sm.L, sm.R, sm.dU, tid - kWave);
        lds_barrier();
        {
            const float u = sm.U[t][j], du = sm.dU[t][j];
            float p = sm.gm[t] * ks, ap = sm.rw.eg[t] * ks;
            for (int s = 0; s < t; ++s) {
                const float ku = sm.KK[t][s] * sm.U[s][j];
                p += sm.Dm[t][s] * ku;
                ap += sm.D[t][s] * ku;
            }
            if (t < n) store_elem(a.dv, (tok + t) * DV + c0 + j, sm.rw.b[t] * du, iob);
            const float s_kap = row16_sum(kds * u), s_rho = row16_sum(qs * sm.dO[t][j]);
            const float s_mu = row16_sum(ks * du), s_db = row16_sum(du * (sm.v[t][j] - ap));
            const float s_dup = row16_sum(du * p);
            kap += s_kap; rho += s_rho; mu += s_mu; dbt += s_db; dup += s_dup;
            A_acc += dot16(sm.dO[r_me], sm.U[x_me]);   // (r_me, x_me) = (r, s)
            B_acc += dot16(sm.dU[r_me], sm.U[x_me]);
        }
        {   // this thread's key dim i is the same for every m: its S0 and dS rows once
            const int i = tid % DK;
#pragma unroll
            for (int m = 0; m < MQ; ++m) {
                const int tt = (tid + NT * m) / DK;
                const float so = dot16(sm.S0[i], sm.dO[tt]);
                const float su = dot16(sm.dS[i], sm.U[tt]);
                const float sdu = dot16(sm.S0[i], sm.dU[tt]);
                accq[m] += sm.rw.eg[tt] * so;
                acck[m] += sm.rw.el[tt] * su - sm.rw.b[tt] * sm.rw.eg[tt] * sdu;
            }
        }
    }
    // the column sums over all tiles
    sm.A[r_me][x_me] = A_acc;
    sm.Bm[r_me][x_me] = B_acc;
    if (x_me == 0) {
        sm.kap[r_me] = kap;
        sm.rho[r_me] = rho;
        sm.mu[r_me] = mu;
        sm.dup[r_me] = dup;
        if (r_me < n) store_elem(a.dbeta, tok + r_me, dbt, gb);
    }
    sig = wave_sum(sig);
    if ((tid & (kWave - 1)) == 0) sm.sig[tid / kWave] = sig;
    __syncthreads();
    {   // dalpha: thread (t, x) takes the terms of row / column x, summed over the 16 lanes
        const int t = r_me, x = x_me;
        const float gm = sm.gm[t];
        float term = 0.f;
        if (x < t) term += sm.rw.el[t] * sm.Dm[t][x] * sm.kap[x];
        if (x >= t) {
            float in = gm * sm.rho[x];
            for (int s = 0; s < t; ++s) in += sm.Dm[t][s] * sm.QK[x][s] * sm.A[x][s];
            term += sm.D[x][t] * in;
        }
        if (x > t) {
            float in = gm * sm.mu[x];
            for (int s = 0; s < t; ++s) in += sm.Dm[t][s] * sm.KK[x][s] * sm.Bm[x][s];
            term -= sm.D[x][t] * sm.rw.b[x] * in;
        }
        term = row16_sum(term);
        if (x == 0 && t < n) {
            float sg = 0.f;
            for (int w = 0; w < NT / kWave; ++w) sg += sm.sig[w];
            const float da = term + sm.rw.el[t] * gm * sg - sm.rw.b[t] * sm.dup[t];
            store_elem(a.dg, tok + t, da, gb);
        }
    }
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
        const int idx = tid + NT * m, t = idx / DK, i = idx % DK;
        float dq = accq[m], dk = acck[m];
        for (int s = 0; s <= t; ++s) dq += sm.D[t][s] * sm.A[t][s] * sm.rw.k[s][i];
        for (int r = t; r < C; ++r) dk += sm.D[r][t] * sm.A[r][t] * sm.rw.q[r][i];
        for (int s = t + 1; s < C; ++s) dk -= sm.D[s][t] * sm.Bm[s][t] * sm.rw.b[s] * sm.rw.k[s][i];
        float bk = 0.f;
        for (int s = 0; s < t; ++s) bk += sm.D[t][s] * sm.Bm[t][s] * sm.rw.k[s][i];
        dk -= sm.rw.b[t] * bk;
        if (t < n) {
            store_elem(a.dq, (tok + t) * DK + i, dq, iob);
            store_elem(a.dk, (tok + t) * DK + i, dk, iob);
        }
    }
}


// ---------------------------------------------------------------------------- KDA
// Rows of one chunk with a gate per key dim: cumulative base-2 logs bq (rows past the end
// have gate 1, so their logs repeat the last real row's).
template <int DK>
struct RowsK {
    alignas(16) float q[C][DK + 4];
    alignas(16) float k[C][DK + 4];
    float bq[C][DK + 1];
    float b[C];
};

template <int DK, bool WQ>
__device__ __forceinline__ void load_rows_kda(RowsK<DK>& sm, const GdnBwdArgs& a, size_t tok, int n) {
    const int tid = threadIdx.x;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        const size_t e = (tok + r) * DK + i;
        const bool in = r < n;
        sm.k[r][i] = in ? load_elem(a.k, e, iob) : 0.f;
        if (WQ) sm.q[r][i] = in ? load_elem(a.q, e, iob) : 0.f;
        sm.bq[r][i] = in ? __builtin_amdgcn_logf(load_elem(a.g, e, gb)) : 0.f;
    }
    if (tid < C) sm.b[tid] = tid < n ? load_elem(a.beta, tok + tid, gb) : 0.f;
    __syncthreads();
    for (int i = tid; i < DK; i += NT) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
            acc += sm.bq[r][i];
            sm.bq[r][i] = acc;
        }
    }
}


template <int DK>
struct PrepSmemK {
    RowsK<DK> rw;
    float L[C][C + 1];
};

template <int DK>
__global__ __launch_bounds__(NT) void kda_bwd_prep_kernel(GdnBwdArgs a) {
    __shared__ PrepSmemK<DK> sm;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0);
    load_rows_kda<DK, true>(sm.rw, a, seq * size_t(a.N) + t0, n);
    __syncthreads();
    const int r = threadIdx.x / C, s2 = threadIdx.x % C;
    float kk = 0.f, qk = 0.f;
    if (s2 <= r) {
        for (int i = 0; i < DK; ++i) {
            const float d = __builtin_amdgcn_exp2f(sm.rw.bq[r][i] - sm.rw.bq[s2][i]);
            kk += sm.rw.k[r][i] * sm.rw.k[s2][i] * d;
            qk += sm.rw.q[r][i] * sm.rw.k[s2][i] * d;
        }
    }
    sm.L[r][s2] = s2 < r ? sm.rw.b[r] * kk : 0.f;
    __syncthreads();
    const size_t off = (seq * a.nchunks + ch) * size_t(C * C);
    store_t_and_p(sm.L, qk, a.Tck + off, a.Pck + off);
}

template <int DK>
struct GradSmemK {
    RowsK<DK> rw;
    float L[C][C + 1], Lt[C][C + 1], P[C][C + 1], A[C][C + 1], Bm[C][C + 1];
    alignas(16) float v[C][VT];
    alignas(16) float dO[C][VT];
    alignas(16) float U[C][VT];
    alignas(16) float dU[C][VT];
    float KS[C][VT], X[C][VT], R[C][VT];
    float sig[DK];
    union {
        struct {   // the tile loop (16-byte aligned rows)
            alignas(16) float S0[DK][VT + 4];
            alignas(16) float dS[DK][VT + 4];
            alignas(16) float kd[C][DK + 4];
            alignas(16) float kt[C][DK + 4];
        } t;
        struct {   // after it: (S0 dO^T)^T, (dS' U^T)^T, (S0 dU^T)^T, rows by token
            float SDO[C][DK + 1], DSU[C][DK + 1], SDU[C][DK + 1];
        } f;
    } w;
};

template <int DK, int DV>
__global__ __launch_bounds__(NT) void kda_bwd_grads_kernel(GdnBwdArgs a) {
    constexpr int MQ = C * DK / NT;
    constexpr int MS = DK * VT / NT;   // state elements per thread in the tile loads
    static_assert(MQ >= 1 && (C * DK) % NT == 0 && MS >= 1, "d_k >= 16");
    __shared__ GradSmemK<DK> sm;
    const int tid = threadIdx.x;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok = seq * size_t(a.N) + t0;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    const int r_me = tid / C, x_me = tid % C;
    load_rows_kda<DK, true>(sm.rw, a, tok, n);
    __syncthreads();
    {
        const int r = r_me, s = x_me;
        float kk = 0.f, qk = 0.f;
        if (s <= r) {
            for (int i = 0; i < DK; ++i) {
                const float d = __builtin_amdgcn_exp2f(sm.rw.bq[r][i] - sm.rw.bq[s][i]);
                kk += sm.rw.k[r][i] * sm.rw.k[s][i] * d;
                qk += sm.rw.q[r][i] * sm.rw.k[s][i] * d;
            }
        }
        sm.Lt[r][s] = s < r ? kk : 0.f;
        sm.L[r][s] = s < r ? sm.rw.b[r] * kk : 0.f;
        sm.P[r][s] = qk;
    }
    float so[MQ], su[MQ], sdu[MQ], sg[MS];
#pragma unroll
    for (int m = 0; m < MQ; ++m) so[m] = su[m] = sdu[m] = 0.f;
#pragma unroll
    for (int m = 0; m < MS; ++m) sg[m] = 0.f;
    float A_acc = 0.f, B_acc = 0.f, dbt = 0.f;
    const size_t ckoff = (seq * a.nchunks + ch) * size_t(DK) * DV;
    // the next tile's state tiles, v and dO are loaded into registers while this one works
    float pS0[MS], pdS[MS], pv, pdO;
    auto fetch = [&](int tile) {
        const int c0 = tile * VT;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = tid + NT * m, i = idx / VT, j = idx % VT;
            const size_t e = ckoff + size_t(i) * DV + c0 + j;
            pS0[m] = a.Sck[e];
            pdS[m] = a.dSck[e];
        }
        const size_t e = (tok + r_me) * DV + c0 + x_me;
        pv = r_me < n ? load_elem(a.v, e, iob) : 0.f;
        pdO = r_me < n ? load_elem(a.dO, e, iob) : 0.f;
    };
    fetch(0);
    for (int tile = 0; tile < a.ntiles; ++tile) {
        lds_barrier();   // the previous tile's readers are done (loads stay in flight)
#pragma unroll
        for (int m = 0; m < MS; ++m) {   // 16 consecutive lanes share a key dim i
            const int idx = tid + NT * m, i = idx / VT, j = idx % VT;
            sm.w.t.S0[i][j] = pS0[m];
            sm.w.t.dS[i][j] = pdS[m];
            sg[m] += row16_sum(pS0[m] * pdS[m]);
        }
        if (tile == 0) {
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, i = idx % DK;
                const float br = sm.rw.bq[r][i];
                sm.w.t.kd[r][i] = sm.rw.k[r][i] * __builtin_amdgcn_exp2f(br);
                sm.w.t.kt[r][i] = sm.rw.k[r][i] * __builtin_amdgcn_exp2f(sm.rw.bq[C - 1][i] - br);
            }
        }
        sm.v[r_me][x_me] = pv;
        sm.dO[r_me][x_me] = pdO;
        if (tile + 1 < a.ntiles) fetch(tile + 1);
        lds_barrier();
        const int t = r_me, j = x_me;
        const int c0 = tile * VT;
        {
            // (decayed K) S_in into KS and (decayed K) dS_out into R on the fp32 matrix cores
            // (16x16x4, one product per wave, two interleaved accumulators; A row jl with
            // k = g, B column jl with k = g, D column jl with rows 4g .. 4g + 3)
            const int w = tid / kWave, l = tid % kWave, g = l >> 4, jl = l & 15;
            if (w < 2) {
                const float* Ar = w == 0 ? &sm.w.t.kd[jl][0] : &sm.w.t.kt[jl][0];
                const float(*Bt)[VT + 4] = w == 0 ? sm.w.t.S0 : sm.w.t.dS;
                f32x4_t c0v = {0.f, 0.f, 0.f, 0.f}, c1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
                for (int kk = 0; kk < DK; kk += 8) {
                    c0v = __builtin_amdgcn_mfma_f32_16x16x4f32(Ar[kk + g], Bt[kk + g][jl], c0v, 0, 0, 0);
                    c1v = __builtin_amdgcn_mfma_f32_16x16x4f32(Ar[kk + 4 + g], Bt[kk + 4 + g][jl],
                                                                c1v, 0, 0, 0);
                }
                float(*Out)[VT] = w == 0 ? sm.KS : sm.R;
#pragma unroll
                for (int r = 0; r < 4; ++r) Out[4 * g + r][jl] = c0v[r] + c1v[r];
            }
        }
        lds_barrier();
        {
            const float ks = sm.KS[t][j];
            float kds = sm.R[t][j];
            for (int r = t; r < C; ++r) kds += sm.P[r][t] * sm.dO[r][j];
            sm.X[t][j] = sm.rw.b[t] * (sm.v[t][j] - ks);
            sm.R[t][j] = kds;
        }
        lds_barrier();
        if (tid < VT) solve_lower(sm.L, sm.X, sm.U, tid);   // U, one column per thread
        else if (tid >= kWave && tid < kWave + VT)          // dU, on another wave
            solve_upper_t(sm.L, sm.R, sm.dU, tid - kWave);
        lds_barrier();
        {
            const float du = sm.dU[t][j];
            float p = sm.KS[t][j];
            for (int s = 0; s < t; ++s) p += sm.Lt[t][s] * sm.U[s][j];
            if (t < n) store_elem(a.dv, (tok + t) * DV + c0 + j, sm.rw.b[t] * du, iob);
            dbt += row16_sum(du * (sm.v[t][j] - p));
            A_acc += dot16(sm.dO[r_me], sm.U[x_me]);
            B_acc += dot16(sm.dU[r_me], sm.U[x_me]);
        }
        {   // this thread's key dim i is the same for every m
            const int i = tid % DK;
#pragma unroll
            for (int m = 0; m < MQ; ++m) {
                const int tt = (tid + NT * m) / DK;
                so[m] += dot16(sm.w.t.S0[i], sm.dO[tt]);
                su[m] += dot16(sm.w.t.dS[i], sm.U[tt]);
                sdu[m] += dot16(sm.w.t.S0[i], sm.dU[tt]);
            }
        }
    }
    __syncthreads();   // the last tile's readers of the tile arrays are done
    sm.A[r_me][x_me] = A_acc;
    sm.Bm[r_me][x_me] = B_acc;
    if (x_me == 0 && r_me < n) store_elem(a.dbeta, tok + r_me, dbt, gb);
#pragma unroll
    for (int m = 0; m < MS; ++m)
        if ((tid % VT) == 0) sm.sig[(tid + NT * m) / VT] = sg[m];
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
        const int idx = tid + NT * m, tt = idx / DK, i = idx % DK;
        sm.w.f.SDO[tt][i] = so[m];
        sm.w.f.DSU[tt][i] = su[m];
        sm.w.f.SDU[tt][i] = sdu[m];
    }
    __syncthreads();
#pragma unroll 1
    for (int m = 0; m < MQ; ++m) {
        const int idx = tid + NT * m, t = idx / DK, i = idx % DK;
        const auto& rw = sm.rw;
        const float bt = rw.bq[t][i], btm = t > 0 ? rw.bq[t - 1][i] : 0.f;
        const float g1 = __builtin_amdgcn_exp2f(btm);              // 2^b_{t-1}
        const float gt = __builtin_amdgcn_exp2f(bt);               // 2^b_t
        const float at = __builtin_amdgcn_exp2f(bt - btm);         // alpha_t[i]
        const float elt = __builtin_amdgcn_exp2f(rw.bq[C - 1][i] - bt);
        float e2[C];   // 2^(b_{t-1} - b_s) k_s[i] for s < t
#pragma unroll
        for (int s = 0; s < C; ++s)
            e2[s] = s < t ? __builtin_amdgcn_exp2f(btm - rw.bq[s][i]) * rw.k[s][i] : 0.f;
        float sA = 0.f, sB = 0.f, sD = 0.f;
#pragma unroll
        for (int s = 0; s < C; ++s) {
            sA += e2[s] * sm.A[t][s];
            sB += e2[s] * sm.Bm[t][s];
            sD += e2[s] * sm.w.f.DSU[s][i];
        }
        const float dq = gt * sm.w.f.SDO[t][i] + sm.A[t][t] * rw.k[t][i] + at * sA;
        float dk = elt * sm.w.f.DSU[t][i] - rw.b[t] * (gt * sm.w.f.SDU[t][i] + at * sB);
        float da = elt * (g1 * sm.sig[i] + sD) - rw.b[t] * rw.k[t][i] * (g1 * sm.w.f.SDU[t][i] + sB);
        for (int r = t; r < C; ++r) {
            const float er = __builtin_amdgcn_exp2f(rw.bq[r][i] - bt) * rw.q[r][i];
            dk += sm.A[r][t] * er;
            float in = g1 * sm.w.f.SDO[r][i];
#pragma unroll
            for (int s = 0; s < C; ++s) in += e2[s] * sm.A[r][s];
            da += er * in;
        }
        for (int s2 = t + 1; s2 < C; ++s2) {
            const float es = __builtin_amdgcn_exp2f(rw.bq[s2][i] - bt) * rw.b[s2] * rw.k[s2][i];
            dk -= sm.Bm[s2][t] * es;
            float in = g1 * sm.w.f.SDU[s2][i];
#pragma unroll
            for (int s = 0; s < C; ++s) in += e2[s] * sm.Bm[s2][s];
            da -= es * in;
        }
        if (t < n) {
            const size_t e = (tok + t) * DK + i;
            store_elem(a.dq, e, dq, iob);
            store_elem(a.dk, e, dk, iob);
            store_elem(a.dg, e, da, gb);
        }
    }
}

struct GdnLayout {
    size_t Sck, dSck, Tck, Pck, total;
};
GdnLayout gdn_layout(const Problem& p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t nseq = size_t(p.B) * p.H, nchunks = size_t((p.N + C - 1) / C);
    GdnLayout L{};
    L.Sck = 0;
    L.dSck = al(nseq * nchunks * p.dk * p.dv * 4);
    L.Tck = L.dSck + al(nseq * nchunks * p.dk * p.dv * 4);
    L.Pck = L.Tck + al(nseq * nchunks * C * C * 4);
    L.total = L.Pck + al(nseq * nchunks * C * C * 4);
    return L;
}

template <int DK, int DV>
hipError_t launch_dims(const Problem& p, GdnBwdArgs a) {
    constexpr int CT = DV % 64 == 0 ? 64 : DV % 32 == 0 ? 32 : 16;   // columns per chain
    const unsigned chains = unsigned(2 * a.nseq * (DV / CT));
    const unsigned units = unsigned(size_t(a.nseq) * a.nchunks);
    if (p.variant == LA_KDA) {
        kda_bwd_prep_kernel<DK><<<dim3(units), dim3(NT), 0, p.stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        bwd_chains_kernel<LA_KDA, DK, DV, CT><<<dim3(chains), dim3(16 * CT), 0, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        kda_bwd_grads_kernel<DK, DV><<<dim3(units), dim3(NT), 0, p.stream>>>(a);
        return hipGetLastError();
    }
    gdn_bwd_prep_kernel<DK><<<dim3(units), dim3(NT), 0, p.stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_chains_kernel<LA_GDN, DK, DV, CT><<<dim3(chains), dim3(16 * CT), 0, p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gdn_bwd_grads_kernel<DK, DV><<<dim3(units), dim3(NT), 0, p.stream>>>(a);
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch_dv(const Problem& p, const GdnBwdArgs& a) {
    switch (p.dv) {
        case 16: return launch_dims<DK, 16>(p, a);
        case 32: return launch_dims<DK, 32>(p, a);
        case 64: return launch_dims<DK, 64>(p, a);
        case 128: return launch_dims<DK, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gdn_backward_workspace_bytes(const Problem& p) {
    if (p.N == 0 || p.B == 0 || p.H == 0) return 0;
    return gdn_layout(p).total;
}

hipError_t launch_backward_gdn(const BwdProblem& bp) {
    const Problem& p = bp.p;
    const size_t nseq = size_t(p.B) * p.H;
    const size_t nchunks = size_t((p.N + C - 1) / C);
    if (2 * nseq * size_t(p.dv / VT) > 0x7fffffffull || nseq * nchunks > 0x7fffffffull)
        return hipErrorInvalidValue;
    const GdnLayout L = gdn_layout(p);
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    GdnBwdArgs a{};
    a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta; a.dO = bp.dO;
    a.S0 = p.S0; a.dSf = bp.dS_final;
    a.dq = bp.dq; a.dk = bp.dk; a.dv = bp.dv; a.dg = bp.dg; a.dbeta = bp.dbeta;
    a.dS0 = bp.dS0;
    a.Sck = reinterpret_cast<float*>(ws + L.Sck);
    a.dSck = reinterpret_cast<float*>(ws + L.dSck);
    a.Tck = reinterpret_cast<float*>(ws + L.Tck);
    a.Pck = reinterpret_cast<float*>(ws + L.Pck);
    a.N = p.N;
    a.nseq = int(nseq);
    a.ntiles = p.dv / VT;
    a.nchunks = int(nchunks);
    a.io_bf16 = p.io_bf16;
    a.gate_bf16 = p.gate_bf16;
    switch (p.dk) {
        case 16: return dispatch_dv<16>(p, a);
        case 32: return dispatch_dv<32>(p, a);
        case 64: return dispatch_dv<64>(p, a);
        case 128: return dispatch_dv<128>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
