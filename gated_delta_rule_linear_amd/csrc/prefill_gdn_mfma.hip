// Chunked prefill for the gated delta rule on bf16 MFMA (d_k = 128, chunk C = 64).
//
// Method ("线性注意力与 SSM", section GDN, rewritten per chunk; the chunkwise UT/WY
// transform the survey pages name for delta-rule chunking). For one chunk with
// entering state S (key-major, fp32), local rows r, s = 0..C-1:
//   c_r = sum_{s<=r} log alpha_s,  gamma_r = exp(c_r)
//   L_rs = beta_r exp(c_r - c_s) k_r.k_s  (s < r),   T = (I + L)^{-1}
//   X_r = beta_r (v_r - gamma_r S^T k_r),   U = T X
//   o_r = gamma_r S^T q_r + sum_{s<=r} exp(c_r - c_s) (q_r.k_s) u_s
//   S  <- gamma_{C-1} S + sum_s exp(c_{C-1} - c_s) k_s u_s^T
// an exact rewrite of u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t), S_t = alpha_t S_{t-1}
// + k_t u_t^T, o_t = S_t^T q_t. Every exponent is <= 0, so no reciprocal of a
// cumulative decay is ever formed.
//
// Parallel structure: columns of S never mix, so one workgroup owns one
// (sequence, value tile of VT columns) chain and walks all chunks with its state
// tile in registers (MFMA accumulators, fp32). The d_k-only work (K K^T, Q K^T, T)
// is recomputed per value tile; the tiles of one sequence share an XCD so their
// q/k reads hit the same L2.
//
// Per chunk (4 waves, wave w owns row block w of the chunk and key blocks 2w, 2w+1
// of the state):
//   0. scan of log alpha (wave 0), q/k/v and khat = k exp(c_last - c) into LDS
//   1. K K^T -> L (fp32) and K Q^T -> P (bf16, decayed, causal)   [10 lower tiles]
//   2. T = (I + L)^{-1} in fp32: diagonal 16x16 blocks by forward substitution,
//      then T = (I - L')(I + L'^2) D with D = blockdiag(T_bb), L' = D L_offdiag
//   3. O^T = S^T Q^T and X^T from K S (state read as bf16 S^T)
//   4. U^T = X^T T^T;  O^T = gamma O^T + U^T P^T -> o;  S = gamma_last S + khat^T U
// Products are arranged so that D tiles are written to LDS transposed (8-byte
// writes) and read back as contiguous 16-byte fragments; fragments whose K index
// runs along tile rows use the LDS transpose read.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;     // pitch (elements) of [*][128] bf16 tiles
constexpr int PC = C + 8;      // pitch of [*][64] bf16 tiles
constexpr int PL = C + 4;      // pitch of the fp32 [64][64] work tile
constexpr int PE = 16 + 4;     // pitch of fp32 16x16 blocks

template <int VT>
struct __align__(16) GdnSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t q[C * PQ];
    __align__(16) uint16_t k[C * PQ];
    __align__(16) uint16_t kh[C * PQ];
    __align__(16) uint16_t st[VT * PQ];  // S^T [c][i], bf16
    __align__(16) uint16_t v[C * PV];    // V [s][c]
    __align__(16) uint16_t u[C * PV];    // U [s][c]
    __align__(16) uint16_t p[C * PC];    // P [r][s]
    __align__(16) uint16_t t[C * PC];    // T [r][s]
    __align__(16) uint16_t xt[VT * PC];  // X^T [c][s]
    __align__(16) float lf[C * PL];      // L -> L' (off-diagonal), T_bb (diagonal)
    __align__(16) float e[3][16 * PE];   // (L'^2)_20, (L'^2)_31, (L'^2)_30
    __align__(16) float m30[16 * PE];    // M_30
    float cum[C], gam[C], beta[C];
};

struct GdnArgs {
    const uint16_t *q, *k, *v;
    const void *alpha, *beta;
    const float* S0;
    uint16_t* o;
    float* S;
    int N, nseq, ntiles, gate_bf16;
};

// One wave: out = (s1 A1 + s2 A2) * B for 16x16 fp32 blocks; lane computes row lane/4,
// columns 4*(lane%4) .. +3. A2 may be null.
__device__ __forceinline__ void mm16(const float* A1, int pa1, float s1, const float* A2, int pa2,
                                     float s2, const float* B, int pb, int lane, float (&out)[4]) {
    const int r = lane >> 2, c = (lane & 3) * 4;
    out[0] = out[1] = out[2] = out[3] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        float av = s1 * A1[r * pa1 + kk];
        if (A2) av += s2 * A2[r * pa2 + kk];
        const float4 b = *reinterpret_cast<const float4*>(B + kk * pb + c);
        out[0] += av * b.x; out[1] += av * b.y; out[2] += av * b.z; out[3] += av * b.w;
    }
}

__device__ __forceinline__ void put16(float* D, int pd, int lane, const float (&x)[4]) {
    const int r = lane >> 2, c = (lane & 3) * 4;
    *reinterpret_cast<float4*>(D + r * pd + c) = make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void put16_bf16(uint16_t* D, int pd, int lane, const float (&x)[4]) {
    const int r = lane >> 2, c = (lane & 3) * 4;
    uint2 w;
    w.x = pack_bf16x2(x[0], x[1]);
    w.y = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2*>(D + r * pd + c) = w;
}

template <int VT>
__global__ __launch_bounds__(NT) void gdn_fwd_kernel(GdnArgs a) {
    constexpr int NVT = VT / 16;
    constexpr int PV = GdnSmem<VT>::PV;
    constexpr int VV = VT / 8;  // 16-byte vectors per V row
    extern __shared__ __align__(16) unsigned char smem_raw[];
    GdnSmem<VT>& sm = *reinterpret_cast<GdnSmem<VT>*>(smem_raw);

    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles, a.nseq);
    if (!mp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT;
    const int c0 = mp.tile * VT;
    const size_t seq = size_t(mp.seq);
    const size_t tok0 = seq * size_t(a.N);
    const bool gb = a.gate_bf16 != 0;

    // state tiles held by this wave: key blocks 2w + ib, column tiles ct
    f32x4_t S[2][NVT];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * w + ib) + 4 * g + j, c = 16 * ct + jl;
                S[ib][ct][j] = a.S0 ? a.S0[seq * DK * DV + size_t(i) * DV + c0 + c] : 0.f;
            }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) store_dT(sm.st, PQ, 16 * (2 * w + ib), 16 * ct, S[ib][ct], lane);

    // register prefetch of one chunk
    uint4 pq[4], pk[4], pv[2];
    float pg = 0.f;
    auto load_chunk = [&](int ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
            if (r < n) {
                const size_t e = (tok0 + t0 + r) * DK + col;
                pq[x4] = ld_g16(a.q + e);
                pk[x4] = ld_g16(a.k + e);
            } else {
                pq[x4] = pk[x4] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            pv[x2] = make_uint4(0, 0, 0, 0);
            if (x < C * VV && r < n) pv[x2] = ld_g16(a.v + (tok0 + t0 + r) * DV + c0 + col);
        }
        if (tid < C) pg = tid < n ? logf(load_elem(a.alpha, tok0 + t0 + tid, gb)) : 0.f;
        else if (tid < 2 * C) pg = (tid - C) < n ? load_elem(a.beta, tok0 + t0 + tid - C, gb) : 0.f;
    };

    const int nchunks = (a.N + C - 1) / C;
    if (nchunks > 0) load_chunk(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
        // ---- phase 0: gates, then stage q, k, khat, v into LDS
        if (w == 0) {
            float x = pg;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sm.cum[lane] = x;
            sm.gam[lane] = __expf(x);
        } else if (w == 1) {
            sm.beta[lane] = pg;
        }
        __syncthreads();
        const float clast = sm.cum[C - 1];
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
            *reinterpret_cast<uint4*>(sm.q + r * PQ + col) = pq[x4];
            *reinterpret_cast<uint4*>(sm.k + r * PQ + col) = pk[x4];
            float f[8];
            unpack8(pk[x4], f);
            const float sc = __expf(clast - sm.cum[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= sc;
            *reinterpret_cast<uint4*>(sm.kh + r * PQ + col) = pack8(f);
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) *reinterpret_cast<uint4*>(sm.v + r * PV + col) = pv[x2];
        }
        __syncthreads();
        if (ch + 1 < nchunks) load_chunk(ch + 1);

        // ---- phase 1: L = stril(beta exp(c_r - c_s) K K^T) (fp32), P = tril(exp(c_r - c_s) Q K^T)
        for (int ti = w; ti < 10; ti += 4) {
            const int rb = ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3;
            const int sb = ti - (rb * (rb + 1)) / 2;
            f32x4_t kk_acc = zero4(), kq_acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const bf16x8_t kr = frag_kc(sm.k, PQ, 16 * rb, 32 * kk, lane);
                const bf16x8_t ks = frag_kc(sm.k, PQ, 16 * sb, 32 * kk, lane);
                const bf16x8_t qr = frag_kc(sm.q, PQ, 16 * rb, 32 * kk, lane);
                kk_acc = mfma16(kr, ks, kk_acc);   // D[r][s] = k_r . k_s
                kq_acc = mfma16(ks, qr, kq_acc);   // D[s][r] = k_s . q_r
            }
            {   // L: lane holds column s = 16 sb + jl, rows r = 16 rb + 4g + j
                const int s = 16 * sb + jl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rb + 4 * g + j;
                    const float val = s < r ? sm.beta[r] * __expf(sm.cum[r] - sm.cum[s]) * kk_acc[j] : 0.f;
                    sm.lf[r * PL + s] = val;
                }
            }
            {   // P: lane holds column r = 16 rb + jl, rows s = 16 sb + 4g + j
                const int r = 16 * rb + jl;
                f32x4_t pv4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * sb + 4 * g + j;
                    pv4[j] = s <= r ? __expf(sm.cum[r] - sm.cum[s]) * kq_acc[j] : 0.f;
                }
                store_dT(sm.p, PC, 16 * sb, 16 * rb, pv4, lane);
            }
        }
        // zero the upper tiles that the row-block products read: (0,1) and (2,3), in P and T
        if (w < 2) {
            const int rb = w == 0 ? 0 : 2, sb = rb + 1;
            const int r = 16 * rb + (lane >> 2), s = 16 * sb + (lane & 3) * 4;
            *reinterpret_cast<uint2*>(sm.p + r * PC + s) = make_uint2(0, 0);
            *reinterpret_cast<uint2*>(sm.t + r * PC + s) = make_uint2(0, 0);
        }
        __syncthreads();

        // ---- phase 2: T = (I + L)^{-1}
        // level 0: diagonal blocks by forward substitution, wave b, lane = column
        if (lane < 16) {
            const int b = w, jc = lane;
            const float* Lb = sm.lf + (16 * b) * PL + 16 * b;
            float tcol[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) tcol[r] = r == jc ? 1.f : 0.f;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc += Lb[r * PL + m] * tcol[m];
                if (r > jc) tcol[r] = -acc;
            }
            float* Tb = sm.lf + (16 * b) * PL + 16 * b;
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[r * PL + jc] = tcol[r];
        }
        __syncthreads();
        auto blk = [&](int bi, int bj) { return sm.lf + (16 * bi) * PL + 16 * bj; };
        // level 1: L'_bm = T_bb L_bm (in place)
        {
            const int lst[6][2] = {{1, 0}, {2, 0}, {2, 1}, {3, 0}, {3, 1}, {3, 2}};
            for (int x = w; x < 6; x += 4) {
                const int bi = lst[x][0], bj = lst[x][1];
                float out[4];
                mm16(blk(bi, bi), PL, 1.f, nullptr, 0, 0.f, blk(bi, bj), PL, lane, out);
                put16(blk(bi, bj), PL, lane, out);
            }
        }
        __syncthreads();
        // level 2: (L'^2)_20 = L'_21 L'_10, (L'^2)_31 = L'_32 L'_21, (L'^2)_30 = L'_31 L'_10 + L'_32 L'_20
        if (w == 0) {
            float out[4];
            mm16(blk(2, 1), PL, 1.f, nullptr, 0, 0.f, blk(1, 0), PL, lane, out);
            put16(sm.e[0], PE, lane, out);
        } else if (w == 1) {
            float out[4];
            mm16(blk(3, 2), PL, 1.f, nullptr, 0, 0.f, blk(2, 1), PL, lane, out);
            put16(sm.e[1], PE, lane, out);
        } else if (w == 2) {
            float o1[4], o2[4];
            mm16(blk(3, 1), PL, 1.f, nullptr, 0, 0.f, blk(1, 0), PL, lane, o1);
            mm16(blk(3, 2), PL, 1.f, nullptr, 0, 0.f, blk(2, 0), PL, lane, o2);
            for (int j = 0; j < 4; ++j) o1[j] += o2[j];
            put16(sm.e[2], PE, lane, o1);
        }
        __syncthreads();
        // level 3: T_ij = M_ij T_jj below the diagonal, M = I - L' + L'^2 - L'^3:
        // M_10 = -L'_10, M_21 = -L'_21, M_32 = -L'_32, M_20 = -L'_20 + (L'^2)_20,
        // M_31 = -L'_31 + (L'^2)_31, M_30 = -L'_30 + (L'^2)_30 - L'_32 (L'^2)_20 (formed here,
        // applied at level 4)
        {
            float out[4];
            if (w == 0) {
                mm16(blk(1, 0), PL, -1.f, nullptr, 0, 0.f, blk(0, 0), PL, lane, out);
                put16_bf16(sm.t + 16 * PC + 0, PC, lane, out);
                mm16(blk(3, 1), PL, -1.f, sm.e[1], PE, 1.f, blk(1, 1), PL, lane, out);
                put16_bf16(sm.t + 48 * PC + 16, PC, lane, out);
            } else if (w == 1) {
                mm16(blk(2, 1), PL, -1.f, nullptr, 0, 0.f, blk(1, 1), PL, lane, out);
                put16_bf16(sm.t + 32 * PC + 16, PC, lane, out);
                mm16(blk(2, 0), PL, -1.f, sm.e[0], PE, 1.f, blk(0, 0), PL, lane, out);
                put16_bf16(sm.t + 32 * PC + 0, PC, lane, out);
            } else if (w == 2) {
                mm16(blk(3, 2), PL, -1.f, nullptr, 0, 0.f, blk(2, 2), PL, lane, out);
                put16_bf16(sm.t + 48 * PC + 32, PC, lane, out);
            } else {
                mm16(blk(3, 2), PL, 1.f, nullptr, 0, 0.f, sm.e[0], PE, lane, out);
                const int r = lane >> 2, c = (lane & 3) * 4;
                const float* L30 = blk(3, 0);
                float m[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    m[j] = -L30[r * PL + c + j] + sm.e[2][r * PE + c + j] - out[j];
                put16(sm.m30, PE, lane, m);
            }
            // diagonal blocks of T (bf16), wave b writes block b
            {
                const int r = lane >> 2, c = (lane & 3) * 4;
                const float* Tb = blk(w, w);
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = Tb[r * PL + c + j];
                put16_bf16(sm.t + (16 * w) * PC + 16 * w, PC, lane, x);
            }
        }
        __syncthreads();
        // level 4: T_30 = M_30 T_00
        if (w == 0) {
            float out[4];
            mm16(sm.m30, PE, 1.f, nullptr, 0, 0.f, blk(0, 0), PL, lane, out);
            put16_bf16(sm.t + 48 * PC + 0, PC, lane, out);
        }

        // ---- phase 3: O^T = S^T Q^T (row block w), X = beta (V - gamma K S) (row block w)
        f32x4_t oacc[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t o_ = zero4(), x_ = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const bf16x8_t sT = frag_kc(sm.st, PQ, 16 * ct, 32 * kk, lane);
                o_ = mfma16(sT, frag_kc(sm.q, PQ, 16 * w, 32 * kk, lane), o_);   // D[c][r]
                x_ = mfma16(frag_kc(sm.k, PQ, 16 * w, 32 * kk, lane), sT, x_);   // D[s][c]
            }
            oacc[ct] = o_;
            const int c = 16 * ct + jl;
            f32x4_t xv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * w + 4 * g + j;
                const float vv = bf16_to_f32(sm.v[s * PV + c]);
                xv[j] = sm.beta[s] * (vv - sm.gam[s] * x_[j]);
            }
            store_dT(sm.xt, PC, 16 * w, 16 * ct, xv, lane);   // X^T[c][s]
        }
        __syncthreads();

        // ---- phase 4a: U^T = X^T T^T (row block w of U)
        const int nk = w < 2 ? 1 : 2;   // T and P vanish for s >= 16 (w + 1)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t u_ = zero4();
            for (int kk = 0; kk < nk; ++kk)
                u_ = mfma16(frag_kc(sm.xt, PC, 16 * ct, 32 * kk, lane),
                            frag_kc(sm.t, PC, 16 * w, 32 * kk, lane), u_);   // D[c][r]
            store_dT(sm.u, PV, 16 * ct, 16 * w, u_, lane);                       // U[r][c]
        }
        __syncthreads();

        // ---- phase 4b: O^T = gamma O^T + U^T P^T, written to o; S update
        {
            const int r = 16 * w + jl;
            const float gr = sm.gam[r];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = oacc[ct] * gr;
                for (int kk = 0; kk < nk; ++kk)
                    o_ = mfma16(frag_kr(sm.u, PV, 32 * kk, 16 * ct, lane),
                                frag_kc(sm.p, PC, 16 * w, 32 * kk, lane), o_);
                if (r < n) {
                    uint2 wv;
                    wv.x = pack_bf16x2(o_[0], o_[1]);
                    wv.y = pack_bf16x2(o_[2], o_[3]);
                    *reinterpret_cast<uint2*>(a.o + (tok0 + t0 + r) * DV + c0 + 16 * ct + 4 * g) = wv;
                }
            }
        }
        {
            const float gl = sm.gam[C - 1];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i0 = 16 * (2 * w + ib);
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct) {
                    f32x4_t s_ = S[ib][ct] * gl;
#pragma unroll
                    for (int kk = 0; kk < C / 32; ++kk)
                        s_ = mfma16(frag_kr(sm.kh, PQ, 32 * kk, i0, lane),
                                    frag_kr(sm.u, PV, 32 * kk, 16 * ct, lane), s_);
                    S[ib][ct] = s_;
                    store_dT(sm.st, PQ, i0, 16 * ct, s_, lane);
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * w + ib) + 4 * g + j, c = 16 * ct + jl;
                a.S[seq * DK * DV + size_t(i) * DV + c0 + c] = S[ib][ct][j];
            }
}

template <int VT>
hipError_t launch_vt(const Problem& p) {
    GdnArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.alpha = p.g;
    a.beta = p.beta;
    a.S0 = p.S0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    a.N = p.N;
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 26)) return hipErrorInvalidValue;
    a.nseq = int(nseq);
    a.ntiles = p.dv / VT;
    a.gate_bf16 = p.gate_bf16;
    const size_t smem = sizeof(GdnSmem<VT>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_fwd_kernel<VT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    const int grid = xcd_grid(a.ntiles, a.nseq);
    gdn_fwd_kernel<VT><<<dim3(grid), dim3(NT), smem, p.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool gdn_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

hipError_t launch_prefill_gdn_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    // value tile: 32 columns when that already gives a full wave of workgroups
    const bool wide = p.dv >= 32 && nseq * size_t(p.dv / 32) >= 256;
    return wide ? launch_vt<32>(p) : launch_vt<16>(p);
}

}  // namespace la
