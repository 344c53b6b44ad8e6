// Backward of the SSD prefill (one decay per token and head: "Linear / RNN 路线",
// sections 3.6 and 4.1) on bf16 MFMA, d_k = 128, d_v = 64, chunk C = 64.
//
// With c_r the cumulative log decay inside a chunk (c_{-1} = 0), E_r = exp(c_r),
// F_s = exp(c_last - c_s), D_rs = exp(c_r - c_s) for s <= r (else 0) and Y_su =
// exp(c_{s-1} - c_u) for u < s (else 0), all at most 1, the gradients for dL/do = dO
// and the state gradient dS_out leaving the chunk (S_in the state entering it) are
//   P = (Q K^T) o D,  A = (dO V^T) o D
//   dV = P^T dO + diag(F) K dS_out
//   dQ = diag(E) dO S_in^T + A K
//   dK = A^T Q + diag(F) V dS_out^T
// and, for the decay, dL/da_s = <dS_s, S_{s-1}> expanded over the chunk's tokens into
//   exp(c_{s-1}) sum_{r>=s} D_rs alpha_r + sum_{r>=s} D_rs Z_rs
//   + F_s exp(c_{s-1}) <dS_out, S_in> + F_s sum_{u<s} Y_su beta_u
// with alpha_r = q_r^T S_in dO_r, beta_u = k_u^T dS_out v_u and Z = ((Q K^T) o (dO V^T)) Y^T
// (Z_rs = sum_{u<s} Y_su (q_r . k_u)(dO_r . v_u)): every factor at most 1, no division.
// The chunk-to-chunk carries are elementwise (S_in[c+1] = a_c S_in[c] + dS_c with
// dS_c = K^T diag(F) V, and dS_out[c-1] = a_c dS_out[c] + G_c with G_c = Q^T diag(E) dO),
// so three kernels: sums (per chunk, matrix cores), scans (per state element, both
// directions, in place), grads (per chunk, all value columns, matrix cores). Decays are
// clamped at exp(-10) as in the forward.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128, DV = 64;
constexpr int C = kMfmaChunk;   // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;      // pitch of [*][128] bf16 tiles
constexpr int PV = DV + 8;      // pitch of [*][64] bf16 tiles
constexpr float kGateMin = 4.539993e-05f;   // exp(-10)

struct SbArgs {
    const uint16_t *q, *k, *v, *dO;
    const void* g;
    const float *S0, *dSf;
    uint16_t *dq, *dk, *dv;
    void* dg;
    float* dS0;
    float *Sst, *dSt, *ac;   // [nseq][nch][DK][DV] x 2 (chunk sums dS, G), [nseq][nch]
    uint16_t *Sb, *dSb;      // [nseq][nch][DK][DV] x 2: S_in, dS_out of every chunk, bf16
    int N, nseq, nch;
};

// cumulative log2 decay of a chunk's rows (wave 0), padding rows gate 1
template <bool GB>
__device__ __forceinline__ void chunk_logs(float* c, const SbArgs& a, size_t tok0, int t0, int n) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float gv = 1.f;
        if (lane < n) {
            const size_t e = tok0 + t0 + lane;
            gv = fmaxf(GB ? bf16_to_f32(static_cast<const uint16_t*>(a.g)[e])
                          : static_cast<const float*>(a.g)[e],
                       kGateMin);
        }
        c[lane] = wave_inclusive_scan(__builtin_amdgcn_logf(gv));
    }
}

// A thread's 16-byte pieces of rows t0 .. t0 + 63 of a [N][W] bf16 matrix (rows past the
// sequence's end read as zero): fetched first and stored to LDS later, so that the loads
// of all of a chunk's matrices are in flight together instead of one round trip each.
template <int W>
struct RowPieces {
    static constexpr int PPR = W / 8, NP = C * PPR / NT;   // pieces per row, per thread
    static_assert(C * PPR % NT == 0, "whole pieces per thread");
    uint4 w[NP];
};
template <int W>
__device__ __forceinline__ void fetch_rows(RowPieces<W>& R, const uint16_t* src, size_t tok0, int t0,
                                           int n) {
    constexpr int PPR = RowPieces<W>::PPR;
    const rsrc_t rs = make_rsrc(src + (tok0 + t0) * W, uint32_t(max(n, 0)) * uint32_t(W) * 2u);
#pragma unroll
    for (int x = 0; x < RowPieces<W>::NP; ++x) {
        const int p = int(threadIdx.x) + NT * x, r = p / PPR, cpos = (p % PPR) * 8;
        R.w[x] = buf_ld16(rs, uint32_t(r * W + cpos) * 2u);
    }
}
// ... into an LDS tile of pitch P, scaled per row by f(row)
template <int W, int P, typename F>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const RowPieces<W>& R, F scale) {
    constexpr int PPR = RowPieces<W>::PPR;
#pragma unroll
    for (int x = 0; x < RowPieces<W>::NP; ++x) {
        const int p = int(threadIdx.x) + NT * x, r = p / PPR, cpos = (p % PPR) * 8;
        uint4 w = R.w[x];
        const float f = scale(r);
        if (f != 1.f) {
            float y[8];
            unpack8(w, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= f;
            w = pack8(y);
        }
        *reinterpret_cast<uint4*>(dst + r * P + cpos) = w;
    }
}

// ---------------------------------------------------------------------------- sums
struct __align__(16) SumsSmem {
    __align__(16) uint16_t kh[C * PQ];   // diag(F) K
    __align__(16) uint16_t qh[C * PQ];   // diag(E) Q
    __align__(16) uint16_t v[C * PV];
    __align__(16) uint16_t dO[C * PV];
    float c[C];
};

template <bool GB>
__global__ __launch_bounds__(NT) void ssd_bwd_sums_kernel(SbArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SumsSmem& sm = *reinterpret_cast<SumsSmem*>(smem_raw);
    const int lane = threadIdx.x & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const size_t seq = blockIdx.x / a.nch;
    const int ch = blockIdx.x % a.nch, t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok0 = seq * size_t(a.N);
    RowPieces<DK> kr, qr;
    RowPieces<DV> vr, dr;
    fetch_rows(kr, a.k, tok0, t0, n);
    fetch_rows(qr, a.q, tok0, t0, n);
    fetch_rows(vr, a.v, tok0, t0, n);
    fetch_rows(dr, a.dO, tok0, t0, n);
    chunk_logs<GB>(sm.c, a, tok0, t0, n);
    __syncthreads();
    const float cl = sm.c[C - 1];
    stage_rows<DK, PQ>(sm.kh, kr, [&](int r) { return __builtin_amdgcn_exp2f(cl - sm.c[r]); });
    stage_rows<DK, PQ>(sm.qh, qr, [&](int r) { return __builtin_amdgcn_exp2f(sm.c[r]); });
    stage_rows<DV, PV>(sm.v, vr, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.dO, dr, [](int) { return 1.f; });
    __syncthreads();
    const size_t base = (seq * a.nch + ch) * size_t(DK) * DV;
    // wave w: key rows 32 w .. 32 w + 31 of dS = Kh^T V and G = Qh^T dO
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int i0 = 32 * w + 16 * ib;
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) {
            f32x4_t ds = zero4(), gq = zero4();
#pragma unroll
            for (int kk = 0; kk < C / 32; ++kk) {
                ds = mfma16(frag_kr(sm.kh, PQ, 32 * kk, i0, lane), frag_kr(sm.v, PV, 32 * kk, 16 * nt, lane), ds);
                gq = mfma16(frag_kr(sm.qh, PQ, 32 * kk, i0, lane), frag_kr(sm.dO, PV, 32 * kk, 16 * nt, lane), gq);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t o = base + size_t(i0 + 4 * g + e) * DV + 16 * nt + jl;
                a.Sst[o] = ds[e];
                a.dSt[o] = gq[e];
            }
        }
    }
    if (threadIdx.x == 0) a.ac[seq * a.nch + ch] = __builtin_amdgcn_exp2f(cl);
}

// ---------------------------------------------------------------------------- scans
__global__ __launch_bounds__(NT) void ssd_bwd_scans_kernel(SbArgs a) {
    // four consecutive state elements per thread: 16-byte reads of the fp32 chunk sums,
    // 8-byte writes of the bf16 chunk states (the state itself is carried in fp32)
    const size_t e4 = size_t(blockIdx.x) * NT + threadIdx.x;
    constexpr size_t SS = size_t(DK) * DV;
    if (e4 >= size_t(a.nseq) * SS / 4) return;
    const size_t e = 4 * e4, seq = e / SS, ij = e % SS;
    const float* Ss = a.Sst + seq * a.nch * SS + ij;
    const float* dSs = a.dSt + seq * a.nch * SS + ij;
    uint16_t* Sbs = a.Sb + seq * a.nch * SS + ij;
    uint16_t* dSbs = a.dSb + seq * a.nch * SS + ij;
    const float* ac = a.ac + seq * a.nch;
    auto ld4 = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
    auto st4 = [](uint16_t* p, const float (&x)[4]) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    };
    float S[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.S0) {
        const float4 s0 = ld4(a.S0 + e);
        S[0] = s0.x; S[1] = s0.y; S[2] = s0.z; S[3] = s0.w;
    }
    // chunks in batches of SB, every load of a batch issued before its stores
    constexpr int SB = 8;
    for (int c0 = 0; c0 < a.nch; c0 += SB) {
        float4 d[SB];
        float g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            d[b] = c0 + b < a.nch ? ld4(Ss + (c0 + b) * SS) : make_float4(0.f, 0.f, 0.f, 0.f);
            g[b] = c0 + b < a.nch ? ac[c0 + b] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            if (c0 + b < a.nch) st4(Sbs + (c0 + b) * SS, S);
            S[0] = g[b] * S[0] + d[b].x;
            S[1] = g[b] * S[1] + d[b].y;
            S[2] = g[b] * S[2] + d[b].z;
            S[3] = g[b] * S[3] + d[b].w;
        }
    }
    float dS[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.dSf) {
        const float4 f = ld4(a.dSf + e);
        dS[0] = f.x; dS[1] = f.y; dS[2] = f.z; dS[3] = f.w;
    }
    for (int c1 = a.nch - 1; c1 >= 0; c1 -= SB) {
        float4 d[SB];
        float g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            d[b] = c1 - b >= 0 ? ld4(dSs + (c1 - b) * SS) : make_float4(0.f, 0.f, 0.f, 0.f);
            g[b] = c1 - b >= 0 ? ac[c1 - b] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            if (c1 - b >= 0) st4(dSbs + (c1 - b) * SS, dS);
            dS[0] = g[b] * dS[0] + d[b].x;
            dS[1] = g[b] * dS[1] + d[b].y;
            dS[2] = g[b] * dS[2] + d[b].z;
            dS[3] = g[b] * dS[3] + d[b].w;
        }
    }
    *reinterpret_cast<float4*>(a.dS0 + e) = make_float4(dS[0], dS[1], dS[2], dS[3]);
}

// ---------------------------------------------------------------------------- grads
struct __align__(16) GradsSmem {
    __align__(16) uint16_t q[C * PQ], k[C * PQ];
    __align__(16) uint16_t v[C * PV], dO[C * PV];
    __align__(16) uint16_t sin[DK * PV], dso[DK * PV];   // S_in, dS_out as [key][column]
    __align__(16) uint16_t P[C * PV], A[C * PV], M[C * PV], Y[C * PV];
    float c[C], alpha[C], beta[C];
    float t2w[NT / 64][C];   // per-wave partials of term2, summed in wave order
    float red[NT / 64];
};

template <bool GB>
__global__ __launch_bounds__(NT) void ssd_bwd_grads_kernel(SbArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    GradsSmem& sm = *reinterpret_cast<GradsSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const size_t seq = blockIdx.x / a.nch;
    const int ch = blockIdx.x % a.nch, t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok0 = seq * size_t(a.N);
    // every load of the chunk first (q, k, v, dO, S_in, dS_out), then the LDS copies
    RowPieces<DK> qr, kr;
    RowPieces<DV> vr, dr;
    fetch_rows(qr, a.q, tok0, t0, n);
    fetch_rows(kr, a.k, tok0, t0, n);
    fetch_rows(vr, a.v, tok0, t0, n);
    fetch_rows(dr, a.dO, tok0, t0, n);
    constexpr int NS = DK * DV / 4 / NT;   // 4-element pieces of S_in (and of dS_out) per thread
    uint2 s4v[NS], d4v[NS];
    const size_t base = (seq * a.nch + ch) * size_t(DK) * DV;
#pragma unroll
    for (int x = 0; x < NS; ++x) {
        const size_t p = size_t(tid + NT * x);
        s4v[x] = *reinterpret_cast<const uint2*>(a.Sb + base + 4 * p);
        d4v[x] = *reinterpret_cast<const uint2*>(a.dSb + base + 4 * p);
    }
    chunk_logs<GB>(sm.c, a, tok0, t0, n);
    if (tid < C) { sm.alpha[tid] = 0.f; sm.beta[tid] = 0.f; }
    stage_rows<DK, PQ>(sm.q, qr, [](int) { return 1.f; });
    stage_rows<DK, PQ>(sm.k, kr, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.v, vr, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.dO, dr, [](int) { return 1.f; });
    // S_in and dS_out (bf16 in the workspace) to their LDS tiles, and gamma = <dS_out, S_in>
    {
        float gam = 0.f;
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            const int p = tid + NT * x;
            const int i = (4 * p) / DV, j = (4 * p) % DV;
            const uint2 s4 = s4v[x], d4 = d4v[x];
            gam += __uint_as_float(s4.x << 16) * __uint_as_float(d4.x << 16) +
                   __uint_as_float(s4.x & 0xffff0000u) * __uint_as_float(d4.x & 0xffff0000u) +
                   __uint_as_float(s4.y << 16) * __uint_as_float(d4.y << 16) +
                   __uint_as_float(s4.y & 0xffff0000u) * __uint_as_float(d4.y & 0xffff0000u);
            *reinterpret_cast<uint2*>(sm.sin + i * PV + j) = s4;
            *reinterpret_cast<uint2*>(sm.dso + i * PV + j) = d4;
        }
        gam = wave_sum(gam);
        if (lane == 0) sm.red[w] = gam;
    }
    __syncthreads();
    const float cl = sm.c[C - 1];
    const float gamma = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
    // P, A, M: wave w owns rows 16 w .. 16 w + 15. The lane's decay sums (rows r = r0 + 4 g
    // + e, columns s = 16 nt + j) are read once before any LDS write: LDS reads issued after
    // an LDS write the compiler cannot tell apart wait for it, one round trip each.
    const int r0 = 16 * w;
    float cr[4], cs4[C / 16];
#pragma unroll
    for (int e = 0; e < 4; ++e) cr[e] = sm.c[r0 + 4 * g + e];
#pragma unroll
    for (int nt = 0; nt < C / 16; ++nt) cs4[nt] = sm.c[16 * nt + jl];
    {   // Y (elementwise): thread tid fills column u = tid mod C of rows tid / C + 4 i
        static_assert(NT % C == 0, "whole rows per pass");
        constexpr int NI = C * C / NT;
        const int u = tid % C, s0 = tid / C;
        const float cu = sm.c[u];
        float cmv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s = s0 + (NT / C) * i;
            cmv[i] = s > 0 ? sm.c[s - 1] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s = s0 + (NT / C) * i;
            sm.Y[s * PV + u] = f32_to_bf16(u < s ? __builtin_amdgcn_exp2f(cmv[i] - cu) : 0.f);
        }
    }
#pragma unroll
    for (int nt = 0; nt < C / 16; ++nt) {
        f32x4_t qk = zero4(), ov = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            qk = mfma16(frag_kc(sm.q, PQ, r0, 32 * kk, lane), frag_kc(sm.k, PQ, 16 * nt, 32 * kk, lane), qk);
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk)
            ov = mfma16(frag_kc(sm.dO, PV, r0, 32 * kk, lane), frag_kc(sm.v, PV, 16 * nt, 32 * kk, lane), ov);
        const int s = 16 * nt + jl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + 4 * g + e;
            const float d = s <= r ? __builtin_amdgcn_exp2f(cr[e] - cs4[nt]) : 0.f;
            sm.P[r * PV + s] = f32_to_bf16(qk[e] * d);
            sm.A[r * PV + s] = f32_to_bf16(ov[e] * d);
            sm.M[r * PV + s] = f32_to_bf16(qk[e] * ov[e]);
        }
    }
    __syncthreads();
    // gradient rows past the sequence's end fall outside these resources and are dropped
    // (branch-free stores)
    auto rows_rsrc = [&](uint16_t* dst, int W) {
        return make_rsrc(dst + (tok0 + t0) * size_t(W), uint32_t(n) * uint32_t(W) * 2u);
    };
    const rsrc_t rdv = rows_rsrc(a.dv, DV), rdq = rows_rsrc(a.dq, DK), rdk = rows_rsrc(a.dk, DK);
    auto store_bf = [&](const rsrc_t& rs, int W, int r, int col, float x) {
        buf_st2(rs, uint32_t(r * W + col) * 2u, f32_to_bf16(x));
    };
    float er[4], fr[4];   // 2^{c_r} and 2^{c_last - c_r} of the lane's rows
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        er[e] = __builtin_amdgcn_exp2f(cr[e]);
        fr[e] = __builtin_amdgcn_exp2f(cl - cr[e]);
    }
    // dV = P^T dO + diag(F) K dS_out (rows s = 16 w ..)
#pragma unroll
    for (int nt = 0; nt < DV / 16; ++nt) {
        f32x4_t x = zero4(), y = zero4();
#pragma unroll
        for (int kk = 0; kk < C / 32; ++kk)
            x = mfma16(frag_kr(sm.P, PV, 32 * kk, r0, lane), frag_kr(sm.dO, PV, 32 * kk, 16 * nt, lane), x);
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            y = mfma16(frag_kc(sm.k, PQ, r0, 32 * kk, lane), frag_kr(sm.dso, PV, 32 * kk, 16 * nt, lane), y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = r0 + 4 * g + e;
            store_bf(rdv, DV, s, 16 * nt + jl, x[e] + fr[e] * y[e]);
        }
    }
    // dQ = diag(E) dO S_in^T + A K, dK = A^T Q + diag(F) V dS_out^T (rows 16 w ..)
#pragma unroll 2
    for (int nt = 0; nt < DK / 16; ++nt) {
        f32x4_t x = zero4(), y = zero4(), u = zero4(), z = zero4();
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk) {
            x = mfma16(frag_kc(sm.dO, PV, r0, 32 * kk, lane), frag_kc(sm.sin, PV, 16 * nt, 32 * kk, lane), x);
            z = mfma16(frag_kc(sm.v, PV, r0, 32 * kk, lane), frag_kc(sm.dso, PV, 16 * nt, 32 * kk, lane), z);
        }
#pragma unroll
        for (int kk = 0; kk < C / 32; ++kk) {
            y = mfma16(frag_kc(sm.A, PV, r0, 32 * kk, lane), frag_kr(sm.k, PQ, 32 * kk, 16 * nt, lane), y);
            u = mfma16(frag_kr(sm.A, PV, 32 * kk, r0, lane), frag_kr(sm.q, PQ, 32 * kk, 16 * nt, lane), u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + 4 * g + e;
            store_bf(rdq, DK, r, 16 * nt + jl, er[e] * x[e] + y[e]);
            store_bf(rdk, DK, r, 16 * nt + jl, u[e] + fr[e] * z[e]);
        }
    }
    // alpha_r = sum_j (Q S_in)_rj dO_rj, beta_u = sum_j (K dS_out)_uj v_uj, and term2
    // partials sum_{r>=s} D_rs Z_rs with Z = M Y^T
    {
        float al[4] = {0.f, 0.f, 0.f, 0.f}, be[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) {
            f32x4_t x = zero4(), y = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                x = mfma16(frag_kc(sm.q, PQ, r0, 32 * kk, lane), frag_kr(sm.sin, PV, 32 * kk, 16 * nt, lane), x);
                y = mfma16(frag_kc(sm.k, PQ, r0, 32 * kk, lane), frag_kr(sm.dso, PV, 32 * kk, 16 * nt, lane), y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 4 * g + e, j = 16 * nt + jl;
                al[e] += x[e] * bf16_to_f32(sm.dO[r * PV + j]);
                be[e] += y[e] * bf16_to_f32(sm.v[r * PV + j]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = al[e], y = be[e];
            x += dpp_f<0xB1, 0xf, 0xf>(x); y += dpp_f<0xB1, 0xf, 0xf>(y);
            x += dpp_f<0x4E, 0xf, 0xf>(x); y += dpp_f<0x4E, 0xf, 0xf>(y);
            x += dpp_f<0x141, 0xf, 0xf>(x); y += dpp_f<0x141, 0xf, 0xf>(y);
            x += dpp_f<0x140, 0xf, 0xf>(x); y += dpp_f<0x140, 0xf, 0xf>(y);
            if (jl == 0) {
                sm.alpha[r0 + 4 * g + e] = x;
                sm.beta[r0 + 4 * g + e] = y;
            }
        }
#pragma unroll
        for (int nt = 0; nt < C / 16; ++nt) {
            f32x4_t z = zero4();
#pragma unroll
            for (int kk = 0; kk < C / 32; ++kk)
                z = mfma16(frag_kc(sm.M, PV, r0, 32 * kk, lane), frag_kc(sm.Y, PV, 16 * nt, 32 * kk, lane), z);
            const int s = 16 * nt + jl;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 4 * g + e;
                if (s <= r) part += __builtin_amdgcn_exp2f(cr[e] - cs4[nt]) * z[e];
            }
            // the four lane groups' rows in a fixed order, then one partial per wave
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (g == 0) sm.t2w[w][s] = part;
        }
    }
    __syncthreads();
    if (tid < n) {
        const int s = tid;
        const float cs = sm.c[s], cm = s > 0 ? sm.c[s - 1] : 0.f;
        const float es1 = __builtin_amdgcn_exp2f(cm), fs = __builtin_amdgcn_exp2f(cl - cs);
        // t1 = sum_{r>=s} 2^(c_r - c_s) alpha_r and t4 = sum_{u<s} 2^(c_{s-1} - c_u) beta_u, in
        // increasing index, as one unrolled pass of 16-byte broadcast reads (a loop with a
        // data-dependent trip count waits on every read)
        float t1 = 0.f, t4 = 0.f;
#pragma unroll
        for (int x4 = 0; x4 < C; x4 += 4) {
            const float4 c4 = *reinterpret_cast<const float4*>(sm.c + x4);
            const float4 a4 = *reinterpret_cast<const float4*>(sm.alpha + x4);
            const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + x4);
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w},
                        bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = x4 + i;
                const float d = __builtin_amdgcn_exp2f(x >= s ? cv[i] - cs : cm - cv[i]);
                if (x >= s) t1 += d * av[i];
                else t4 += d * bv[i];
            }
        }
        static_assert(NT == 256, "four waves");
        const float t2 = ((sm.t2w[0][s] + sm.t2w[1][s]) + sm.t2w[2][s]) + sm.t2w[3][s];
        const float da = es1 * t1 + t2 + fs * es1 * gamma + fs * t4;
        const size_t e = tok0 + t0 + s;
        if (GB) static_cast<uint16_t*>(a.dg)[e] = f32_to_bf16(da);
        else static_cast<float*>(a.dg)[e] = da;
    }
}

struct SbLayout {
    size_t Sst, dSt, Sb, dSb, ac, total;
};
SbLayout sb_layout(const Problem& p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t nseq = size_t(p.B) * p.H, nch = size_t((p.N + C - 1) / C);
    SbLayout L{};
    size_t off = 0;
    L.Sst = off; off += al(nseq * nch * DK * DV * 4);
    L.dSt = off; off += al(nseq * nch * DK * DV * 4);
    L.Sb = off; off += al(nseq * nch * DK * DV * 2);
    L.dSb = off; off += al(nseq * nch * DK * DV * 2);
    L.ac = off; off += al(nseq * nch * 4);
    L.total = off;
    return L;
}

template <bool GB>
hipError_t launch_gb(const BwdProblem& bp, SbArgs a) {
    const Problem& p = bp.p;
    const unsigned units = unsigned(size_t(a.nseq) * a.nch);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_bwd_sums_kernel<GB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(SumsSmem)));
    if (e != hipSuccess) return e;
    ssd_bwd_sums_kernel<GB><<<dim3(units), dim3(NT), sizeof(SumsSmem), p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t nel4 = size_t(a.nseq) * DK * DV / 4;
    ssd_bwd_scans_kernel<<<dim3(unsigned((nel4 + NT - 1) / NT)), dim3(NT), 0, p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_bwd_grads_kernel<GB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(GradsSmem)));
    if (e != hipSuccess) return e;
    ssd_bwd_grads_kernel<GB><<<dim3(units), dim3(NT), sizeof(GradsSmem), p.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool ssd_backward_mfma_supported(const Problem& p) {
    return p.variant == LA_SSD && p.io_bf16 && p.dk == DK && p.dv == DV;
}

size_t ssd_backward_mfma_workspace_bytes(const Problem& p) {
    if (p.N == 0 || p.B == 0 || p.H == 0) return 0;
    return sb_layout(p).total;
}

hipError_t launch_backward_ssd_mfma(const BwdProblem& bp) {
    const Problem& p = bp.p;
    const size_t nseq = size_t(p.B) * p.H, nch = size_t((p.N + C - 1) / C);
    if (nseq * nch > 0x7fffffffull || nseq * DK * DV / NT > 0x7fffffffull) return hipErrorInvalidValue;
    const SbLayout L = sb_layout(p);
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    SbArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dO = static_cast<const uint16_t*>(bp.dO);
    a.g = p.g;
    a.S0 = p.S0;
    a.dSf = bp.dS_final;
    a.dq = static_cast<uint16_t*>(bp.dq);
    a.dk = static_cast<uint16_t*>(bp.dk);
    a.dv = static_cast<uint16_t*>(bp.dv);
    a.dg = bp.dg;
    a.dS0 = bp.dS0;
    a.Sst = reinterpret_cast<float*>(ws + L.Sst);
    a.dSt = reinterpret_cast<float*>(ws + L.dSt);
    a.Sb = reinterpret_cast<uint16_t*>(ws + L.Sb);
    a.dSb = reinterpret_cast<uint16_t*>(ws + L.dSb);
    a.ac = reinterpret_cast<float*>(ws + L.ac);
    a.N = p.N;
    a.nseq = int(nseq);
    a.nch = int(nch);
    return p.gate_bf16 ? launch_gb<true>(bp, a) : launch_gb<false>(bp, a);
}

}  // namespace la
