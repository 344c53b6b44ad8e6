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
    float *Sst, *dSt, *ac;   // [nseq][nch][DK][DV] x 2, [nseq][nch]
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

// rows t0 .. t0 + 63 of a [N][W] bf16 matrix into an LDS tile of pitch P, scaled per row
// by f(row) (padding rows zero); 16-byte pieces
template <int W, int P, typename F>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, size_t tok0, int t0,
                                           int n, F scale) {
    constexpr int PPR = W / 8;   // pieces per row
    for (int p = threadIdx.x; p < C * PPR; p += NT) {
        const int r = p / PPR, cpos = (p % PPR) * 8;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (r < n) w = *reinterpret_cast<const uint4*>(src + (tok0 + t0 + r) * W + cpos);
        const float f = scale(r);
        if (f != 1.f) {
            float x[8];
            unpack8(w, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= f;
            w = pack8(x);
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
    chunk_logs<GB>(sm.c, a, tok0, t0, n);
    __syncthreads();
    const float cl = sm.c[C - 1];
    stage_rows<DK, PQ>(sm.kh, a.k, tok0, t0, n, [&](int r) { return __builtin_amdgcn_exp2f(cl - sm.c[r]); });
    stage_rows<DK, PQ>(sm.qh, a.q, tok0, t0, n, [&](int r) { return __builtin_amdgcn_exp2f(sm.c[r]); });
    stage_rows<DV, PV>(sm.v, a.v, tok0, t0, n, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.dO, a.dO, tok0, t0, n, [](int) { return 1.f; });
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
    const size_t e = size_t(blockIdx.x) * NT + threadIdx.x;
    constexpr size_t SS = size_t(DK) * DV;
    if (e >= size_t(a.nseq) * SS) return;
    const size_t seq = e / SS, ij = e % SS;
    float* Ss = a.Sst + seq * a.nch * SS + ij;
    float* dSs = a.dSt + seq * a.nch * SS + ij;
    const float* ac = a.ac + seq * a.nch;
    float S = a.S0 ? a.S0[e] : 0.f;
    // chunks in batches of SB: a batch's loads are issued before its stores (same array)
    constexpr int SB = 8;
    for (int c0 = 0; c0 < a.nch; c0 += SB) {
        float d[SB], g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            d[b] = c0 + b < a.nch ? Ss[(c0 + b) * SS] : 0.f;
            g[b] = c0 + b < a.nch ? ac[c0 + b] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            if (c0 + b < a.nch) Ss[(c0 + b) * SS] = S;
            S = g[b] * S + d[b];
        }
    }
    float dS = a.dSf ? a.dSf[e] : 0.f;
    for (int c1 = a.nch - 1; c1 >= 0; c1 -= SB) {
        float d[SB], g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            d[b] = c1 - b >= 0 ? dSs[(c1 - b) * SS] : 0.f;
            g[b] = c1 - b >= 0 ? ac[c1 - b] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            if (c1 - b >= 0) dSs[(c1 - b) * SS] = dS;
            dS = g[b] * dS + d[b];
        }
    }
    a.dS0[e] = dS;
}

// ---------------------------------------------------------------------------- grads
struct __align__(16) GradsSmem {
    __align__(16) uint16_t q[C * PQ], k[C * PQ];
    __align__(16) uint16_t v[C * PV], dO[C * PV];
    __align__(16) uint16_t sin[DK * PV], dso[DK * PV];   // S_in, dS_out as [key][column]
    __align__(16) uint16_t P[C * PV], A[C * PV], M[C * PV], Y[C * PV];
    float c[C], alpha[C], beta[C], t2[C];
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
    chunk_logs<GB>(sm.c, a, tok0, t0, n);
    if (tid < C) { sm.alpha[tid] = 0.f; sm.beta[tid] = 0.f; sm.t2[tid] = 0.f; }
    stage_rows<DK, PQ>(sm.q, a.q, tok0, t0, n, [](int) { return 1.f; });
    stage_rows<DK, PQ>(sm.k, a.k, tok0, t0, n, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.v, a.v, tok0, t0, n, [](int) { return 1.f; });
    stage_rows<DV, PV>(sm.dO, a.dO, tok0, t0, n, [](int) { return 1.f; });
    // S_in and dS_out (fp32 in the workspace) as bf16 tiles, and gamma = <dS_out, S_in>
    {
        const size_t base = (seq * a.nch + ch) * size_t(DK) * DV;
        float gam = 0.f;
        for (int p = tid; p < DK * DV / 4; p += NT) {
            const int i = (4 * p) / DV, j = (4 * p) % DV;
            const float4 s4 = *reinterpret_cast<const float4*>(a.Sst + base + 4 * size_t(p));
            const float4 d4 = *reinterpret_cast<const float4*>(a.dSt + base + 4 * size_t(p));
            gam += s4.x * d4.x + s4.y * d4.y + s4.z * d4.z + s4.w * d4.w;
            *reinterpret_cast<uint2*>(sm.sin + i * PV + j) =
                make_uint2(pack_bf16x2(s4.x, s4.y), pack_bf16x2(s4.z, s4.w));
            *reinterpret_cast<uint2*>(sm.dso + i * PV + j) =
                make_uint2(pack_bf16x2(d4.x, d4.y), pack_bf16x2(d4.z, d4.w));
        }
        gam = wave_sum(gam);
        if (lane == 0) sm.red[w] = gam;
    }
    __syncthreads();
    const float cl = sm.c[C - 1];
    const float gamma = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
    auto cm1 = [&](int s) { return s > 0 ? sm.c[s - 1] : 0.f; };
    // Y (elementwise)
    for (int idx = tid; idx < C * C; idx += NT) {
        const int s = idx / C, u = idx % C;
        sm.Y[s * PV + u] = f32_to_bf16(u < s ? __builtin_amdgcn_exp2f(cm1(s) - sm.c[u]) : 0.f);
    }
    // P, A, M: wave w owns rows 16 w .. 16 w + 15
    const int r0 = 16 * w;
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
            const float d = s <= r ? __builtin_amdgcn_exp2f(sm.c[r] - sm.c[s]) : 0.f;
            sm.P[r * PV + s] = f32_to_bf16(qk[e] * d);
            sm.A[r * PV + s] = f32_to_bf16(ov[e] * d);
            sm.M[r * PV + s] = f32_to_bf16(qk[e] * ov[e]);
        }
    }
    __syncthreads();
    auto store_bf = [&](uint16_t* dst, int W, int r, int col, float x) {
        if (r < n) dst[(tok0 + t0 + r) * size_t(W) + col] = f32_to_bf16(x);
    };
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
            store_bf(a.dv, DV, s, 16 * nt + jl, x[e] + __builtin_amdgcn_exp2f(cl - sm.c[s]) * y[e]);
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
            store_bf(a.dq, DK, r, 16 * nt + jl, __builtin_amdgcn_exp2f(sm.c[r]) * x[e] + y[e]);
            store_bf(a.dk, DK, r, 16 * nt + jl, u[e] + __builtin_amdgcn_exp2f(cl - sm.c[r]) * z[e]);
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
                if (s <= r) part += __builtin_amdgcn_exp2f(sm.c[r] - sm.c[s]) * z[e];
            }
            atomicAdd(&sm.t2[s], part);
        }
    }
    __syncthreads();
    if (tid < n) {
        const int s = tid;
        const float es1 = __builtin_amdgcn_exp2f(cm1(s)), fs = __builtin_amdgcn_exp2f(cl - sm.c[s]);
        float t1 = 0.f, t4 = 0.f;
        for (int r = s; r < C; ++r) t1 += __builtin_amdgcn_exp2f(sm.c[r] - sm.c[s]) * sm.alpha[r];
        for (int u = 0; u < s; ++u) t4 += __builtin_amdgcn_exp2f(cm1(s) - sm.c[u]) * sm.beta[u];
        const float da = es1 * t1 + sm.t2[s] + fs * es1 * gamma + fs * t4;
        const size_t e = tok0 + t0 + s;
        if (GB) static_cast<uint16_t*>(a.dg)[e] = f32_to_bf16(da);
        else static_cast<float*>(a.dg)[e] = da;
    }
}

struct SbLayout {
    size_t Sst, dSt, ac, total;
};
SbLayout sb_layout(const Problem& p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t nseq = size_t(p.B) * p.H, nch = size_t((p.N + C - 1) / C);
    SbLayout L{};
    size_t off = 0;
    L.Sst = off; off += al(nseq * nch * DK * DV * 4);
    L.dSt = off; off += al(nseq * nch * DK * DV * 4);
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
    const size_t nel = size_t(a.nseq) * DK * DV;
    ssd_bwd_scans_kernel<<<dim3(unsigned((nel + NT - 1) / NT)), dim3(NT), 0, p.stream>>>(a);
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
    a.ac = reinterpret_cast<float*>(ws + L.ac);
    a.N = p.N;
    a.nseq = int(nseq);
    a.nch = int(nch);
    return p.gate_bf16 ? launch_gb<true>(bp, a) : launch_gb<false>(bp, a);
}

}  // namespace la
