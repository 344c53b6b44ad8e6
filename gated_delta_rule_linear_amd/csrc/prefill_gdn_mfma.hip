// Chunked prefill for the gated delta rule on bf16 MFMA (d_k = 128, chunk C = 64).
//
// Method ("线性注意力与 SSM", section GDN, rewritten per chunk; the chunkwise UT/WY
// transform the survey pages name for delta-rule chunking). For one chunk with
// entering state S (key-major, fp32), local rows r, s = 0..C-1:
//   c_r = sum_{s<=r} log alpha_s,  gamma_r = exp(c_r)
//   L_rs = beta_r exp(c_r - c_s) k_r.k_s  (s < r),   T = (I + L)^{-1}
//   X_r = beta_r (v_r - gamma_r S^T k_r),   U = T X
//   o_r = gamma_r S^T q_r + sum_{s<=r} exp(c_r - c_s) (q_r.k_s) u_s
//   S  <- gamma_{C-1} S + sum_s k_s (exp(c_{C-1} - c_s) u_s)^T
// an exact rewrite of u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t), S_t = alpha_t S_{t-1}
// + k_t u_t^T, o_t = S_t^T q_t. Every exponent is <= 0, so no reciprocal of a
// cumulative decay is ever formed.
//
// T is built blockwise (16-row blocks b = 0..3):
//   * diagonal blocks T_bb = (I + L_bb)^{-1} by forward substitution in fp32, all four
//     at once in one wave (lane = 16 b + column);
//   * T_10 = -T_11 L_10 T_00 and T_32 = -T_33 L_32 T_22 (the two 32 x 32 diagonal
//     inverses A^{-1}, B^{-1});
//   * the lower 32 x 32 block -B^{-1} L[32:64, 0:32] A^{-1} in two products;
// the off-diagonal products run on the matrix cores in bf16 with fp32 accumulation.
//
// Two kernels:
//   prep     one workgroup per (sequence, chunk), fully parallel: L and T = (I + L)^{-1}
//            for every chunk, written to the workspace in bf16 (T depends only on the
//            chunk's k, alpha, beta, never on the state);
//   forward  one workgroup per (sequence, value tile of VT columns): walks the chunks
//            in order with its fp32 state tile in registers (MFMA accumulators).
//            Columns of S never mix, so value tiles are independent chains; the tiles
//            of one sequence share an XCD so their q/k/T reads hit the same L2.
// Taking the triangular inverse out of the sequential loop leaves that loop four
// barriers per chunk of pure matrix-core work; the cost is one extra pass over k
// and a 64 x 64 bf16 T per chunk in HBM.
//
// MFMA products are arranged so that result tiles are written to LDS transposed
// (8-byte writes) and read back as contiguous 16-byte fragments; fragments whose K
// index runs along tile rows use the LDS transpose read.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;     // pitch (elements) of [*][128] bf16 tiles
constexpr int PC = C + 8;      // pitch of [*][64] bf16 tiles
constexpr int PD = 16 + 4;     // pitch of the fp32 16 x 16 diagonal L blocks
constexpr int PY = 32 + 8;     // pitch of the bf16 32-row scratch tiles

struct __align__(16) PrepSmem {
    __align__(16) uint16_t k[C * PQ];
    __align__(16) uint16_t t[C * PC];      // T [r][s]
    __align__(16) uint16_t lo[C * PC];     // off-diagonal blocks of L [r][s]
    __align__(16) uint16_t ya[2][32 * PY];  // level-a scratch: Y = L_ij T_jj (16 rows used)
    __align__(16) uint16_t yb[32 * PY];    // level-b scratch: Y = L[32:64, 0:32] A^{-1}
    __align__(16) float ld[4][16 * PD];    // diagonal blocks of L, fp32
    float cum[C], beta[C];
};

template <int VT>
struct __align__(16) FwdSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t q[C * PQ];
    __align__(16) uint16_t k[C * PQ];
    __align__(16) uint16_t st[VT * PQ];    // S^T [c][i], bf16
    __align__(16) uint16_t v[C * PV];      // V [s][c]
    __align__(16) uint16_t u[C * PV];      // U [s][c]
    __align__(16) uint16_t uh[C * PV];     // U scaled by exp(c_last - c_s)
    __align__(16) uint16_t p[C * PC];      // P [r][s]
    __align__(16) uint16_t t[C * PC];      // T [r][s]
    __align__(16) uint16_t xt[VT * PC];    // X^T [c][s]
    float cum[C], gam[C], beta[C], dec[C];
};

struct GdnArgs {
    const uint16_t *q, *k, *v;
    const void *alpha, *beta;
    const float* S0;
    uint16_t* o;
    float* S;
    uint16_t* T;   // workspace: [nseq][nchunks][64][64] bf16
    int N, nseq, ntiles, nchunks, gate_bf16;
};

// bf16 fragment with the K half 16..31 (lane groups 2, 3) forced to zero: 16 x 16 x 16
// products on the 16 x 16 x 32 instruction.
__device__ __forceinline__ bf16x8_t k16(bf16x8_t f, int lane) {
    if (lane >= 32) {
        const i16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
        return __builtin_bit_cast(bf16x8_t, z);
    }
    return f;
}

// Inclusive scan of log alpha over the chunk by wave 0 (lane = row); padding rows
// carry log alpha = 0.
__device__ __forceinline__ float scan64(float x, int) { return wave_inclusive_scan(x); }

// ---------------------------------------------------------------------------
// prep kernel: T = (I + L)^{-1} per chunk
// ---------------------------------------------------------------------------
template <bool GB>
__global__ __launch_bounds__(NT) void gdn_prep_kernel(GdnArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const size_t seq = blockIdx.x / a.nchunks;
    const int ch = blockIdx.x % a.nchunks;
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok0 = seq * size_t(a.N);

    // loads from clamped rows (always valid), padding applied when staging
    uint4 kv[4];
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        kv[x4] = ld_g16(a.k + (tok0 + t0 + min(r, n - 1)) * DK + col);
    }
    uint32_t graw = 0;
    if (w < 2) graw = ld_gate_raw<GB>(w == 0 ? a.alpha : a.beta, tok0 + t0 + min(lane, n - 1));
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        *reinterpret_cast<uint4*>(sm.k + r * PQ + col) = r < n ? kv[x4] : zero_u4();
    }
    if (w == 0) {
        const float lg = fast_log(gate_val<GB>(graw));
        const float x = lane < n ? lg : 0.f;
        sm.cum[lane] = scan64(x, lane);
    } else if (w == 1) {
        sm.beta[lane] = lane < n ? gate_val<GB>(graw) : 0.f;
    } else {
        // zero the six upper blocks of T and the unused rows of the level-a scratch
        const int r = lane >> 2, cc = (lane & 3) * 4;
        const int ub[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};
        for (int x = w - 2; x < 6; x += 2)
            *reinterpret_cast<uint2*>(sm.t + (16 * ub[x][0] + r) * PC + 16 * ub[x][1] + cc) =
                make_uint2(0, 0);
        uint16_t* y = sm.ya[w - 2];
        for (int x = lane; x < 32 * PY / 4; x += 64) *reinterpret_cast<uint2*>(y + 4 * x) = make_uint2(0, 0);
    }
    lds_barrier();

    if (w == 0) {
        // diagonal blocks of L (fp32): D'[s][r] = k_s . k_r, written as ld[b][r][s..s+3]
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4_t d = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const bf16x8_t kb = frag_kc(sm.k, PQ, 16 * b, 32 * kk, lane);
                d = mfma16(kb, kb, d);
            }
            const int r = 16 * b + jl;
            const float br = sm.beta[r], cr = sm.cum[r];
            float4 val;
            float* vv = reinterpret_cast<float*>(&val);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * b + 4 * g + j;
                const float e = br * fast_exp(cr - sm.cum[s]) * d[j];
                vv[j] = s < r ? e : 0.f;
            }
            *reinterpret_cast<float4*>(sm.ld[b] + jl * PD + 4 * g) = val;
        }
        wave_lds_sync();
        // forward substitution, lane = 16 b + column jc: T_bb[:, jc]
        const int b = g, jc = jl;
        const float* Lb = sm.ld[b];
        float tc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tc[r] = r == jc ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < r; m4 += 4) {
                const float4 l4 = *reinterpret_cast<const float4*>(Lb + r * PD + m4);
                acc += l4.x * tc[m4];
                if (m4 + 1 < r) acc += l4.y * tc[m4 + 1];
                if (m4 + 2 < r) acc += l4.z * tc[m4 + 2];
                if (m4 + 3 < r) acc += l4.w * tc[m4 + 3];
            }
            if (r > jc) tc[r] = -acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.t[(16 * b + r) * PC + 16 * b + jc] = f32_to_bf16(tc[r]);
    } else {
        // waves 1..3: the six off-diagonal L blocks (bf16): D'[s][r] = k_s . k_r -> lo[r][s..]
        for (int task = w - 1; task < 6; task += 3) {
            const int rb = task < 1 ? 1 : task < 3 ? 2 : 3;
            const int sb = task - (rb * (rb - 1)) / 2;
            f32x4_t d = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                d = mfma16(frag_kc(sm.k, PQ, 16 * sb, 32 * kk, lane),
                           frag_kc(sm.k, PQ, 16 * rb, 32 * kk, lane), d);
            const int r = 16 * rb + jl;
            const float br = sm.beta[r], cr = sm.cum[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] *= br * fast_exp(cr - sm.cum[16 * sb + 4 * g + j]);
            store_dT(sm.lo, PC, 16 * sb, 16 * rb, d, lane);
        }
    }
    lds_barrier();
    // level a: T_10 = -T_11 L_10 T_00 (wave 1), T_32 = -T_33 L_32 T_22 (wave 2)
    if (w == 1 || w == 2) {
        const int i = w == 1 ? 1 : 3, j = i - 1;
        uint16_t* y = sm.ya[w - 1];
        // Y^T = T_jj^T L_ij^T -> y[r][jj] (rows 0..15)
        f32x4_t d = mfma16(k16(frag_kr(sm.t, PC, 16 * j, 16 * j, lane), lane),
                           k16(frag_kc(sm.lo, PC, 16 * i, 16 * j, lane), lane), zero4());
        store_dT(y, PY, 0, 0, d, lane);
        wave_lds_sync();
        // T_ij^T = -(Y^T T_ii^T) -> t[16 i + r][16 j + jj]
        d = mfma16(k16(frag_kr(y, PY, 0, 0, lane), lane),
                   k16(frag_kc(sm.t, PC, 16 * i, 16 * i, lane), lane), zero4());
        store_dT(sm.t, PC, 16 * j, 16 * i, -d, lane);
    }
    lds_barrier();
    // level b: Y = L[32:64, 0:32] A^{-1}, tile (rb, jb) per wave
    {
        const int jb = w & 1, rb = w >> 1;
        const f32x4_t d = mfma16(frag_kr(sm.t, PC, 0, 16 * jb, lane),
                                 frag_kc(sm.lo, PC, 32 + 16 * rb, 0, lane), zero4());
        store_dT(sm.yb, PY, 16 * jb, 16 * rb, d, lane);   // Y[r][j]
    }
    lds_barrier();
    // level c: T[32:64, 0:32] = -B^{-1} Y
    {
        const int jb = w & 1, rb = w >> 1;
        const f32x4_t d = mfma16(frag_kr(sm.yb, PY, 0, 16 * jb, lane),
                                 frag_kc(sm.t, PC, 32 + 16 * rb, 32, lane), zero4());
        store_dT(sm.t, PC, 16 * jb, 32 + 16 * rb, -d, lane);
    }
    lds_barrier();
    uint16_t* Tg = a.T + (seq * a.nchunks + ch) * size_t(C * C);
#pragma unroll
    for (int x2 = 0; x2 < 2; ++x2) {
        const int x = tid + NT * x2, r = x >> 3, col = (x & 7) * 8;
        *reinterpret_cast<uint4*>(Tg + r * C + col) = *reinterpret_cast<const uint4*>(sm.t + r * PC + col);
    }
}

// ---------------------------------------------------------------------------
// forward kernel
// ---------------------------------------------------------------------------
template <int VT, bool GB>
__global__ __launch_bounds__(NT) void gdn_fwd_kernel(GdnArgs a) {
    constexpr int NVT = VT / 16;
    constexpr int PV = FwdSmem<VT>::PV;
    constexpr int VV = VT / 8;  // 16-byte vectors per V row
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FwdSmem<VT>& sm = *reinterpret_cast<FwdSmem<VT>*>(smem_raw);

    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles, a.nseq);
    if (!mp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT;
    const int c0 = mp.tile * VT;
    const size_t seq = size_t(mp.seq);
    const size_t tok0 = seq * size_t(a.N);

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
    // zero, once, the P tiles above the diagonal that the row-block products read
    if (w < 2) {
        const int rb = w == 0 ? 0 : 2, sb = rb + 1;
        const int r = 16 * rb + (lane >> 2), s = 16 * sb + (lane & 3) * 4;
        *reinterpret_cast<uint2*>(sm.p + r * PC + s) = make_uint2(0, 0);
    }

    // register prefetch of one chunk: loads from clamped rows (always valid) without
    // control flow, so nothing waits on them until the next chunk is staged
    uint4 pq[4], pk[4], pv[2], pt[2];
    uint32_t pg = 0;
    auto load_chunk = [&](int ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
            const size_t e = (tok0 + t0 + min(r, n - 1)) * DK + col;
            pq[x4] = ld_g16(a.q + e);
            pk[x4] = ld_g16(a.k + e);
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) pv[x2] = ld_g16(a.v + (tok0 + t0 + min(r, n - 1)) * DV + c0 + col);
            const int rt = x >> 3, ctl = (x & 7) * 8;
            pt[x2] = ld_g16(a.T + (seq * a.nchunks + ch) * size_t(C * C) + rt * C + ctl);
        }
        if (tid < 2 * C)
            pg = ld_gate_raw<GB>(tid < C ? a.alpha : a.beta, tok0 + t0 + min(tid & (C - 1), n - 1));
    };

    const int nchunks = a.nchunks;
    if (nchunks > 0) load_chunk(0);
    lds_barrier();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
        // ---- stage: gates (wave 0 scans log alpha, wave 1 holds beta), q, k, v, T
        if (w == 0) {
            const float lg = fast_log(gate_val<GB>(pg));
            const float x = scan64(lane < n ? lg : 0.f, lane);
            const float clast = __shfl(x, 63, 64);
            sm.cum[lane] = x;
            sm.gam[lane] = fast_exp(x);
            sm.dec[lane] = fast_exp(clast - x);
        } else if (w == 1) {
            sm.beta[lane] = lane < n ? gate_val<GB>(pg) : 0.f;
        }
        if (n < C) {   // tail chunk: padding rows are zero
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4) {
                const int r = (tid + NT * x4) >> 4;
                if (r >= n) pq[x4] = pk[x4] = zero_u4();
            }
#pragma unroll
            for (int x2 = 0; x2 < 2; ++x2)
                if ((tid + NT * x2) / VV >= n) pv[x2] = zero_u4();
        }
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
            *reinterpret_cast<uint4*>(sm.q + r * PQ + col) = pq[x4];
            *reinterpret_cast<uint4*>(sm.k + r * PQ + col) = pk[x4];
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) *reinterpret_cast<uint4*>(sm.v + r * PV + col) = pv[x2];
            const int rt = x >> 3, ctl = (x & 7) * 8;
            *reinterpret_cast<uint4*>(sm.t + rt * PC + ctl) = pt[x2];
        }
        lds_barrier();
        if (ch + 1 < nchunks) load_chunk(ch + 1);

        // ---- O^T = S^T Q^T for row block w (scaled by gamma later); P and X tiles
        f32x4_t oacc[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t o_ = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                o_ = mfma16(frag_kc(sm.st, PQ, 16 * ct, 32 * kk, lane),
                            frag_kc(sm.q, PQ, 16 * w, 32 * kk, lane), o_);   // D[c][r]
            oacc[ct] = o_;
        }
        constexpr int NTASK = 10 + 4 * NVT;
        for (int task = w; task < NTASK; task += 4) {
            if (task < 10) {
                // P tile (rb, sb), sb <= rb: D'[s][r] = k_s . q_r -> p[r][s..]
                const int rb = task < 1 ? 0 : task < 3 ? 1 : task < 6 ? 2 : 3;
                const int sb = task - (rb * (rb + 1)) / 2;
                f32x4_t d = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    d = mfma16(frag_kc(sm.k, PQ, 16 * sb, 32 * kk, lane),
                               frag_kc(sm.q, PQ, 16 * rb, 32 * kk, lane), d);
                const int r = 16 * rb + jl;
                const float cr = sm.cum[r];
                const float4 cs = *reinterpret_cast<const float4*>(sm.cum + 16 * sb + 4 * g);
                const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * sb + 4 * g + j;
                    const float e = fast_exp(cr - csv[j]) * d[j];
                    d[j] = s <= r ? e : 0.f;
                }
                store_dT(sm.p, PC, 16 * sb, 16 * rb, d, lane);
            } else {
                // X tile (s block sb, column tile ct): X = beta (V - gamma K S)
                const int xi = task - 10, sb = xi / NVT, ct = xi % NVT;
                f32x4_t d = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    d = mfma16(frag_kc(sm.k, PQ, 16 * sb, 32 * kk, lane),
                               frag_kc(sm.st, PQ, 16 * ct, 32 * kk, lane), d);   // D[s][c]
                const int c = 16 * ct + jl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * sb + 4 * g + j;
                    d[j] = sm.beta[s] * (bf16_to_f32(sm.v[s * PV + c]) - sm.gam[s] * d[j]);
                }
                store_dT(sm.xt, PC, 16 * sb, 16 * ct, d, lane);   // X^T[c][s]
            }
        }
        lds_barrier();

        // ---- U^T = X^T T^T (row block w): U and U scaled by exp(c_last - c_r)
        const int nk = w < 2 ? 1 : 2;   // T and P vanish for s >= 16 (w + 1)
        {
            const int r = 16 * w + jl;
            const float dr = sm.dec[r];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t u_ = zero4();
                for (int kk = 0; kk < nk; ++kk)
                    u_ = mfma16(frag_kc(sm.xt, PC, 16 * ct, 32 * kk, lane),
                                frag_kc(sm.t, PC, 16 * w, 32 * kk, lane), u_);   // D[c][r]
                store_dT(sm.u, PV, 16 * ct, 16 * w, u_, lane);                       // U[r][c]
                store_dT(sm.uh, PV, 16 * ct, 16 * w, u_ * dr, lane);
            }
        }
        lds_barrier();

        // ---- O^T = gamma O^T + U^T P^T -> o;  S = gamma_last S + K^T U^
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
                        s_ = mfma16(frag_kr(sm.k, PQ, 32 * kk, i0, lane),
                                    frag_kr(sm.uh, PV, 32 * kk, 16 * ct, lane), s_);
                    S[ib][ct] = s_;
                    store_dT(sm.st, PQ, i0, 16 * ct, s_, lane);
                }
            }
        }
        lds_barrier();
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

GdnArgs make_args(const Problem& p) {
    GdnArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.alpha = p.g;
    a.beta = p.beta;
    a.S0 = p.S0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    a.T = static_cast<uint16_t*>(p.ws);
    a.N = p.N;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    a.nchunks = (p.N + C - 1) / C;
    a.gate_bf16 = p.gate_bf16;
    return a;
}

template <int VT, bool GB>
hipError_t launch_vt(const Problem& p) {
    GdnArgs a = make_args(p);
    a.ntiles = p.dv / VT;
    hipError_t e;
    {
        const size_t smem = sizeof(PrepSmem);
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_prep_kernel<GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        const size_t blocks = size_t(a.nseq) * size_t(a.nchunks);
        if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
        gdn_prep_kernel<GB><<<dim3(unsigned(blocks)), dim3(NT), smem, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t smem = sizeof(FwdSmem<VT>);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_fwd_kernel<VT, GB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    gdn_fwd_kernel<VT, GB><<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(NT), smem, p.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool gdn_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

size_t gdn_mfma_workspace_bytes(const Problem& p) {
    const size_t nchunks = size_t((p.N + C - 1) / C);
    return size_t(p.B) * size_t(p.H) * nchunks * C * C * sizeof(uint16_t);
}

hipError_t launch_prefill_gdn_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 26) || !p.ws) return hipErrorInvalidValue;
    // value tile: 16 columns keeps the forward kernel's LDS under half a CU, so two
    // workgroups share each CU and hide each other's barrier and LDS latency; 32
    // columns only when 16 would leave more than two waves of workgroups per CU
    const bool wide = p.dv >= 32 && nseq * size_t(p.dv / 16) > 2048;
    if (p.gate_bf16) return wide ? launch_vt<32, true>(p) : launch_vt<16, true>(p);
    return wide ? launch_vt<32, false>(p) : launch_vt<16, false>(p);
}

}  // namespace la
