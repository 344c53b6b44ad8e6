// Chunked prefill for the diagonal-transition variants on bf16 MFMA (d_k = 128,
// chunk C = 64): normalized Katharopoulos attention (KATH, "Linear / RNN 路线" section
// 2.1) and gated linear attention with a per-key-dim gate (GLA, section 2.2).
//
// A diagonal transition lets a sequence be cut into segments that run in parallel:
// the state entering segment j is an associative scan of per-segment summaries,
//   S_in[j+1] = diag(A_j) S_in[j] + dS_j,   A_j = prod of the gates over segment j,
//   dS_j = sum_{s in seg j} diag(prod_{s < r <= end of seg} g_r) k_s v_s^T
// (KATH: A_j = 1, keys phi(k), and z carried the same way). Two kernels:
//   summary  (seq, segment < P-1, value tile): dS_j, log A_j (and dz_j), walking the
//            segment backwards so that every key is scaled by its suffix decay <= 1
//   forward  (seq, segment, value tile): folds S0 and the earlier summaries into
//            S_in[j] (the scan), then runs the chunked forward; the last segment
//            writes S_final (and z_final)
// Per chunk of the forward pass, with B_r = sum_{s<=r} log g_s (chunk-local, per key dim):
//   P_rs = sum_i q_ri k_si exp(B_ri - B_si)  (s <= r)       [KATH: phi(q_r).phi(k_s)]
//   o_r  = (q_r * exp(B_r))^T S + sum_s P_rs v_s             [KATH: / (phi(q_r).z + sum_s P_rs + eps)]
//   S    = diag(exp(B_last)) S + sum_s diag(exp(B_last - B_s)) k_s v_s^T
// P is formed on the matrix cores from scaled copies of q and k. To keep every scale
// factor bounded the chunk is cut into four 16-row blocks; row block b uses the
// reference rho_b = B at its middle row:
//   q~_r = q_r exp(B_r - rho_b),  k~(b)_s = k_s exp(rho_b - B_s)  (s < 16(b+1))
// so no factor exceeds exp(8 * max |log g|). The matrix-core path clamps log g at
// -10 (g >= 4.5e-5; a gate below that keeps less than 4.5e-5 of the state, so the
// clamp changes no result beyond bf16 rounding) which bounds every factor by e^80.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;
constexpr int PC = C + 8;
constexpr int PB = DK + 4;     // pitch of the fp32 [64][128] gate tile
constexpr float kLogGateMin = -10.f;

// row offset of the k~(b) copy inside the stacked key tile (GLA): 16 + 32 + 48 + 64 rows
__host__ __device__ constexpr int koff(int b) { return 8 * b * (b + 1); }

template <int VAR, int VT>
struct __align__(16) FwdSmem {
    static constexpr int PV = VT + 8;
    static constexpr bool G = VAR == LA_GLA;
    static constexpr int KROWS = G ? 160 : 64;
    __align__(16) uint16_t qt[C * PQ];            // q~ (KATH: phi(q))
    __align__(16) uint16_t qh[G ? C * PQ : 8];    // q^ = q exp(B) (GLA)
    __align__(16) uint16_t kt[KROWS * PQ];        // k~ copies (KATH: phi(k))
    __align__(16) uint16_t kh[G ? C * PQ : 8];    // k^ = k exp(B_last - B) (GLA)
    __align__(16) uint16_t st[VT * PQ];           // S^T [c][i], bf16
    __align__(16) uint16_t v[C * PV];             // V [s][c]
    __align__(16) uint16_t p[C * PC];             // P [r][s]
    // GLA: gate scan; KATH: per-thread column partial sums of phi(k) for z
    __align__(16) float bg[G ? C * PB : 16 * DK];
    // GLA per-column factor tables (chunk-local): rho_b, exp(rho_b), exp(B_last - rho_b),
    // exp(rho_bb - rho_b) for the six pairs b < bb
    __align__(16) float rho[G ? 4 : 1][DK];
    __align__(16) float fq[G ? 4 : 1][DK];
    __align__(16) float fk[G ? 4 : 1][DK];
    __align__(16) float fe[G ? 6 : 1][DK];
    __align__(16) float dec[DK];                  // GLA: exp(B_last); KATH: z
    float psum[G ? 1 : 10][16];                   // KATH: partial row sums of P per tile
    float qz[G ? 1 : C];                          // KATH: phi(q_r).z
};

// index of the pair (b, bb), b < bb, in the exp(rho_bb - rho_b) table
__host__ __device__ constexpr int pair_index(int b, int bb) {
    return b == 0 ? bb - 1 : b == 1 ? bb + 1 : 5;
}

struct DiagArgs {
    const uint16_t *q, *k, *v;
    const void* g;
    const float *S0, *z0;
    uint16_t* o;
    float *S, *z;
    float *dS, *lgA, *dz;  // workspace: segment summaries
    int N, nseq, ntiles, nseg, cps, gate_bf16;
    float eps;
};

// ---------------------------------------------------------------------------
// staging helpers
// ---------------------------------------------------------------------------

// Thread -> (row, 8-column group) for a [64][128] tile, x4 = 0..3.
__device__ __forceinline__ void tile_rc(int tid, int x4, int& r, int& col) {
    const int x = tid + NT * x4;
    r = x >> 4;
    col = (x & 15) * 8;
}

// In-place inclusive (reverse = false) or exclusive-suffix (reverse = true) scan down
// the 64 rows of each column of a fp32 [64][PB] LDS tile; returns via the tile. Two
// threads per column, 32 rows each. Ends with a barrier.
template <bool REVERSE>
__device__ void column_scan(float* bg, int tid) {
    const int col = tid & 127, half = tid >> 7;
    float x[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) x[r] = bg[(half * 32 + r) * PB + col];
    lds_barrier();
    float tot = 0.f;
    if (!REVERSE) {
#pragma unroll
        for (int r = 0; r < 32; ++r) { tot += x[r]; x[r] = tot; }
    } else {
        // exclusive suffix: x[r] <- sum_{r' > r} x[r'] (within this half)
#pragma unroll
        for (int r = 31; r >= 0; --r) { const float t = x[r]; x[r] = tot; tot += t; }
    }
    __shared__ float part[128];
    if (REVERSE ? half == 1 : half == 0) part[col] = tot;
    lds_barrier();
    const float add = (REVERSE ? half == 0 : half == 1) ? part[col] : 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) bg[(half * 32 + r) * PB + col] = x[r] + add;
    lds_barrier();
}

// ---------------------------------------------------------------------------
// summary kernel: dS_j = sum over segment of (k_s * suffix decay)^T v_s
// ---------------------------------------------------------------------------

template <int VAR, int VT>
struct __align__(16) SumSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t kh[C * PQ];
    __align__(16) uint16_t v[C * PV];
    __align__(16) float bg[VAR == LA_GLA ? C * PB : 16 * DK];   // GLA scan / KATH z partials
    float runcol[DK];
};

template <int VAR, int VT, bool GB>
__global__ __launch_bounds__(NT) void diag_summary_kernel(DiagArgs a) {
    constexpr int NVT = VT / 16;
    constexpr int PV = SumSmem<VAR, VT>::PV;
    constexpr int VV = VT / 8;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SumSmem<VAR, VT>& sm = *reinterpret_cast<SumSmem<VAR, VT>*>(smem_raw);
    const int nsum = a.nseg - 1;
    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles * nsum, a.nseq);
    if (!mp.valid) return;
    const int seg = mp.tile / a.ntiles, vtile = mp.tile % a.ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT, c0 = vtile * VT;
    const size_t seq = size_t(mp.seq), tok0 = seq * size_t(a.N);
    const bool gb = a.gate_bf16 != 0;
    const int nchunks = (a.N + C - 1) / C;
    const int ch_lo = seg * a.cps, ch_hi = min(nchunks, ch_lo + a.cps);

    f32x4_t acc[2][NVT];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) acc[ib][ct] = zero4();
    float zacc[8];   // KATH: this thread's column partial sums of phi(k)
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[e] = 0.f;
    if (tid < DK) sm.runcol[tid] = 0.f;   // GLA: sum of log g over the later chunks
    lds_barrier();

    for (int ch = ch_hi - 1; ch >= ch_lo; --ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
        uint4 kraw[4], graw[4][2];
        float lg0[8];
        // loads from clamped rows (always valid, no control flow), padding applied below
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            int r, col;
            tile_rc(tid, x4, r, col);
            const size_t e = (tok0 + t0 + min(r, n - 1)) * DK + col;
            kraw[x4] = ld_g16(a.k + e);
            if (VAR == LA_GLA) ld_gate8_raw<GB>(a.g, e, graw[x4]);
        }
        uint4 vraw[2];
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) vraw[x2] = ld_g16(a.v + (tok0 + t0 + min(r, n - 1)) * DV + c0 + col);
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) *reinterpret_cast<uint4*>(sm.v + r * PV + col) = r < n ? vraw[x2] : zero_u4();
        }
        if (VAR == LA_GLA) {
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4) {
                int r, col;
                tile_rc(tid, x4, r, col);
                float f[8];
                gate8_val<GB>(graw[x4], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) { const float lg = fmaxf(fast_log(f[q]), kLogGateMin); f[q] = r < n ? lg : 0.f; }
                if (x4 == 0) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) lg0[q] = f[q];
                }
                *reinterpret_cast<float4*>(sm.bg + r * PB + col) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4*>(sm.bg + r * PB + col + 4) = make_float4(f[4], f[5], f[6], f[7]);
            }
        }
        if (VAR == LA_GLA) {
            lds_barrier();
            column_scan<true>(sm.bg, tid);   // bg[r][i] = sum_{r' > r in chunk} log g
        }
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            int r, col;
            tile_rc(tid, x4, r, col);
            float f[8];
            unpack8(r < n ? kraw[x4] : zero_u4(), f);
            if (VAR == LA_KATH) {
#pragma unroll
                for (int q = 0; q < 8; ++q) { const float e = elu_plus_one_fast(f[q]); f[q] = r < n ? e : 0.f; }
                // z uses the same bf16-rounded features as the matrix cores
                const uint4 pk = pack8(f);
                float fr[8];
                unpack8(pk, fr);
#pragma unroll
                for (int q = 0; q < 8; ++q) zacc[q] += fr[q];
                *reinterpret_cast<uint4*>(sm.kh + r * PQ + col) = pk;
            } else {
                // suffix decay of key s to the end of the segment, exponent <= 0
                const float4 b0 = *reinterpret_cast<const float4*>(sm.bg + r * PB + col);
                const float4 b1 = *reinterpret_cast<const float4*>(sm.bg + r * PB + col + 4);
                const float4 r0 = *reinterpret_cast<const float4*>(sm.runcol + col);
                const float4 r1 = *reinterpret_cast<const float4*>(sm.runcol + col + 4);
                f[0] *= fast_exp(b0.x + r0.x); f[1] *= fast_exp(b0.y + r0.y);
                f[2] *= fast_exp(b0.z + r0.z); f[3] *= fast_exp(b0.w + r0.w);
                f[4] *= fast_exp(b1.x + r1.x); f[5] *= fast_exp(b1.y + r1.y);
                f[6] *= fast_exp(b1.z + r1.z); f[7] *= fast_exp(b1.w + r1.w);
                *reinterpret_cast<uint4*>(sm.kh + r * PQ + col) = pack8(f);
            }
        }
        lds_barrier();
        // dS += kh^T V  (wave w: key blocks 2w, 2w+1)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = acc[ib][ct];
#pragma unroll
                for (int kk = 0; kk < C / 32; ++kk)
                    s_ = mfma16(frag_kr(sm.kh, PQ, 32 * kk, 16 * (2 * w + ib), lane),
                                frag_kr(sm.v, PV, 32 * kk, 16 * ct, lane), s_);
                acc[ib][ct] = s_;
            }
        if (VAR == LA_GLA && tid < 16) {
            // chunk total of log g = exclusive suffix at row 0 + row 0's own log gate
#pragma unroll
            for (int q = 0; q < 8; ++q) sm.runcol[tid * 8 + q] += sm.bg[tid * 8 + q] + lg0[q];
        }
        lds_barrier();
    }
    // write dS_j tile
    float* dS = a.dS + ((seq * nsum + seg) * DK) * DV;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * w + ib) + 4 * g + j, c = 16 * ct + jl;
                dS[size_t(i) * DV + c0 + c] = acc[ib][ct][j];
            }
    if (vtile == 0) {
        if (VAR == LA_GLA) {
            if (tid < DK) a.lgA[(seq * nsum + seg) * DK + tid] = sm.runcol[tid];
        } else {
            // 16 threads share each 8-column group: reduce over tid >> 4 through LDS
#pragma unroll
            for (int q = 0; q < 8; ++q) sm.bg[(tid >> 4) * DK + (tid & 15) * 8 + q] = zacc[q];
            lds_barrier();
            if (tid < DK) {
                float s_ = 0.f;
#pragma unroll
                for (int x = 0; x < 16; ++x) s_ += sm.bg[x * DK + tid];
                a.dz[(seq * nsum + seg) * DK + tid] = s_;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// forward kernel
// ---------------------------------------------------------------------------

template <int VAR, int VT, bool GB>
__global__ __launch_bounds__(NT) void diag_fwd_kernel(DiagArgs a) {
    constexpr int NVT = VT / 16;
    using Sm = FwdSmem<VAR, VT>;
    constexpr int PV = Sm::PV;
    constexpr int VV = VT / 8;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles * a.nseg, a.nseq);
    if (!mp.valid) return;
    const int seg = mp.tile / a.ntiles, vtile = mp.tile % a.ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT, c0 = vtile * VT;
    const size_t seq = size_t(mp.seq), tok0 = seq * size_t(a.N);
    const bool gb = a.gate_bf16 != 0;
    const int nchunks = (a.N + C - 1) / C;
    const int ch_lo = seg * a.cps, ch_hi = min(nchunks, ch_lo + a.cps);
    const int nsum = a.nseg - 1;

    // entering state: S0, then the summaries of the earlier segments folded in order
    // (S <- diag(A_j) S + dS_j; the scan of the segment-level recurrence)
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
    for (int j = 0; j < seg; ++j) {
        const float* dS = a.dS + ((seq * nsum + j) * DK) * DV;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * (2 * w + ib) + 4 * g + jj;
                const float dec = VAR == LA_GLA ? fast_exp(a.lgA[(seq * nsum + j) * DK + i]) : 1.f;
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct)
                    S[ib][ct][jj] = dec * S[ib][ct][jj] + dS[size_t(i) * DV + c0 + 16 * ct + jl];
            }
    }
    if (VAR == LA_KATH && tid < DK) {
        float z = a.z0 ? a.z0[seq * DK + tid] : 0.f;
        for (int j = 0; j < seg; ++j) z += a.dz[(seq * nsum + j) * DK + tid];
        sm.dec[tid] = z;
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
    uint4 pq[4], pk[4], pv[2], pg[4][2];
    auto load_chunk = [&](int ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            int r, col;
            tile_rc(tid, x4, r, col);
            const size_t e = (tok0 + t0 + min(r, n - 1)) * DK + col;
            pq[x4] = ld_g16(a.q + e);
            pk[x4] = ld_g16(a.k + e);
            if (VAR == LA_GLA) ld_gate8_raw<GB>(a.g, e, pg[x4]);
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) pv[x2] = ld_g16(a.v + (tok0 + t0 + min(r, n - 1)) * DV + c0 + col);
        }
    };
    if (ch_lo < ch_hi) load_chunk(ch_lo);
    lds_barrier();

    for (int ch = ch_lo; ch < ch_hi; ++ch) {
        const int t0 = ch * C, n = min(C, a.N - t0);
        // ---- stage operands
        if (VAR == LA_GLA) {
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4) {
                int r, col;
                tile_rc(tid, x4, r, col);
                float f[8];
                gate8_val<GB>(pg[x4], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) { const float lg = fmaxf(fast_log(f[q]), kLogGateMin); f[q] = r < n ? lg : 0.f; }
                *reinterpret_cast<float4*>(sm.bg + r * PB + col) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4*>(sm.bg + r * PB + col + 4) = make_float4(f[4], f[5], f[6], f[7]);
            }
            lds_barrier();
            column_scan<false>(sm.bg, tid);   // bg[r][i] = B_r (inclusive)
            if (tid < DK) {
                const float bl = sm.bg[(C - 1) * PB + tid];
                float rb[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    rb[b] = sm.bg[(16 * b + 7) * PB + tid];
                    sm.rho[b][tid] = rb[b];
                    sm.fq[b][tid] = fast_exp(rb[b]);
                    sm.fk[b][tid] = fast_exp(bl - rb[b]);
                }
#pragma unroll
                for (int b = 0; b < 3; ++b)
#pragma unroll
                    for (int bb = b + 1; bb < 4; ++bb) sm.fe[pair_index(b, bb)][tid] = fast_exp(rb[bb] - rb[b]);
                sm.dec[tid] = fast_exp(bl);
            }
            lds_barrier();
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4) {
                int r, col;
                tile_rc(tid, x4, r, col);
                const int b = x4;   // rows (tid >> 4) + 16 x4 lie in row block x4
                float q8[8], k8[8], br[8], rho[8], fq[8], fk[8];
                unpack8(r < n ? pq[x4] : zero_u4(), q8);
                unpack8(r < n ? pk[x4] : zero_u4(), k8);
                auto ld8 = [&](const float* src, float (&dst)[8]) {
                    const float4 u0 = *reinterpret_cast<const float4*>(src);
                    const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
                    dst[0] = u0.x; dst[1] = u0.y; dst[2] = u0.z; dst[3] = u0.w;
                    dst[4] = u1.x; dst[5] = u1.y; dst[6] = u1.z; dst[7] = u1.w;
                };
                ld8(sm.bg + r * PB + col, br);
                ld8(sm.rho[b] + col, rho);
                ld8(sm.fq[b] + col, fq);
                ld8(sm.fk[b] + col, fk);
                float qt[8], qh[8], kt[8], kh[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float x = fast_exp(br[q] - rho[q]);   // exp(B_r - rho_b)
                    const float inv = __builtin_amdgcn_rcpf(x);  // exp(rho_b - B_r)
                    qt[q] = q8[q] * x;
                    qh[q] = qt[q] * fq[q];                     // q exp(B_r)
                    kt[q] = k8[q] * inv;                       // k exp(rho_b - B_r)
                    kh[q] = kt[q] * fk[q];                     // k exp(B_last - B_r)
                }
                *reinterpret_cast<uint4*>(sm.qt + r * PQ + col) = pack8(qt);
                *reinterpret_cast<uint4*>(sm.qh + r * PQ + col) = pack8(qh);
                *reinterpret_cast<uint4*>(sm.kh + r * PQ + col) = pack8(kh);
                *reinterpret_cast<uint4*>(sm.kt + (koff(b) + r) * PQ + col) = pack8(kt);
                // k~(bb) = k exp(rho_bb - B_r) for the later row blocks bb
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    if (bb <= b) continue;
                    float fe[8], kb[8];
                    ld8(sm.fe[pair_index(b, bb)] + col, fe);
#pragma unroll
                    for (int q = 0; q < 8; ++q) kb[q] = kt[q] * fe[q];
                    *reinterpret_cast<uint4*>(sm.kt + (koff(bb) + r) * PQ + col) = pack8(kb);
                }
            }
        } else {
            float zp[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) zp[q] = 0.f;
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4) {
                int r, col;
                tile_rc(tid, x4, r, col);
                float f[8];
                unpack8(pq[x4], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) { const float e = elu_plus_one_fast(f[q]); f[q] = r < n ? e : 0.f; }
                *reinterpret_cast<uint4*>(sm.qt + r * PQ + col) = pack8(f);
                unpack8(pk[x4], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) { const float e = elu_plus_one_fast(f[q]); f[q] = r < n ? e : 0.f; }
                const uint4 pk8 = pack8(f);
                *reinterpret_cast<uint4*>(sm.kt + r * PQ + col) = pk8;
                float fr[8];
                unpack8(pk8, fr);   // z uses the bf16 features the matrix cores see
#pragma unroll
                for (int q = 0; q < 8; ++q) zp[q] += fr[q];
            }
            const int col = (tid & 15) * 8;
            *reinterpret_cast<float4*>(sm.bg + (tid >> 4) * DK + col) = make_float4(zp[0], zp[1], zp[2], zp[3]);
            *reinterpret_cast<float4*>(sm.bg + (tid >> 4) * DK + col + 4) = make_float4(zp[4], zp[5], zp[6], zp[7]);
        }
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2) {
            const int x = tid + NT * x2, r = x / VV, col = (x % VV) * 8;
            if (x < C * VV) *reinterpret_cast<uint4*>(sm.v + r * PV + col) = r < n ? pv[x2] : zero_u4();
        }
        lds_barrier();
        if (ch + 1 < ch_hi) load_chunk(ch + 1);

        const uint16_t* QH = VAR == LA_GLA ? sm.qh : sm.qt;
        const uint16_t* KH = VAR == LA_GLA ? sm.kh : sm.kt;

        // ---- P (10 lower tiles) and, for KATH, phi(q).z
        for (int ti = w; ti < 10; ti += 4) {
            const int rb = ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3;
            const int sb = ti - (rb * (rb + 1)) / 2;
            const int kbase = VAR == LA_GLA ? koff(rb) : 0;
            f32x4_t acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                acc = mfma16(frag_kc(sm.kt, PQ, kbase + 16 * sb, 32 * kk, lane),
                             frag_kc(sm.qt, PQ, 16 * rb, 32 * kk, lane), acc);   // D[s][r]
            const int r = 16 * rb + jl;
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * sb + 4 * g + j;
                acc[j] = s <= r ? acc[j] : 0.f;
                rs += acc[j];
            }
            store_dT(sm.p, PC, 16 * sb, 16 * rb, acc, lane);
            if (VAR == LA_KATH) {
                rs += __shfl_xor(rs, 16, 64);
                rs += __shfl_xor(rs, 32, 64);
                if (g == 0) sm.psum[ti][jl] = rs;
            }
        }
        if (VAR == LA_KATH) {
            // phi(q_r) . z with the bf16 features: 4 threads per row
            const int r = tid >> 2, part = tid & 3;
            float acc = 0.f;
#pragma unroll
            for (int q8 = 0; q8 < 4; ++q8) {
                const int col = part * 32 + q8 * 8;
                float f[8];
                unpack8(*reinterpret_cast<const uint4*>(sm.qt + r * PQ + col), f);
                const float4 z0 = *reinterpret_cast<const float4*>(sm.dec + col);
                const float4 z1 = *reinterpret_cast<const float4*>(sm.dec + col + 4);
                acc += f[0] * z0.x + f[1] * z0.y + f[2] * z0.z + f[3] * z0.w;
                acc += f[4] * z1.x + f[5] * z1.y + f[6] * z1.z + f[7] * z1.w;
            }
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            if (part == 0) sm.qz[r] = acc;
        }
        lds_barrier();

        // ---- O^T = S^T Q^^T + V^T P^T  (row block w), then o
        {
            const int r = 16 * w + jl;
            float inv_den = 1.f;
            if (VAR == LA_KATH) {
                float den = sm.qz[r] + a.eps;
                const int tb = (w * (w + 1)) / 2;
                for (int sb = 0; sb <= w; ++sb) den += sm.psum[tb + sb][jl];
                inv_den = 1.f / den;
            }
            const int nk = w < 2 ? 1 : 2;
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    o_ = mfma16(frag_kc(sm.st, PQ, 16 * ct, 32 * kk, lane),
                                frag_kc(QH, PQ, 16 * w, 32 * kk, lane), o_);
                for (int kk = 0; kk < nk; ++kk)
                    o_ = mfma16(frag_kr(sm.v, PV, 32 * kk, 16 * ct, lane),
                                frag_kc(sm.p, PC, 16 * w, 32 * kk, lane), o_);
                if (r < n) {
                    o_ = o_ * inv_den;
                    uint2 wv;
                    wv.x = pack_bf16x2(o_[0], o_[1]);
                    wv.y = pack_bf16x2(o_[2], o_[3]);
                    *reinterpret_cast<uint2*>(a.o + (tok0 + t0 + r) * DV + c0 + 16 * ct + 4 * g) = wv;
                }
            }
        }
        lds_barrier();   // all reads of S^T and z are done

        // ---- S = diag(dec) S + K^^T V; KATH: z += sum of phi(k)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i0 = 16 * (2 * w + ib);
            f32x4_t dec4;
#pragma unroll
            for (int j = 0; j < 4; ++j) dec4[j] = VAR == LA_GLA ? sm.dec[i0 + 4 * g + j] : 1.f;
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * dec4;
#pragma unroll
                for (int kk = 0; kk < C / 32; ++kk)
                    s_ = mfma16(frag_kr(KH, PQ, 32 * kk, i0, lane),
                                frag_kr(sm.v, PV, 32 * kk, 16 * ct, lane), s_);
                S[ib][ct] = s_;
                store_dT(sm.st, PQ, i0, 16 * ct, s_, lane);
            }
        }
        if (VAR == LA_KATH && tid < DK) {
            float s_ = 0.f;
#pragma unroll
            for (int x = 0; x < 16; ++x) s_ += sm.bg[x * DK + tid];
            sm.dec[tid] += s_;
        }
        lds_barrier();
    }

    if (seg == a.nseg - 1) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 16 * (2 * w + ib) + 4 * g + j, c = 16 * ct + jl;
                    a.S[seq * DK * DV + size_t(i) * DV + c0 + c] = S[ib][ct][j];
                }
        if (VAR == LA_KATH && vtile == 0 && tid < DK) a.z[seq * DK + tid] = sm.dec[tid];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// value-tile width: 32 columns (KATH then fits two workgroups per CU in LDS)
int pick_vt(int variant, int dv) {
    (void)variant;
    return dv >= 32 ? 32 : 16;
}

struct WsLayout {
    size_t dS, lgA, dz, total;
};

WsLayout ws_layout(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t nsum = size_t(p.segments > 1 ? p.segments - 1 : 0);
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    WsLayout L{};
    size_t off = 0;
    L.dS = off;  off += al(nseq * nsum * DK * p.dv * 4);
    L.lgA = off; off += al(p.variant == LA_GLA ? nseq * nsum * DK * 4 : 0);
    L.dz = off;  off += al(p.variant == LA_KATH ? nseq * nsum * DK * 4 : 0);
    L.total = nsum ? off : 0;
    return L;
}

template <int VAR, int VT, bool GB>
hipError_t launch_var_vt(const Problem& p) {
    DiagArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.g = p.g;
    a.S0 = p.S0;
    a.z0 = p.z0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    a.z = p.z;
    a.N = p.N;
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24)) return hipErrorInvalidValue;
    a.nseq = int(nseq);
    a.ntiles = p.dv / VT;
    const int nchunks = (p.N + C - 1) / C;
    a.cps = (nchunks + p.segments - 1) / p.segments;
    a.nseg = p.segments;   // exact: every segment holds at least one chunk
    if ((a.nseg - 1) * a.cps >= nchunks) return hipErrorInvalidValue;
    a.gate_bf16 = p.gate_bf16;
    a.eps = p.eps;
    const WsLayout L = ws_layout(p);
    char* ws = static_cast<char*>(p.ws);
    a.dS = reinterpret_cast<float*>(ws + L.dS);
    a.lgA = reinterpret_cast<float*>(ws + L.lgA);
    a.dz = reinterpret_cast<float*>(ws + L.dz);
    hipError_t e;
    if (a.nseg > 1) {
        if (!ws) return hipErrorInvalidValue;
        const size_t smem = sizeof(SumSmem<VAR, VT>);
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&diag_summary_kernel<VAR, VT, GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        diag_summary_kernel<VAR, VT, GB><<<dim3(xcd_grid(a.ntiles * (a.nseg - 1), a.nseq)), dim3(NT), smem,
                                       p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t smem = sizeof(FwdSmem<VAR, VT>);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&diag_fwd_kernel<VAR, VT, GB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    diag_fwd_kernel<VAR, VT, GB><<<dim3(xcd_grid(a.ntiles * a.nseg, a.nseq)), dim3(NT), smem, p.stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_gla(const Problem& p) {
    const bool w32 = pick_vt(LA_GLA, p.dv) == 32;
    if (p.gate_bf16) return w32 ? launch_var_vt<LA_GLA, 32, true>(p) : launch_var_vt<LA_GLA, 16, true>(p);
    return w32 ? launch_var_vt<LA_GLA, 32, false>(p) : launch_var_vt<LA_GLA, 16, false>(p);
}

hipError_t launch_kath(const Problem& p) {
    // KATH has no gates: the gate-dtype parameter is unused
    switch (pick_vt(LA_KATH, p.dv)) {
        case 64: return launch_var_vt<LA_KATH, 64, true>(p);
        case 32: return launch_var_vt<LA_KATH, 32, true>(p);
        default: return launch_var_vt<LA_KATH, 16, true>(p);
    }
}

}  // namespace

bool diag_mfma_supported(int variant, int dk, int dv, bool io_bf16) {
    return io_bf16 && (variant == LA_KATH || variant == LA_GLA) && dk == DK &&
           (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

int diag_mfma_auto_segments(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t tiles = nseq * size_t(p.dv / pick_vt(p.variant, p.dv));
    const int nchunks = (p.N + C - 1) / C;
    // enough chains for two workgroups per CU (KATH) or one (GLA, LDS-bound), but keep
    // at least 4 chunks per segment
    const size_t target = p.variant == LA_KATH ? 512 : 256;
    size_t want = (target + tiles - 1) / tiles;
    const size_t cap = size_t((nchunks + 3) / 4);
    if (want > cap) want = cap;
    return want < 1 ? 1 : int(want);
}

size_t diag_mfma_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

hipError_t launch_prefill_diag_mfma(const Problem& p) {
    return p.variant == LA_GLA ? launch_gla(p) : launch_kath(p);
}

}  // namespace la
