// Chunked prefill for the gated delta rule on bf16 MFMA (d_k = 128, chunk C = 64).
//
// Method ("线性注意力与 SSM", section GDN, rewritten per chunk; the chunkwise UT/WY
// transform that "状态空间与线性注意力" names for delta-rule chunking). For one chunk with
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
//   prep     one workgroup per (sequence, chunk), fully parallel: T = (I + L)^{-1} of
//            every chunk, written to the workspace in bf16 and in MFMA fragment order
//            (T depends only on the chunk's k, alpha, beta, never on the state);
//   forward  one workgroup per (sequence, value tile): walks the chunks in order with
//            its fp32 state tile in MFMA accumulators. Columns of S never mix, so value
//            tiles are independent chains; the tiles of one sequence share an XCD so
//            their q/k/T/P reads hit the same L2.
// Per chunk the forward kernel has three barriers: (S^T q, S^T k) -> X | U = T X and
// the causal score tile P_rs = exp(c_r - c_s) q_r.k_s (s <= r) of the wave's rows |
// O = gamma (S^T q) + P U and S = gamma_last S + K^T U^. Each wave loads the operands
// that only it uses (rows of q, T, V; its own alpha/beta) straight into registers in
// fragment layout through per-sequence buffer resources, two chunks ahead; K and the
// bf16 copy of S^T are shared through LDS. P stays in registers in the order the
// matrix cores return it. Ragged tails need no branches: buffer loads past the
// sequence read zeros and stores past it are dropped.
//
// Fragments whose K index runs along tile rows use the LDS transpose read; result
// tiles are written to LDS with 8-byte stores.
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
    __align__(16) uint16_t k[2][C * PQ];   // K [s][i] of the current and the next chunk
    __align__(16) uint16_t st[VT * PQ];    // S^T [c][i], bf16 copy of the state tile
    __align__(16) uint16_t x[C * PV];      // X [s][c]
    __align__(16) uint16_t u[C * PV];      // U [s][c]
    __align__(16) uint16_t uh[C * PV];     // U scaled by exp(c_last - c_s)
    __align__(16) float cum[8][C];         // each wave's prefix sums of log alpha
};

struct GdnArgs {
    const uint16_t *q, *k, *v;
    const void *alpha, *beta;
    const float* S0;
    uint16_t* o;
    float* S;
    uint16_t* T;   // workspace: [nseq][nchunks][64][64] bf16, T per chunk
    int N, nseq, ntiles, nchunks, gate_bf16;
    const int32_t* cu;   // packed variable-length batch, or null
    int H, L;            // heads; longest sequence (chunk counts are sized for it)
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
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const int t0 = ch * C, n = min(C, sp.len - t0);
    const size_t tok0 = sp.base;
    if (n <= 0) return;   // past this sequence's end: the forward reads zeros instead

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
            const float cr = sm.cum[r], br = sm.beta[r];
            const float4 cs = *reinterpret_cast<const float4*>(sm.cum + 16 * sb + 4 * g);
            const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] *= br * fast_exp(cr - csv[j]);
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
    // T in fragment order: 16-byte piece (rb, kk, lane = 16 g + j) holds row 16 rb + j,
    // columns 32 kk + 8 g .. + 7, so that a wave of the forward kernel reads its B
    // fragment as one contiguous kilobyte
    uint16_t* Tg = a.T + (seq * a.nchunks + ch) * size_t(C * C);
#pragma unroll
    for (int x2 = 0; x2 < 2; ++x2) {
        const int x = tid + NT * x2, rb = x >> 7, kk = (x >> 6) & 1, l = x & 63;
        const int off = (16 * rb + (l & 15)) * PC + 32 * kk + 8 * (l >> 4);
        *reinterpret_cast<uint4*>(Tg + 8 * x) = *reinterpret_cast<const uint4*>(sm.t + off);
    }
}

// ---------------------------------------------------------------------------
// forward kernel
// ---------------------------------------------------------------------------
// Per-chunk operands a wave reads straight from global memory in MFMA fragment layout
// (lane = 16 g + j): rows 16 rb + j of q and T, K halves 8 g .. 8 g + 7 of each 32-wide
// slice; V at the X tile's D layout; the chunk's alpha / beta at lane = token; and this
// thread's share of the chunk's K rows for the LDS copy.
template <int NVT, int KST>
struct ChunkRegs {
    uint4 q[4], t[2], kst[KST];
    uint2 v[NVT];
    uint32_t ga, gb;
};

// Forward kernel. A workgroup owns VT = 16 NVT CG value columns of one sequence and
// runs 4 CG waves: wave w works on row block rb = w % 4 of every chunk (rows of q, T, P,
// key rows 32 rb .. of S) for column group cg = w / 4 (16 NVT columns). The CG column
// groups share the LDS copy of K and load the same q / T lines, so a wider group cuts
// the vector-memory traffic per column.
template <int NVT, int CG, bool GB>
__global__ __launch_bounds__(NT * CG) void gdn_fwd_kernel(GdnArgs a) {
    constexpr int VT = 16 * NVT * CG;
    constexpr int NTW = NT * CG;          // threads per workgroup
    constexpr int KST = (C * DK / 8) / NTW;   // 16-byte K pieces per thread
    constexpr int PV = FwdSmem<VT>::PV;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FwdSmem<VT>& sm = *reinterpret_cast<FwdSmem<VT>*>(smem_raw);

    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles, a.nseq);
    if (!mp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int rb = w & 3, cg = w >> 2;
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT;
    const int cw = 16 * NVT * cg;      // first column of this wave, within the tile
    const int c0 = mp.tile * VT + cw;  // ... and within the row
    const size_t seq = size_t(mp.seq);
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nchunks = (sp.len + C - 1) / C;   // this sequence's chunks
    const int rw = 16 * rb + jl;       // this lane's row of the wave's 16-row block
    const int nk = rb < 2 ? 1 : 2;     // T and P vanish for s >= 16 (rb + 1)

    // state tiles held by this wave: key blocks 2 rb + ib, column tiles ct (D layout)
    f32x4_t S[2][NVT];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * rb + ib) + 4 * g + j, c = colmap<NVT>(ct, jl);
                S[ib][ct][j] = a.S0 ? a.S0[seq * DK * DV + size_t(i) * DV + c0 + c] : 0.f;
            }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
            store_st<NVT>(sm.st, PQ, 16 * (2 * rb + ib), cw, ct, S[ib][ct], lane);

    // Per-sequence buffer resources: rows past the end of the sequence read as zero
    // (the ragged last chunk's padding) and o rows past it are dropped on store.
    const rsrc_t rq = make_rsrc(a.q + tok0 * DK, uint32_t(sp.len) * DK * 2u);
    const rsrc_t rk = make_rsrc(a.k + tok0 * DK, uint32_t(sp.len) * DK * 2u);
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, uint32_t(sp.len) * uint32_t(DV) * 2u);
    const rsrc_t ro = make_rsrc(a.o + tok0 * DV, uint32_t(sp.len) * uint32_t(DV) * 2u);
    const rsrc_t rt = make_rsrc(a.T + seq * size_t(a.nchunks) * size_t(C * C),
                                uint32_t(nchunks) * (C * C * 2u));
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t ra = make_rsrc(static_cast<const char*>(a.alpha) + tok0 * GS, uint32_t(sp.len) * GS);
    const rsrc_t rb_ = make_rsrc(static_cast<const char*>(a.beta) + tok0 * GS, uint32_t(sp.len) * GS);

    // loads of one chunk, all unconditional (a chunk index past the end reads zeros);
    // K first, since its LDS copy is written before the other operands are needed
    // A chunk's loads go out in three parts spread over the processing of the chunk two
    // before it (gates and K, then q, then T and V), so that the memory unit's queue is
    // not handed all of them at once. Each part stays together and in program order:
    // the memory-counter waits before a chunk is used count the loads issued after it.
    auto load_part = [&](ChunkRegs<NVT, KST>& R, int ch, int part) {
        const uint32_t t0 = uint32_t(ch) * C;
        if (part == 0) {
            R.ga = buf_ld_gate<GB>(ra, t0 + lane);
            R.gb = buf_ld_gate<GB>(rb_, t0 + lane);
#pragma unroll
            for (int x4 = 0; x4 < KST; ++x4) {
                const int x = tid + NTW * x4, r = x >> 4, col = (x & 15) * 8;
                R.kst[x4] = buf_ld16(rk, ((t0 + r) * DK + col) * 2u);
            }
        } else if (part == 1) {
            const uint32_t oq = ((t0 + rw) * DK + 8 * g) * 2u;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) R.q[kk] = buf_ld16(rq, oq + 64u * kk);
        } else {
            const uint32_t ot = (uint32_t(ch) * (C * C) + (2 * rb * 64 + lane) * 8) * 2u;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) R.t[kk] = buf_ld16(rt, ot + 1024u * kk);
            const uint32_t ov = ((t0 + rw) * uint32_t(DV) + c0 + colmap<NVT>(0, 4 * g)) * 2u;
            if constexpr (NVT == 2) {
                const uint4 v4 = buf_ld16(rv, ov);
                R.v[0] = make_uint2(v4.x, v4.y);
                R.v[1] = make_uint2(v4.z, v4.w);
            } else {
                R.v[0] = buf_ld8(rv, ov);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_chunk = [&](ChunkRegs<NVT, KST>& R, int ch) {
        load_part(R, ch, 0);
        load_part(R, ch, 1);
        load_part(R, ch, 2);
    };
    auto stage_k = [&](const ChunkRegs<NVT, KST>& R, uint16_t* kb) {
#pragma unroll
        for (int x4 = 0; x4 < KST; ++x4) {
            const int x = tid + NTW * x4, r = x >> 4, col = (x & 15) * 8;
            *reinterpret_cast<uint4*>(kb + r * PQ + col) = R.kst[x4];
        }
    };

    auto process = [&](const ChunkRegs<NVT, KST>& R, const ChunkRegs<NVT, KST>& Rn,
                       ChunkRegs<NVT, KST>& Rl, int ch, int cur) {
        load_part(Rl, ch + 2, 0);
        const int t0 = ch * C, n = min(C, sp.len - t0);
        const uint16_t* kc = sm.k[cur];
        // gates: every wave scans log alpha itself (lane = token); lane (g, j) then
        // takes the values of token 16 rb + j
        const float lg = fast_log(gate_val<GB>(R.ga));
        const float cum = wave_inclusive_scan(lane < n ? lg : 0.f);
        const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 63));
        const float braw = gate_val<GB>(R.gb);
        const float cr = __shfl(cum, rw, 64);
        const float br = rw < n ? __shfl(braw, rw, 64) : 0.f;
        const float gr = fast_exp(cr);
        const float dr = fast_exp(clast - cr);
        const float glast = fast_exp(clast);
        sm.cum[w][lane] = cum;   // read back by this wave only (for the P tiles)

        // ---- (S^T Q^T) and (S^T K^T) for rows 16 rb .. : D[c][r]; the S^T fragment
        // is shared by both products
        f32x4_t oq[NVT], ks[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) { oq[ct] = zero4(); ks[ct] = zero4(); }
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const bf16x8_t kf = frag_kc(kc, PQ, 16 * rb, 32 * kk, lane);
            const bf16x8_t qf = __builtin_bit_cast(bf16x8_t, R.q[kk]);   // rows >= n unused
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                const bf16x8_t sf = frag_st<NVT>(sm.st, PQ, cw, ct, 32 * kk, lane);
                oq[ct] = mfma16(sf, qf, oq[ct]);
                ks[ct] = mfma16(sf, kf, ks[ct]);
            }
        }
        // ---- X[s][c] = beta_s (v_s,c - gamma_s (S^T k_s)_c), s = 16 rb + j
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            const uint2 vv = R.v[ct];
            const float vf[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                                 __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
            f32x4_t x_;
#pragma unroll
            for (int j = 0; j < 4; ++j) x_[j] = br * (vf[j] - gr * ks[ct][j]);
            store_rows<NVT>(sm.x, PV, cw, ct, 16 * rb, x_, lane);   // X[s][c]
        }
        lds_barrier();
        load_part(Rl, ch + 2, 1);

        // ---- U^T = X^T T^T for rows 16 rb .. : D[c][r] -> U[r][c], U^[r][c]
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t u_ = mfma16(frag_kr_cols<NVT>(sm.x, PV, 0, cw, ct, lane),
                                __builtin_bit_cast(bf16x8_t, R.t[0]), zero4());
            if (nk > 1)
                u_ = mfma16(frag_kr_cols<NVT>(sm.x, PV, 32, cw, ct, lane),
                            __builtin_bit_cast(bf16x8_t, R.t[1]), u_);
            store_rows<NVT>(sm.u, PV, cw, ct, 16 * rb, u_, lane);
            store_rows<NVT>(sm.uh, PV, cw, ct, 16 * rb, u_ * dr, lane);
        }
        // ---- P^T tiles of rows 16 rb ..: D[s][r] = exp(c_r - c_s) k_s . q_r (s <= r),
        // kept as B fragments in the order the matrix cores return them
        f32x4_t pt[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            pt[sb] = zero4();
            if (sb <= rb) {
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    pt[sb] = mfma16(frag_kc(kc, PQ, 16 * sb, 32 * kk, lane),
                                    __builtin_bit_cast(bf16x8_t, R.q[kk]), pt[sb]);
                const float4 cs = *reinterpret_cast<const float4*>(sm.cum[w] + 16 * sb + 4 * g);
                const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * sb + 4 * g + j;
                    const float e = fast_exp(cr - csv[j]) * pt[sb][j];
                    pt[sb][j] = s <= rw ? e : 0.f;
                }
            }
        }
        const bf16x8_t pf0 = pack_pk(pt[0], pt[1]), pf1 = pack_pk(pt[2], pt[3]);
        lds_barrier();
        load_part(Rl, ch + 2, 2);

        // ---- O^T = gamma_r (S^T Q^T) + U^T P^T -> o rows 16 rb ..
        uint2 ow[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t o_ = mfma16(frag_kr_cols_pk<NVT>(sm.u, PV, 0, cw, ct, lane), pf0, oq[ct] * gr);
            if (nk > 1) o_ = mfma16(frag_kr_cols_pk<NVT>(sm.u, PV, 1, cw, ct, lane), pf1, o_);
            ow[ct].x = pack_bf16x2(o_[0], o_[1]);
            ow[ct].y = pack_bf16x2(o_[2], o_[3]);
        }
        {
            const uint32_t oo = ((uint32_t(t0) + rw) * uint32_t(DV) + c0 + colmap<NVT>(0, 4 * g)) * 2u;
            if constexpr (NVT == 2) buf_st16(ro, oo, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
            else buf_st8(ro, oo, ow[0]);
        }
        // ---- S = gamma_last S + K^T U^ (key rows 32 rb ..), bf16 copy to st
        bf16x8_t uf[2][NVT];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                uf[kk][ct] = frag_kr_cols<NVT>(sm.uh, PV, 32 * kk, cw, ct, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i0 = 16 * (2 * rb + ib);
            const bf16x8_t kt0 = frag_kr(kc, PQ, 0, i0, lane);
            const bf16x8_t kt1 = frag_kr(kc, PQ, 32, i0, lane);
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * glast;
                s_ = mfma16(kt0, uf[0][ct], s_);
                s_ = mfma16(kt1, uf[1][ct], s_);
                S[ib][ct] = s_;
                store_st<NVT>(sm.st, PQ, i0, cw, ct, s_, lane);
            }
        }
        // next chunk's K into the other buffer (its readers finished before the
        // previous barrier)
        stage_k(Rn, sm.k[cur ^ 1]);
        lds_barrier();
    };

    // three register sets rotate so that each chunk's loads are issued two chunks
    // before it is processed (one chunk of compute is shorter than the memory latency)
    ChunkRegs<NVT, KST> RA, RB, RC;
    load_chunk(RA, 0);
    load_chunk(RB, 1);
    stage_k(RA, sm.k[0]);
    lds_barrier();
    // whole triples only: a chunk past the end reads zeros (alpha = beta = 0 masked to
    // the identity step, T = 0), leaves the state unchanged and stores nothing, so no
    // exit sits between the triple's memory operations
    for (int ch = 0; ch < nchunks; ch += 3) {
        process(RA, RB, RC, ch, ch & 1);
        process(RB, RC, RA, ch + 1, (ch + 1) & 1);
        process(RC, RA, RB, ch + 2, ch & 1);
    }

#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * rb + ib) + 4 * g + j, c = colmap<NVT>(ct, jl);
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
    a.nchunks = (p.L + C - 1) / C;
    a.gate_bf16 = p.gate_bf16;
    a.cu = p.cu;
    a.H = p.H;
    a.L = p.L;
    return a;
}

template <int NVT, int CG, bool GB>
hipError_t launch_cfg(const Problem& p) {
    constexpr int VT = 16 * NVT * CG;
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
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_fwd_kernel<NVT, CG, GB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    gdn_fwd_kernel<NVT, CG, GB>
        <<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(NT * CG), smem, p.stream>>>(a);
    return hipGetLastError();
}

template <bool GB>
hipError_t launch_gb(const Problem& p, bool wide) {
    return wide ? launch_cfg<2, 1, GB>(p) : launch_cfg<1, 1, GB>(p);
}

}  // namespace

bool gdn_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

size_t gdn_mfma_workspace_bytes(const Problem& p) {
    const size_t nchunks = size_t((p.L + C - 1) / C);
    return size_t(p.B) * size_t(p.H) * nchunks * C * C * sizeof(uint16_t);
}

hipError_t launch_prefill_gdn_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 26) || !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's rows and its chunk transforms
    if (size_t(p.L) * DK * 4 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    // Forward shape: each value tile is an independent chain of chunks, so the tile
    // count sets the parallelism, while every tile re-reads the chunk's q, K, T and P
    // through the vector memory path, whose request rate bounds the loop. 32-column
    // tiles on 4 waves (one workgroup per CU at 64 sequences x 128 columns) halve that
    // traffic per column and measure faster than 16-column tiles at two per CU, or
    // 32-column tiles on 8 waves.
    const bool wide = p.dv >= 32;
    if (p.gate_bf16) return launch_gb<true>(p, wide);
    return launch_gb<false>(p, wide);
}

}  // namespace la
