// Chunked prefill for gated linear attention with a per-key-dim gate (GLA, "Linear /
// RNN 路线" section 2.2: S_t = diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t) on bf16
// MFMA, d_k = 128, chunk C = 64.
//
// Per chunk, with B_r = sum_{s<=r} log g_s (chunk-local, per key dim i) and the state S
// entering the chunk:
//   o_r = (q_r * exp(B_r))^T S + sum_{s<=r} P_rs v_s,  P_rs = sum_i q_ri k_si exp(B_ri - B_si)
//   S  <- diag(a) S + sum_s (k_s * exp(B_last - B_s)) v_s^T,  a = exp(B_last)
// an exact rewrite of the token recurrence. Everything that involves the gates depends
// on one chunk's q, k, g only, never on the state, so it is done once per chunk in a
// fully parallel prep kernel; what remains per chunk on the sequential path is three
// dense products on the matrix cores. A diagonal transition also lets the sequence be
// cut into segments that run in parallel: the state entering segment j is
// S_in[j] = sum_{m < j} (prod_{m < l < j} A_l) dS_m + (prod_{l < j} A_l) S0, a sum over
// per-segment summaries (the parallel-scan idea the same page applies to linear
// recurrences). Three kernels:
//   prep     (sequence, chunk): B by a column scan, then q^ = q exp(B), k^ = k exp(B_last
//            - B), a = exp(B_last) and the masked score tile P, all to the workspace;
//   summary  (sequence, segment < last, value tile): dS_j and A_j = prod of a over the
//            segment, by the state update alone from a zero state (segment 0 also
//            copies its tile of S0 to the workspace);
//   forward  (sequence, segment, value tile): S_in[j] from the summaries before it, then
//            per chunk o = q^ S + P V and the state update; the last segment writes
//            S_final. No workgroup that reads S0 runs beside one that writes S_final,
//            so the two may be one buffer.
// P is formed from scaled copies of q and k. To keep every factor bounded the chunk is
// cut into four 16-row blocks; row block b uses the reference rho_b = B at its middle
// row: q~_r = q_r exp(B_r - rho_b), k~(b)_s = k_s exp(rho_b - B_s) for s < 16 (b + 1), so
// no factor exceeds exp(8 max |log g|). log g is clamped at -10 (g >= 4.5e-5: a gate
// below that keeps less than 4.5e-5 of the state, so the clamp changes no result
// beyond bf16 rounding), which bounds every factor by e^80 in fp32.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;     // pitch of [*][128] bf16 tiles
constexpr int PB = DK;         // pitch of the fp32 [64][128] gate tile
constexpr float kLogGateMin = -10.f;

// Workspace of one chunk, written by prep (bytes), each matrix in MFMA fragment order
// so that a wave reads its fragment as one contiguous kilobyte: q^ (piece (rb, kk, lane =
// 16 g + j) = row 16 rb + j, columns 32 kk + 8 g .. + 7), k^ transposed (piece (ib, kk,
// lane) = key dim 16 ib + j, tokens 32 kk + 8 g .. + 7), P (piece (rb, kk, lane) = row
// 16 rb + j, tokens 32 kk + 4 g .. + 3 then 32 kk + 16 + 4 g .. + 3: the order in which
// the matrix cores return the tile, matched by the forward kernel's V fragment), then
// a (fp32).
constexpr uint32_t kWsQ = 0, kWsK = 16384, kWsP = 32768, kWsA = 40960, kWsChunk = 41472;

__host__ __device__ constexpr int pair_index(int b, int bb) {   // (0,1)..(2,3) -> 0..5
    return b == 0 ? bb - 1 : b == 1 ? bb + 1 : 5;
}

struct GlaArgs {
    const uint16_t *q, *k, *v;
    const void* g;
    const float* S0;
    uint16_t* o;
    float* S;
    unsigned char* ws;   // per-chunk prep output
    float* dS;           // [nseq][nseg][tile][DK x VT]: S0, then the segment summaries
    float* A;            // [nseq][nseg - 1][DK]
    int N, nseq, nchunks, nseg, cps, ntiles, DV;
};

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
struct __align__(16) PrepSmem {
    // the fp32 gate tile is dead once every thread holds its B values, so the scaled
    // q / k copies reuse its storage (and k^ reuses q~ once P is done)
    union {
        __align__(16) float bg[C * PB];
        struct {
            __align__(16) uint16_t qt[C * PQ];   // q~ (row block's own reference)
            __align__(16) uint16_t kt[C * PQ];   // k~ (row block's own reference)
        } s;
    } u;
    __align__(16) float rho[4][DK];
    __align__(16) float fq[4][DK];    // exp(rho_b)
    __align__(16) float fk[4][DK];    // exp(B_last - rho_b)
    __align__(16) float fe[6][DK];    // exp(rho_bb - rho_b), b < bb
    __align__(16) float dec[DK];      // exp(B_last)
};

template <bool GB>
__global__ __launch_bounds__(NT) void gla_prep_kernel(GlaArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    // all chunks of a sequence on one XCD, where its later kernels run too
    const XcdMap mp = xcd_map(blockIdx.x, a.nchunks, a.nseq);
    if (!mp.valid) return;
    const size_t seq = size_t(mp.seq);
    const int ch = mp.tile;
    const int t0 = ch * C, n = min(C, a.N - t0);
    const size_t tok0 = seq * size_t(a.N);

    // rows past the end of the sequence read as zero
    const uint32_t rows_left = uint32_t(a.N - t0);
    const rsrc_t rq = make_rsrc(a.q + (tok0 + t0) * DK, rows_left * DK * 2u);
    const rsrc_t rk = make_rsrc(a.k + (tok0 + t0) * DK, rows_left * DK * 2u);
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t rg = make_rsrc(static_cast<const char*>(a.g) + (tok0 + t0) * DK * GS,
                                rows_left * DK * GS);
    uint4 qv[4], kv[4], gv[4][2];
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        const uint32_t e = uint32_t(r * DK + col);
        qv[x4] = buf_ld16(rq, e * 2u);
        kv[x4] = buf_ld16(rk, e * 2u);
        if constexpr (GB) {
            gv[x4][0] = buf_ld16(rg, e * 2u);
        } else {
            gv[x4][0] = buf_ld16(rg, e * 4u);
            gv[x4][1] = buf_ld16(rg, e * 4u + 16u);
        }
    }
    // log g, clamped, zero on padding rows
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        float f[8];
        gate8_val<GB>(gv[x4], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float lg = fmaxf(fast_log(f[q]), kLogGateMin);
            f[q] = r < n ? lg : 0.f;
        }
        *reinterpret_cast<float4*>(sm.u.bg + r * PB + col) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(sm.u.bg + r * PB + col + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    lds_barrier();
    // inclusive scan down each column: a thread takes 4 columns x 8 rows (16-byte LDS
    // accesses), scans them, then adds the totals of the row groups above it
    {
        const int c4 = (tid & 31) * 4, rg = tid >> 5;
        float4 x[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) x[r] = *reinterpret_cast<const float4*>(sm.u.bg + (8 * rg + r) * PB + c4);
#pragma unroll
        for (int r = 1; r < 8; ++r) {
            x[r].x += x[r - 1].x; x[r].y += x[r - 1].y; x[r].z += x[r - 1].z; x[r].w += x[r - 1].w;
        }
        __shared__ float4 part[8][DK / 4];
        part[rg][tid & 31] = x[7];
        lds_barrier();
        float4 add = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q = 0; q < rg; ++q) {
            const float4 t = part[q][tid & 31];
            add.x += t.x; add.y += t.y; add.z += t.z; add.w += t.w;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            x[r].x += add.x; x[r].y += add.y; x[r].z += add.z; x[r].w += add.w;
            *reinterpret_cast<float4*>(sm.u.bg + (8 * rg + r) * PB + c4) = x[r];
        }
    }
    lds_barrier();
    if (tid < DK) {
        const float bl = sm.u.bg[(C - 1) * PB + tid];
        float rb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            rb[b] = sm.u.bg[(16 * b + 7) * PB + tid];
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
    // every thread takes its B values before the gate tile is overwritten
    float br[4][8];
    uint4 khp[4];
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        const float4 u0 = *reinterpret_cast<const float4*>(sm.u.bg + r * PB + col);
        const float4 u1 = *reinterpret_cast<const float4*>(sm.u.bg + r * PB + col + 4);
        br[x4][0] = u0.x; br[x4][1] = u0.y; br[x4][2] = u0.z; br[x4][3] = u0.w;
        br[x4][4] = u1.x; br[x4][5] = u1.y; br[x4][6] = u1.z; br[x4][7] = u1.w;
    }
    lds_barrier();

    unsigned char* wsc = a.ws + (seq * a.nchunks + ch) * size_t(kWsChunk);
    auto ld8 = [&](const float* src, float (&dst)[8]) {
        const float4 u0 = *reinterpret_cast<const float4*>(src);
        const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
        dst[0] = u0.x; dst[1] = u0.y; dst[2] = u0.z; dst[3] = u0.w;
        dst[4] = u1.x; dst[5] = u1.y; dst[6] = u1.z; dst[7] = u1.w;
    };
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        const int b = x4;   // rows (tid >> 4) + 16 x4 lie in row block x4
        float q8[8], k8[8], rho[8], fq[8], fk[8];
        unpack8(qv[x4], q8);   // padding rows read as zero
        unpack8(kv[x4], k8);
        ld8(sm.rho[b] + col, rho);
        ld8(sm.fq[b] + col, fq);
        ld8(sm.fk[b] + col, fk);
        float qt[8], qh[8], kt[8], kh[8];   // k^ stays in registers until after P
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float e = fast_exp(br[x4][q] - rho[q]);   // exp(B_r - rho_b)
            const float inv = __builtin_amdgcn_rcpf(e);      // exp(rho_b - B_r)
            qt[q] = q8[q] * e;
            qh[q] = qt[q] * fq[q];                          // q exp(B_r)
            kt[q] = k8[q] * inv;                            // k exp(rho_b - B_r)
            kh[q] = kt[q] * fk[q];                          // k exp(B_last - B_r)
        }
        *reinterpret_cast<uint4*>(sm.u.s.qt + r * PQ + col) = pack8(qt);
        *reinterpret_cast<uint4*>(sm.u.s.kt + r * PQ + col) = pack8(kt);
        // q^ in fragment order, k^ row-major
        const int jr = r & 15, kk = col >> 5, gg = (col & 31) >> 3;
        *reinterpret_cast<uint4*>(wsc + kWsQ + (((r >> 4) * 4 + kk) * 64 + 16 * gg + jr) * 16) = pack8(qh);
        khp[x4] = pack8(kh);
    }
    if (tid < DK / 4)
        *reinterpret_cast<float4*>(wsc + kWsA + tid * 16) = *reinterpret_cast<const float4*>(sm.dec + 4 * tid);
    lds_barrier();
    // P: ten lower tiles, D'[s][r] = k~_s . q~_r exp(rho_rb - rho_sb) for key block sb <
    // row block rb (the q~ fragment rescaled on the fly, a factor <= 1), stored straight
    // from the accumulators as half pieces; the two upper half pieces the forward
    // kernel reads, (0, 1) and (2, 3), are written as zeros
    // (unrolled over a wave's up to three tiles so that their MFMA chains interleave)
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) {
        const int ti = w + 4 * tt;
        if (ti >= 10) continue;
        const int rb = ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3;
        const int sb = ti - (rb * (rb + 1)) / 2;
        f32x4_t acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            bf16x8_t qb = frag_kc(sm.u.s.qt, PQ, 16 * rb, 32 * kk, lane);
            if (sb < rb) {
                float f[8], fe[8];
                unpack8(__builtin_bit_cast(uint4, qb), f);
                ld8(sm.fe[pair_index(sb, rb)] + 32 * kk + 8 * g, fe);
#pragma unroll
                for (int q = 0; q < 8; ++q) f[q] *= fe[q];
                qb = __builtin_bit_cast(bf16x8_t, pack8(f));
            }
            acc = mfma16(frag_kc(sm.u.s.kt, PQ, 16 * sb, 32 * kk, lane), qb, acc);
        }
        const int r = 16 * rb + jl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = 16 * sb + 4 * g + j;
            acc[j] = s <= r ? acc[j] : 0.f;
        }
        unsigned char* piece = wsc + kWsP + ((rb * 2 + (sb >> 1)) * 64 + lane) * 16;
        *reinterpret_cast<uint2*>(piece + (sb & 1) * 8) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        if (sb == rb && (rb & 1) == 0) *reinterpret_cast<uint2*>(piece + 8) = make_uint2(0, 0);
    }
    lds_barrier();
    // k^ row-major into the (now dead) q~ storage, then transposed out
    uint16_t* kht = sm.u.s.qt;
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
        const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
        *reinterpret_cast<uint4*>(kht + r * PQ + col) = khp[x4];
    }
    lds_barrier();
    // k^ transposed, in fragment order: wave w writes key blocks 2 w, 2 w + 1
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int blk = 2 * w + ib;
            const bf16x8_t f = frag_kr(kht, PQ, 32 * kk, 16 * blk, lane);
            *reinterpret_cast<uint4*>(wsc + kWsK + ((blk * 2 + kk) * 64 + lane) * 16) =
                __builtin_bit_cast(uint4, f);
        }
}

// ---------------------------------------------------------------------------
// summary (OUT = false) and forward (OUT = true): the chunk walk of one segment
// ---------------------------------------------------------------------------
template <int VT>
struct __align__(16) ChainSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t v[2][C * PV];    // V [s][c]
    __align__(16) uint16_t st[2][VT * PQ];  // S^T [c][i], bf16 (forward only)
    __align__(16) float a[2][DK];           // chunk decay exp(B_last)
};

// One chunk's operands in registers: the wave's k^T fragments (state update, key rows
// 32 w ..), q^ and P fragments (forward), this thread's V pieces and decay piece for the
// LDS copies.
template <int KV>
struct ChainRegs {
    uint4 kt[4], qf[4], pf[2], vst[KV], ast;
};

template <bool OUT, int NVT>
__global__ __launch_bounds__(NT) void gla_chain_kernel(GlaArgs a) {
    constexpr int VT = 16 * NVT;
    constexpr int PV = ChainSmem<VT>::PV;
    constexpr int KV = VT >= 32 ? VT / 32 : 1;   // 16-byte V pieces per thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainSmem<VT>& sm = *reinterpret_cast<ChainSmem<VT>*>(smem_raw);

    const int nrun = OUT ? a.nseg : a.nseg - 1;   // segments this kernel walks
    // all (segment, tile) units of a sequence on the XCD that prepared its chunks
    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles * nrun, a.nseq);
    if (!mp.valid) return;
    const int seq = mp.seq, seg = mp.tile / a.ntiles, tile = mp.tile % a.ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.DV;
    const int c0 = tile * VT;
    const size_t tok0 = size_t(seq) * size_t(a.N);
    const int ch0 = seg * a.cps, ch1 = min(a.nchunks, ch0 + a.cps);
    const int nloc = ch1 - ch0;
    const int nk = w < 2 ? 1 : 2;   // P rows 16 w .. vanish for s >= 16 (w + 1)
    const int rw = 16 * w + jl;

    // state tile: key rows 16 (2 w + ib) + 4 g + j, columns c0 + colmap(ct, jl)
    f32x4_t S[2][NVT];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) S[ib][ct] = zero4();
    // Segment state slots, in this kernel's register order (slot m, tile: the float4
    // (ib NVT + ct) NT + tid): slot 0 holds S0's tile, slot m + 1 the summary dS_m.
    float4* const slots = reinterpret_cast<float4*>(a.dS) +
                          (size_t(seq) * a.nseg * a.ntiles + tile) * (DK * VT / 4);
    const size_t slot_stride = size_t(a.ntiles) * (DK * VT / 4);
    auto S0_elem = [&](int ib, int ct, int j) {
        const int i = 16 * (2 * w + ib) + 4 * g + j, c = c0 + colmap<NVT>(ct, jl);
        return a.S0[size_t(seq) * DK * DV + size_t(i) * DV + c];
    };
    float aprod[2][4];   // running product of the chunk decays (summary)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int j = 0; j < 4; ++j) aprod[ib][j] = 1.f;

    // Every load is unconditional: the workspace resource covers this segment's chunks
    // only, so a prefetch past the segment reads zeros.
    const rsrc_t rw_ = make_rsrc(a.ws + (size_t(seq) * a.nchunks + ch0) * kWsChunk,
                                 uint32_t(nloc) * kWsChunk);
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, uint32_t(a.N) * uint32_t(DV) * 2u);
    const uint32_t obytes = uint32_t(a.N) * uint32_t(DV) * 2u;
    const rsrc_t ro = make_rsrc(a.o + tok0 * DV, obytes);
    if (!OUT && seg == 0 && a.S0) {
        // the forward reads S0 from slot 0, so S_final may alias S0
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                slots[(ib * NVT + ct) * NT + tid] = make_float4(S0_elem(ib, ct, 0), S0_elem(ib, ct, 1),
                                                                S0_elem(ib, ct, 2), S0_elem(ib, ct, 3));
    }

    auto load_chunk = [&](ChainRegs<KV>& R, int lc) {   // lc: chunk index within the segment
        const uint32_t cb = uint32_t(lc) * kWsChunk;
        const uint32_t t0 = uint32_t(ch0 + lc) * C;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                R.kt[2 * ib + kk] =
                    buf_ld16(rw_, cb + kWsK + uint32_t(((2 * w + ib) * 2 + kk) * 64 + lane) * 16u);
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            // V pieces: 64 rows x VT columns in 16-byte pieces, VT / 8 per row; with
            // VT = 16 the upper half of the threads reads past the range (zeros, unused)
            const int id = tid + NT * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
            const uint32_t off = VT >= 32 || id < C * VT / 8
                                     ? ((t0 + r) * uint32_t(DV) + c0 + col) * 2u : obytes;
            R.vst[x] = buf_ld16(rv, off);
        }
        R.ast = buf_ld16(rw_, tid < DK / 4 ? cb + kWsA + uint32_t(tid) * 16u
                                           : uint32_t(nloc) * kWsChunk);
        if (OUT) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                R.qf[kk] = buf_ld16(rw_, cb + kWsQ + uint32_t((w * 4 + kk) * 64 + lane) * 16u);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                R.pf[kk] = buf_ld16(rw_, cb + kWsP + uint32_t((w * 2 + kk) * 64 + lane) * 16u);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](const ChainRegs<KV>& R, int buf) {
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            const int id = tid + NT * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
            if (VT >= 32 || id < C * VT / 8)
                *reinterpret_cast<uint4*>(sm.v[buf] + r * PV + col) = R.vst[x];
        }
        if (tid < DK / 4) *reinterpret_cast<uint4*>(sm.a[buf] + 4 * tid) = R.ast;
    };

    auto process = [&](const ChainRegs<KV>& R, const ChainRegs<KV>& Rn, int lc, int cur) {
        const uint16_t* vv = sm.v[cur];
        if (OUT) {
            // O^T = S^T q^^T + V^T P^T for rows 16 w ..; 4 NVT contiguous columns per lane
            uint2 ow[NVT];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    o_ = mfma16(frag_st<NVT>(sm.st[cur], PQ, 0, ct, 32 * kk, lane),
                                __builtin_bit_cast(bf16x8_t, R.qf[kk]), o_);
                o_ = mfma16(frag_kr_cols_pk<NVT>(vv, PV, 0, 0, ct, lane),
                            __builtin_bit_cast(bf16x8_t, R.pf[0]), o_);
                if (nk > 1)
                    o_ = mfma16(frag_kr_cols_pk<NVT>(vv, PV, 1, 0, ct, lane),
                                __builtin_bit_cast(bf16x8_t, R.pf[1]), o_);
                ow[ct].x = pack_bf16x2(o_[0], o_[1]);
                ow[ct].y = pack_bf16x2(o_[2], o_[3]);
            }
            const uint32_t orow = ((uint32_t(ch0 + lc) * C + rw) * uint32_t(DV) + c0 + 4 * NVT * g) * 2u;
            if constexpr (NVT == 4) {
                buf_st16(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
                buf_st16(ro, orow + 16u, make_uint4(ow[2].x, ow[2].y, ow[3].x, ow[3].y));
            } else if constexpr (NVT == 2) {
                buf_st16(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
            } else {
                buf_st8(ro, orow, ow[0]);
            }
        }
        // S = diag(a) S + K^^T V (key rows 32 w ..)
        bf16x8_t vf[2][NVT];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) vf[kk][ct] = frag_kr_cols<NVT>(vv, PV, 32 * kk, 0, ct, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i0 = 16 * (2 * w + ib);
            const float4 a4 = *reinterpret_cast<const float4*>(sm.a[cur] + i0 + 4 * g);
            const f32x4_t av = {a4.x, a4.y, a4.z, a4.w};
            if (!OUT) {
#pragma unroll
                for (int j = 0; j < 4; ++j) aprod[ib][j] *= av[j];
            }
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * av;
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kt[2 * ib]), vf[0][ct], s_);
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kt[2 * ib + 1]), vf[1][ct], s_);
                S[ib][ct] = s_;
                if (OUT) store_st<NVT>(sm.st[cur ^ 1], PQ, i0, 0, ct, s_, lane);
            }
        }
        stage(Rn, cur ^ 1);
        lds_barrier();
    };

    // three register sets rotate: each chunk's loads go out two chunks before it is
    // processed (a prefetch past the segment reads zeros and is never processed)
    ChainRegs<KV> RA, RB, RC;
    load_chunk(RA, 0);
    load_chunk(RB, 1);
    if (OUT) {
        if (a.nseg == 1) {
            if (a.S0) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j) S[ib][ct][j] = S0_elem(ib, ct, j);
            }
        } else {
            // state entering segment seg, from the summaries of the segments before it:
            // S_in = sum_m (prod_{l > m} A_l) dS_m + (prod_l A_l) S0, newest first, two
            // summaries per batch of loads
            float dcur[2][4];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int j = 0; j < 4; ++j) dcur[ib][j] = 1.f;
            const float* Abase = a.A + size_t(seq) * (a.nseg - 1) * DK + 16 * (2 * w) + 4 * g;
            for (int m = seg - 1; m >= 0; m -= 2) {
                float4 ds[2][2][NVT], am[2][2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int mm = max(m - u, 0);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                        for (int ct = 0; ct < NVT; ++ct)
                            ds[u][ib][ct] = slots[(mm + 1) * slot_stride + (ib * NVT + ct) * NT + tid];
                        am[u][ib] = *reinterpret_cast<const float4*>(Abase + size_t(mm) * DK + 16 * ib);
                    }
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (m - u < 0) break;
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const float av[4] = {am[u][ib].x, am[u][ib].y, am[u][ib].z, am[u][ib].w};
#pragma unroll
                        for (int ct = 0; ct < NVT; ++ct) {
                            const float dv4[4] = {ds[u][ib][ct].x, ds[u][ib][ct].y, ds[u][ib][ct].z,
                                                  ds[u][ib][ct].w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) S[ib][ct][j] += dcur[ib][j] * dv4[j];
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) dcur[ib][j] *= av[j];
                    }
                }
            }
            if (a.S0) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int ct = 0; ct < NVT; ++ct) {
                        const float4 x = slots[(ib * NVT + ct) * NT + tid];
                        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) S[ib][ct][j] += dcur[ib][j] * xv[j];
                    }
            }
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                store_st<NVT>(sm.st[0], PQ, 16 * (2 * w + ib), 0, ct, S[ib][ct], lane);
    }
    stage(RA, 0);
    lds_barrier();
    for (int lc = 0; lc < nloc; lc += 3) {
        load_chunk(RC, lc + 2);
        process(RA, RB, lc, lc & 1);
        if (lc + 1 >= nloc) break;
        load_chunk(RA, lc + 3);
        process(RB, RC, lc + 1, (lc + 1) & 1);
        if (lc + 2 >= nloc) break;
        load_chunk(RB, lc + 4);
        process(RC, RA, lc + 2, lc & 1);
    }

    if (OUT) {
        if (seg == a.nseg - 1) {
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 16 * (2 * w + ib) + 4 * g + j, c = c0 + colmap<NVT>(ct, jl);
                        a.S[size_t(seq) * DK * DV + size_t(i) * DV + c] = S[ib][ct][j];
                    }
        }
    } else {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                slots[(seg + 1) * slot_stride + (ib * NVT + ct) * NT + tid] =
                    make_float4(S[ib][ct][0], S[ib][ct][1], S[ib][ct][2], S[ib][ct][3]);
        if (tile == 0 && jl == 0) {
            float* A = a.A + (size_t(seq) * (a.nseg - 1) + seg) * DK;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int j = 0; j < 4; ++j) A[16 * (2 * w + ib) + 4 * g + j] = aprod[ib][j];
        }
    }
}

struct WsLayout {
    size_t chunks, dS, A, total;
};
WsLayout ws_layout(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t nchunks = size_t((p.N + C - 1) / C);
    const size_t nsum = size_t(p.segments > 1 ? p.segments - 1 : 0);
    const size_t nslot = p.segments > 1 ? size_t(p.segments) : 0;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L{};
    L.chunks = 0;
    size_t off = al(nseq * nchunks * kWsChunk);
    L.dS = off;
    off += al(nseq * nslot * DK * size_t(p.dv) * 4);
    L.A = off;
    off += al(nseq * nsum * DK * 4);
    L.total = off;
    return L;
}

int pick_nvt(int dv) { return dv >= 64 ? 4 : dv / 16; }

template <bool GB, int NVT>
hipError_t launch_nvt(const Problem& p) {
    constexpr int VT = 16 * NVT;
    const WsLayout L = ws_layout(p);
    GlaArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.g = p.g;
    a.S0 = p.S0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    a.ws = ws + L.chunks;
    a.dS = reinterpret_cast<float*>(ws + L.dS);
    a.A = reinterpret_cast<float*>(ws + L.A);
    a.N = p.N;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    a.nchunks = (p.N + C - 1) / C;
    a.nseg = p.segments;
    a.cps = (a.nchunks + a.nseg - 1) / a.nseg;
    a.DV = p.dv;
    a.ntiles = p.dv / VT;
    hipError_t e;
    {
        const size_t smem = sizeof(PrepSmem);
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_prep_kernel<GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        const size_t blocks = size_t(xcd_grid(a.nchunks, (a.nseq + 7) & ~7));
        if (size_t(a.nseq + 7) * size_t(a.nchunks) > 0x7fffffffull) return hipErrorInvalidValue;
        gla_prep_kernel<GB><<<dim3(unsigned(blocks)), dim3(NT), smem, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t smem = sizeof(ChainSmem<VT>);
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_chain_kernel<false, NVT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        gla_chain_kernel<false, NVT><<<dim3(xcd_grid(a.ntiles * (a.nseg - 1), a.nseq)), dim3(NT),
                                       smem, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_chain_kernel<true, NVT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    gla_chain_kernel<true, NVT><<<dim3(xcd_grid(a.ntiles * a.nseg, a.nseq)), dim3(NT), smem,
                                  p.stream>>>(a);
    return hipGetLastError();
}

template <bool GB>
hipError_t launch_gb(const Problem& p) {
    switch (pick_nvt(p.dv)) {
        case 1: return launch_nvt<GB, 1>(p);
        case 2: return launch_nvt<GB, 2>(p);
        default: return launch_nvt<GB, 4>(p);
    }
}

}  // namespace

bool gla_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

size_t gla_mfma_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

int gla_mfma_auto_segments(const Problem& p) {
    // enough (sequence, segment, value tile) units for one workgroup per CU, with at
    // least two chunks per segment
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t ntiles = size_t(p.dv / (16 * pick_nvt(p.dv)));
    const size_t nchunks = size_t((p.N + C - 1) / C);
    const size_t units = nseq * ntiles;
    size_t want = (256 + units - 1) / units;
    const size_t cap = nchunks / 2;
    if (want > cap) want = cap;
    return want < 1 ? 1 : int(want);
}

hipError_t launch_prefill_gla_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24) || !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's v / o rows and its chunk workspace
    if (size_t(p.N) * size_t(p.dv) * 2 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    if (size_t((p.N + C - 1) / C) * kWsChunk >= (size_t(1) << 31)) return hipErrorInvalidValue;
    return p.gate_bf16 ? launch_gb<true>(p) : launch_gb<false>(p);
}

}  // namespace la
