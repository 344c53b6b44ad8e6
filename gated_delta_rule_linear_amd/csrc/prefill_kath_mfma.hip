// Chunked prefill for normalized Katharopoulos linear attention (KATH: phi = ELU + 1,
// "Linear / RNN 路线" section 2.1; "线性注意力与 SSM" section 02 for the normalized form
// with epsilon) on bf16 MFMA, d_k = 128, chunk C = 64.
//
// Per chunk, with phi applied to q and k (padding rows are identity steps: phi rows 0)
// and the state (S, z) entering the chunk:
//   P_rs = phi(q_r) . phi(k_s)  (s <= r)
//   o_r  = (phi(q_r)^T S + sum_s P_rs v_s) / (phi(q_r) . z + sum_s P_rs + eps)
//   S   += sum_s phi(k_s) v_s^T,   z += sum_s phi(k_s)
// an exact rewrite of the token recurrence with the post-update read. The transition is
// the identity, so a sequence cuts into segments that run in parallel: the state
// entering segment j is the sum of S0 and the earlier segments' summaries. Three
// kernels, all placing one sequence's work on one XCD:
//   summary  (sequence, segment < last, value tile): dS_j = sum phi(k)^T V over the
//            segment and dz_j = sum phi(k);
//   scan     (sequence, state element): S_in[j] and z_in[j] for every segment, in place
//            over the summaries;
//   forward  (sequence, segment, value tile): from (S_in[j], z_in[j]), per chunk the
//            output and the state update; the last segment writes S_final and z_final.
// phi is computed where the chunk is staged, in both chain kernels: it is one exponential
// per element, cheaper than a pass that would write phi(q), phi(k) to memory.
#include <cstddef>

#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 16;    // pitch of [*][128] bf16 tiles (72 dwords: 16-byte reads of 16 rows
                               // at one column are free of bank conflicts)

struct KathArgs {
    const uint16_t *q, *k, *v;
    const float *S0, *z0;
    uint16_t* o;
    float *S, *z;
    float* dS;   // [nseq][nseg][DK][DV]: S0, then the summaries; after the scan S_in[j]
    float* dz;   // [nseq][nseg][DK]: likewise for z
    float eps;
    int N, nseq, nchunks, nseg, cps, ntiles, DV;
    const int32_t* cu;   // packed variable-length batch, or null
    int H, L;            // heads; longest sequence (chunk counts are sized for it)
};

// The summary kernel uses only the fields up to `qt`, and is launched with that much
// LDS. NW = waves per workgroup. S^T is kept in fragment order per column group: piece
// (cg, kk, ct, lane = 16 g + L) holds column colmap(ct, L) of the group and key rows
// 32 kk + 4 g .. + 3, 32 kk + 16 + 4 g .. + 3, which is what lane (g, L) of the group's
// wave with row block kk holds in its two state tiles; so each lane writes one
// contiguous 16-byte piece and each reader loads one (the matching phi(q) fragments are
// read as two 8-byte halves).
template <int VT, int NW>
struct __align__(16) ChainSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t kt[2][C * PQ];          // phi(k) [s][i]
    __align__(16) uint16_t v[2][C * PV];           // V [s][c]
    __align__(16) float zp[2][NW][DK];             // per-wave column sums of phi(k)
    __align__(16) float z[2][DK];                  // z entering the chunk
    __align__(16) uint16_t qt[2][C * PQ];          // phi(q) [r][i] (forward)
    __align__(16) uint4 st[2][VT / 16 * 4 * 64];   // S^T fragments, bf16 (forward)
};

template <int KST, int KV>
struct ChainRegs {
    uint4 kst[KST], qst[KST], vst[KV];
};

// A workgroup owns VT = 16 NVT CG value columns of one (sequence, segment) and runs
// 4 CG waves: wave w takes row block rb = w % 4 (output rows 16 rb .., state key rows
// 32 rb ..) of column group cg = w / 4 (16 NVT columns). The column groups share the
// staged phi(q), phi(k) and V; each wave forms the score tiles of its own row block in
// registers (the two waves of a row block both do), with their row sums, and phi(q) . z
// for its rows, so that nothing but the staged chunk and S^T passes through LDS and one
// barrier per chunk suffices.
template <bool OUT, int NVT, int CG>
__global__ __launch_bounds__(NT * CG) void kath_chain_kernel(KathArgs a) {
    constexpr int VT = 16 * NVT * CG;
    constexpr int NW = 4 * CG, NTW = NT * CG;
    constexpr int PV = ChainSmem<VT, NW>::PV;
    constexpr int KST = 4 / CG;                      // 16-byte q / k pieces per thread
    constexpr int VP = C * VT / 8;                   // 16-byte V pieces per chunk
    constexpr int KV = VP >= NTW ? VP / NTW : 1;     // ... per thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainSmem<VT, NW>& sm = *reinterpret_cast<ChainSmem<VT, NW>*>(smem_raw);

    const int nrun = OUT ? a.nseg : a.nseg - 1;
    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles * nrun, a.nseq);
    if (!mp.valid) return;
    const int seq = mp.seq, seg = mp.tile / a.ntiles, tile = mp.tile % a.ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int rb = w & 3, cg = w >> 2;
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.DV;
    const int cw = 16 * NVT * cg;              // the wave's first column in the tile
    const int c0 = tile * VT;
    const SeqSpan sp = seq_span(seq, a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nch = (sp.len + C - 1) / C;   // this sequence's chunks
    const int ch0 = seg * a.cps, ch1 = min(nch, ch0 + a.cps);
    const int nloc = max(ch1 - ch0, 0);     // a segment past the end is an identity step
    const int nsum = a.nseg - 1;
    const int rw = 16 * rb + jl;

    // entering state: key rows 16 (2 rb + ib) + 4 g + j, columns c0 + cw + colmap(ct, jl)
    f32x4_t S[2][NVT];
    const float* Sinit = nullptr;
    const float* zinit = nullptr;
    if (OUT) {
        // with several segments every entering state comes from the scan's slots (slot 0
        // holds the copy of S0, z0), so no workgroup here reads S0 while the last
        // segment writes S_final over it
        Sinit = nsum == 0 ? (a.S0 ? a.S0 + size_t(seq) * DK * DV : nullptr)
                          : a.dS + (size_t(seq) * a.nseg + seg) * DK * DV;
        zinit = nsum == 0 ? (a.z0 ? a.z0 + size_t(seq) * DK : nullptr)
                          : a.dz + (size_t(seq) * a.nseg + seg) * DK;
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * rb + ib) + 4 * g + j, c = c0 + cw + colmap<NVT>(ct, jl);
                S[ib][ct][j] = Sinit ? Sinit[size_t(i) * DV + c] : 0.f;
            }
    if (tid < DK) sm.z[0][tid] = zinit ? zinit[tid] : 0.f;
    if (OUT) {
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
            sm.st[0][((cg * 4 + rb) * NVT + ct) * 64 + lane] =
                __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));
    }

    // Per-sequence resources: rows past the end of the sequence read as zero and
    // output rows past it are dropped. Every load is unconditional.
    const uint32_t obytes = uint32_t(sp.len) * uint32_t(DV) * 2u;
    const rsrc_t rq = make_rsrc(a.q + tok0 * DK, uint32_t(sp.len) * DK * 2u);
    const rsrc_t rk = make_rsrc(a.k + tok0 * DK, uint32_t(sp.len) * DK * 2u);
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, obytes);
    const rsrc_t ro = make_rsrc(a.o + tok0 * DV, obytes);

    // A chunk's loads go out in two parts (K and V, then q) over the processing of the
    // chunk two before it, so that the memory unit's queue is not handed all of them at
    // once; each part stays in program order (the memory-counter waits before a chunk
    // is used count the loads issued after it).
    auto load_part = [&](ChainRegs<KST, KV>& R, int lc, int part) {
        const uint32_t t0 = uint32_t(ch0 + lc) * C;
        if (part == 0) {
#pragma unroll
            for (int x4 = 0; x4 < KST; ++x4) {
                const int x = tid + NTW * x4, r = x >> 4, col = (x & 15) * 8;
                R.kst[x4] = buf_ld16(rk, ((t0 + r) * DK + col) * 2u);
            }
#pragma unroll
            for (int x = 0; x < KV; ++x) {
                // V pieces, VT / 8 per row; threads past the pieces read past the range
                const int id = tid + NTW * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
                const uint32_t off = id < VP ? ((t0 + r) * uint32_t(DV) + c0 + col) * 2u : obytes;
                R.vst[x] = buf_ld16(rv, off);
            }
        } else if (OUT) {
#pragma unroll
            for (int x4 = 0; x4 < KST; ++x4) {
                const int x = tid + NTW * x4, r = x >> 4, col = (x & 15) * 8;
                R.qst[x4] = buf_ld16(rq, ((t0 + r) * DK + col) * 2u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_chunk = [&](ChainRegs<KST, KV>& R, int lc) {
        load_part(R, lc, 0);
        load_part(R, lc, 1);
    };
    // phi of one chunk's q and k (zero on padding rows), V, and per-wave column sums
    // of phi(k)
    auto stage = [&](const ChainRegs<KST, KV>& R, int buf, int lc) {
        const int n = min(C, sp.len - (ch0 + lc) * C);
        float zpart[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) zpart[q] = 0.f;
#pragma unroll
        for (int x4 = 0; x4 < KST; ++x4) {
            const int x = tid + NTW * x4, r = x >> 4, col = (x & 15) * 8;
            // rows past the sequence's end read as zeros, whose phi is 1: zero them
            float f[8];
            unpack8(R.kst[x4], f);
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = elu_plus_one_fast(f[q]);
            if (r >= n) {
#pragma unroll
                for (int q = 0; q < 8; ++q) f[q] = 0.f;
            }
            *reinterpret_cast<uint4*>(sm.kt[buf] + r * PQ + col) = pack8(f);
#pragma unroll
            for (int q = 0; q < 8; ++q) zpart[q] += f[q];
            if (OUT) {
                unpack8(R.qst[x4], f);
#pragma unroll
                for (int q = 0; q < 8; ++q) f[q] = elu_plus_one_fast(f[q]);
                if (r >= n) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) f[q] = 0.f;
                }
                *reinterpret_cast<uint4*>(sm.qt[buf] + r * PQ + col) = pack8(f);
            }
        }
        // the four 16-lane groups of a wave hold the same columns: fold them first
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            zpart[q] += __shfl_xor(zpart[q], 16, 64);
            zpart[q] += __shfl_xor(zpart[q], 32, 64);
        }
        if (g == 0) {
            const int col = jl * 8;
            *reinterpret_cast<float4*>(&sm.zp[buf][w][col]) = make_float4(zpart[0], zpart[1], zpart[2], zpart[3]);
            *reinterpret_cast<float4*>(&sm.zp[buf][w][col + 4]) = make_float4(zpart[4], zpart[5], zpart[6], zpart[7]);
        }
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            const int id = tid + NTW * x, r = id / (VT / 8), vc = (id % (VT / 8)) * 8;
            if (id < VP) *reinterpret_cast<uint4*>(sm.v[buf] + r * PV + vc) = R.vst[x];
        }
    };

    // The two waves that share a SIMD (same row block, column groups 0 and 1) stage the
    // next chunk at opposite ends of the chunk, so that one's vector work overlaps the
    // other's products.
    const bool early = OUT && (cg & 1) != 0;
    auto process = [&](const ChainRegs<KST, KV>& Rn, ChainRegs<KST, KV>& Rl, int lc, int cur) {
        load_part(Rl, lc + 2, 0);
        if (early) stage(Rn, cur ^ 1, lc + 1);
        const uint16_t* kt = sm.kt[cur];
        const uint16_t* vv = sm.v[cur];
        // z entering the next chunk
        if (tid < DK) {
            float zs = sm.z[cur][tid];
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) zs += sm.zp[cur][ww][tid];
            sm.z[cur ^ 1][tid] = zs;
        }
        if (OUT) {
            const uint16_t* qt = sm.qt[cur];
            // every LDS operand first: phi(q) of rows 16 rb .. (keys in natural order for
            // the scores, in the S^T fragments' order for the state part), S^T, V for P V,
            // and this lane's 32 keys of phi(q) with z
            bf16x8_t qf[4], qs[4], sf[4][NVT], vpk[2][NVT];
            const uint16_t* qrow = qt + (16 * rb + jl) * PQ;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                qf[kk] = frag_kc(qt, PQ, 16 * rb, 32 * kk, lane);
                const uint2 lo = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 4 * g);
                const uint2 hi = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 16 + 4 * g);
                qs[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct)
                    sf[kk][ct] = __builtin_bit_cast(bf16x8_t, sm.st[cur][((cg * 4 + kk) * NVT + ct) * 64 + lane]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct) vpk[kk][ct] = frag_kr_cols_pk<NVT>(vv, PV, kk, cw, ct, lane);
            float qz = 0.f;
#pragma unroll
            for (int q8 = 0; q8 < 4; ++q8) {
                float f[8];
                unpack8(*reinterpret_cast<const uint4*>(qrow + 32 * g + 8 * q8), f);
                const float4 z0 = *reinterpret_cast<const float4*>(sm.z[cur] + 32 * g + 8 * q8);
                const float4 z1 = *reinterpret_cast<const float4*>(sm.z[cur] + 32 * g + 8 * q8 + 4);
                qz += f[0] * z0.x + f[1] * z0.y + f[2] * z0.z + f[3] * z0.w;
                qz += f[4] * z1.x + f[5] * z1.y + f[6] * z1.z + f[7] * z1.w;
            }
            // P^T tiles D[s][r] = phi(k_s) . phi(q_r) of this row block, s <= r (the tiles
            // past the diagonal vanish under the mask), and their row sums
            f32x4_t pt[4];
            float rs = 0.f;
            const int r = 16 * rb + jl;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                f32x4_t acc = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    acc = mfma16(frag_kc(kt, PQ, 16 * sb, 32 * kk, lane), qf[kk], acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[j] = 16 * sb + 4 * g + j <= r ? acc[j] : 0.f;
                    rs += acc[j];
                }
                pt[sb] = acc;
            }
            rs += __shfl_xor(rs, 16, 64);
            rs += __shfl_xor(rs, 32, 64);
            qz += __shfl_xor(qz, 16, 64);
            qz += __shfl_xor(qz, 32, 64);
            const float inv = 1.f / (qz + rs + a.eps);
            const bf16x8_t pb0 = pack_pk(pt[0], pt[1]), pb1 = pack_pk(pt[2], pt[3]);
            load_part(Rl, lc + 2, 1);
            // O^T = S^T phi(Q)^T + V^T P^T, divided by the row's denominator
            const int nk = rb < 2 ? 1 : 2;
            uint2 ow[NVT];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) o_ = mfma16(sf[kk][ct], qs[kk], o_);
                o_ = mfma16(vpk[0][ct], pb0, o_);
                if (nk > 1) o_ = mfma16(vpk[1][ct], pb1, o_);
                o_ = o_ * inv;
                ow[ct].x = pack_bf16x2(o_[0], o_[1]);
                ow[ct].y = pack_bf16x2(o_[2], o_[3]);
            }
            const uint32_t orow =
                ((uint32_t(ch0 + lc) * C + rw) * uint32_t(DV) + c0 + cw + 4 * NVT * g) * 2u;
            if constexpr (NVT == 4) {
                buf_st16_out(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
                buf_st16_out(ro, orow + 16u, make_uint4(ow[2].x, ow[2].y, ow[3].x, ow[3].y));
            } else if constexpr (NVT == 2) {
                buf_st16_out(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
            } else {
                buf_st8(ro, orow, ow[0]);
            }
        }
        // ---- S += phi(K)^T V (key rows 32 rb ..)
        bf16x8_t vf[2][NVT], kf[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) vf[kk][ct] = frag_kr_cols<NVT>(vv, PV, 32 * kk, cw, ct, lane);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) kf[ib][kk] = frag_kr(kt, PQ, 32 * kk, 16 * (2 * rb + ib), lane);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = mfma16(kf[ib][0], vf[0][ct], S[ib][ct]);
                S[ib][ct] = mfma16(kf[ib][1], vf[1][ct], s_);
            }
        if (OUT) {
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                sm.st[cur ^ 1][((cg * 4 + rb) * NVT + ct) * 64 + lane] =
                    __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));
        } else {
            load_part(Rl, lc + 2, 1);
        }
        if (!early) stage(Rn, cur ^ 1, lc + 1);
        lds_barrier();
    };

    ChainRegs<KST, KV> RA, RB, RC;
    load_chunk(RA, 0);
    load_chunk(RB, 1);
    stage(RA, 0, 0);
    lds_barrier();
    for (int lc = 0; lc < nloc; lc += 3) {
        process(RB, RC, lc, lc & 1);
        if (lc + 1 >= nloc) break;
        process(RC, RA, lc + 1, (lc + 1) & 1);
        if (lc + 2 >= nloc) break;
        process(RA, RB, lc + 2, lc & 1);
    }

    if (OUT) {
        if (seg == a.nseg - 1) {
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 16 * (2 * rb + ib) + 4 * g + j;
                        const int c = c0 + cw + colmap<NVT>(ct, jl);
                        a.S[size_t(seq) * DK * DV + size_t(i) * DV + c] = S[ib][ct][j];
                    }
            if (tile == 0 && tid < DK) a.z[size_t(seq) * DK + tid] = sm.z[nloc & 1][tid];
        }
    } else {
        float* dS = a.dS + (size_t(seq) * a.nseg + seg + 1) * DK * DV;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 16 * (2 * rb + ib) + 4 * g + j;
                    const int c = c0 + cw + colmap<NVT>(ct, jl);
                    dS[size_t(i) * DV + c] = S[ib][ct][j];
                }
        if (tile == 0 && tid < DK) a.dz[(size_t(seq) * a.nseg + seg + 1) * DK + tid] = sm.z[nloc & 1][tid];
    }
}

// S_in[j + 1] = S_in[j] + dS_j and z_in[j + 1] = z_in[j] + dz_j, in place over the
// summaries in slot j + 1; slot 0 receives S_in[0] = S0 and z_in[0] = z0 (or zeros).
// One thread per 4 consecutive elements of S (the z row rides along with the threads
// of column group 0).
__global__ __launch_bounds__(256) void kath_scan_kernel(KathArgs a) {
    const int per_seq = DK * (a.DV / 4);
    const XcdMap mp = xcd_map(blockIdx.x, (per_seq + 255) / 256, a.nseq);
    if (!mp.valid) return;
    const int e = mp.tile * 256 + int(threadIdx.x);
    if (e >= per_seq) return;
    const size_t seq = size_t(mp.seq);
    const int i = e / (a.DV / 4), c = (e % (a.DV / 4)) * 4;
    const size_t so = size_t(i) * a.DV + c;
    const int nsum = a.nseg - 1;
    const size_t slot = size_t(DK) * a.DV;
    float* Sb = a.dS + seq * a.nseg * slot + so;
    float* zb = a.dz + seq * a.nseg * DK + i;
    float4 s = a.S0 ? *reinterpret_cast<const float4*>(a.S0 + seq * DK * a.DV + so)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    const bool zrow = c == 0;
    float z = zrow && a.z0 ? a.z0[seq * DK + i] : 0.f;
    *reinterpret_cast<float4*>(Sb) = s;
    if (zrow) zb[0] = z;
    constexpr int kBatch = 16;
    for (int j0 = 0; j0 < nsum; j0 += kBatch) {
        float4 ds[kBatch];
        float dz[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = min(j0 + u, nsum - 1);
            ds[u] = *reinterpret_cast<const float4*>(Sb + (j + 1) * slot);
            dz[u] = zrow ? zb[(j + 1) * DK] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (j0 + u < nsum) {
                s.x += ds[u].x; s.y += ds[u].y; s.z += ds[u].z; s.w += ds[u].w;
                *reinterpret_cast<float4*>(Sb + (j0 + u + 1) * slot) = s;
                if (zrow) {
                    z += dz[u];
                    zb[(j0 + u + 1) * DK] = z;
                }
            }
        }
    }
}

struct WsLayout {
    size_t dS, dz, total;
};
WsLayout ws_layout(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t nslot = size_t(p.segments > 1 ? p.segments : 0);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L{};
    L.dS = 0;
    size_t off = al(nseq * nslot * DK * size_t(p.dv) * 4);
    L.dz = off;
    off += al(nseq * nslot * DK * 4);
    L.total = nslot ? off : 0;
    return L;
}

// Value tile: NVT 16-column tiles per wave times CG column groups. dv >= 64 takes
// 64-column tiles on 8 waves (two column groups of 32): twice the waves of a 4-wave
// tile for the same staged phi(q), phi(k), V and P.
struct TileCfg {
    int nvt, cg;
};
TileCfg pick_tile(int dv) {
    if (dv >= 64) return {2, 2};
    return {dv / 16, 1};
}

template <int NVT, int CG>
hipError_t launch_cfg(const Problem& p) {
    constexpr int VT = 16 * NVT * CG;
    const WsLayout L = ws_layout(p);
    KathArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.S0 = p.S0;
    a.z0 = p.z0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    a.z = p.z;
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    a.dS = ws ? reinterpret_cast<float*>(ws + L.dS) : nullptr;
    a.dz = ws ? reinterpret_cast<float*>(ws + L.dz) : nullptr;
    a.eps = p.eps;
    a.N = p.N;
    a.cu = p.cu;
    a.H = p.H;
    a.L = p.L;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    a.nchunks = (p.L + C - 1) / C;
    a.nseg = p.segments;
    a.cps = (a.nchunks + a.nseg - 1) / a.nseg;
    a.DV = p.dv;
    a.ntiles = p.dv / VT;
    using Sm = ChainSmem<VT, 4 * CG>;
    const size_t smem = sizeof(Sm);
    const size_t smem_sum = offsetof(Sm, qt);
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kath_chain_kernel<false, NVT, CG>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem_sum));
        if (e != hipSuccess) return e;
        kath_chain_kernel<false, NVT, CG><<<dim3(xcd_grid(a.ntiles * (a.nseg - 1), a.nseq)),
                                            dim3(NT * CG), smem_sum, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int blocks = (DK * (p.dv / 4) + 255) / 256;
        kath_scan_kernel<<<dim3(xcd_grid(blocks, a.nseq)), dim3(256), 0, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kath_chain_kernel<true, NVT, CG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    kath_chain_kernel<true, NVT, CG><<<dim3(xcd_grid(a.ntiles * a.nseg, a.nseq)), dim3(NT * CG),
                                       smem, p.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool kath_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

size_t kath_mfma_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

int kath_mfma_auto_segments(const Problem& p) {
    // one forward workgroup per CU (its LDS takes most of a CU) over (sequence, segment,
    // value tile), at least four chunks per segment
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const TileCfg t = pick_tile(p.dv);
    const size_t ntiles = size_t(p.dv / (16 * t.nvt * t.cg));
    const size_t nchunks = size_t((p.L + C - 1) / C);
    const size_t units = nseq * ntiles;
    size_t want = (256 + units - 1) / units;
    // a packed batch: cut the longest sequence into pieces about the mean length, so that
    // it does not outlast the others (B sequences share the N tokens of each head)
    if (p.packed && p.N > 0) {
        const size_t even = (size_t(p.L) * size_t(p.B) + size_t(p.N) - 1) / size_t(p.N);
        if (even > want) want = even;
    }
    const size_t cap = nchunks / 4;
    if (want > cap) want = cap;
    return want < 1 ? 1 : int(want);
}

hipError_t launch_prefill_kath_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24)) return hipErrorInvalidValue;
    if (p.segments > 1 && !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's q / k / v / o rows
    if (size_t(p.L) * DK * 2 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    const TileCfg t = pick_tile(p.dv);
    if (t.cg == 2) return launch_cfg<2, 2>(p);
    return t.nvt == 1 ? launch_cfg<1, 1>(p) : launch_cfg<2, 1>(p);
}

}  // namespace la
