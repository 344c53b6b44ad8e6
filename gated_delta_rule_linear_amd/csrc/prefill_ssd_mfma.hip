// Chunked prefill for Mamba-2's SSD on bf16 MFMA in one pass over the inputs (d_k = 128,
// chunk C = 64): S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, one decay a_t per token
// and head ("Linear / RNN 路线", sections 3.6 and 4.1; "状态空间与线性注意力", section State
// Space Duality: the semiseparable matrix C_j^T (A_j .. A_{i+1}) B_i).
//
// Per chunk, with c_r = sum_{s<=r} log2 a_s (chunk-local) and the state S entering it:
//   o_r = 2^{c_r} q_r^T S + sum_{s<=r} 2^{c_r - c_s} (q_r . k_s) v_s
//   S  <- 2^{c_last} S + sum_s k_s (2^{c_last - c_s} v_s)^T
// an exact rewrite of the token recurrence. With one decay per row every factor is a
// scalar at most 1, so nothing needs the bounded per-block references of GLA's gates:
// each chunk's raw K is staged in LDS as it is, the score tile P = (Q K^T) o D comes off
// the matrix cores from it and from q's fragments, and the row factors 2^{c_last - c_s}
// go onto V when it is staged (a second, scaled copy), so the state update is K^T V^
// with K as given. Nothing is written per chunk to global memory: the step reads q, k,
// v and the decays, writes o and the final state, plus the segment summaries below.
//
// Like the GLA chain, a sequence is cut into segments that run in parallel (the
// parallel-scan idea of "Linear / RNN 路线"): a summary kernel walks every segment but
// the last from a zero state and writes its end state dS_j and decay product A_j; the
// forward kernel forms the state entering its segment from the summaries before it,
// S_in[j] = sum_{m < j} (prod_{m < l < j} A_l) dS_m + (prod_{l < j} A_l) S0, then walks
// its chunks. Decays are clamped at a >= exp(-10) like GLA's gates.
//
// One workgroup of four waves per (sequence, segment, value tile of VT = 16 NVT
// columns): wave w carries key rows 32 w .. 32 w + 31 of the state tile (two 16-row
// result tiles per column tile) and forms the outputs of token rows 16 w .. 16 w + 15.
// A chunk's loads go out two chunks ahead into registers and are staged into LDS
// (double-buffered) at the end of the chunk before, one barrier per chunk.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;   // 64
constexpr int NT = 256;
constexpr int PQ = DK + 16;     // pitch of [*][128] bf16 tiles (conflict-free 16-byte reads)
constexpr float kDecayMin = 4.539993e-05f;   // exp(-10)

struct SsdArgs {
    const uint16_t *q, *k, *v;
    const void* g;       // decay a per token and head
    const float* S0;
    uint16_t* o;
    float* S;
    float* dS;           // [nseq][nseg][tile][DK x VT]: slot 0 S0, slot m + 1 the summary dS_m
    float* A;            // [nseq][nseg - 1]: segment decay products
    int N, nseq, nseg, cps, ntiles, DV;
    const int32_t* cu;   // packed variable-length batch, or null
    int H, L;
};

template <int VT>
struct __align__(16) SsdSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t k[2][C * PQ];    // K [s][i] as given
    __align__(16) uint16_t v[2][C * PV];    // V [s][c] as given
    __align__(16) uint16_t vh[2][C * PV];   // 2^{c_last - c_s} V [s][c]
    __align__(16) uint16_t st[2][VT * PQ];  // S^T [c][i], bf16 (forward)
    __align__(16) float c[2][C];            // cumulative log2 decay
};

// One chunk's loads: this thread's four 16-byte pieces of K, its V pieces, the wave's q
// fragments (forward: row 16 w + j, keys 32 kk + 8 g ..) and the decay of token `lane`.
template <int KV>
struct SsdRegs {
    uint4 k[4], qf[4], v[KV];
    uint32_t a;
};

template <bool OUT, int NVT, bool GB>
__global__ __launch_bounds__(NT) void ssd_chain_kernel(SsdArgs a) {
    constexpr int VT = 16 * NVT;
    constexpr int PV = SsdSmem<VT>::PV;
    constexpr int KV = VT >= 32 ? VT / 32 : 1;   // 16-byte V pieces per thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SsdSmem<VT>& sm = *reinterpret_cast<SsdSmem<VT>*>(smem_raw);

    const int nrun = OUT ? a.nseg : a.nseg - 1;
    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles * nrun, a.nseq);
    if (!mp.valid) return;
    const int seq = mp.seq, seg = mp.tile / a.ntiles, tile = mp.tile % a.ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.DV;
    const int c0 = tile * VT;
    const SeqSpan sp = seq_span(seq, a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nch = (sp.len + C - 1) / C;
    const int ch0 = seg * a.cps, ch1 = min(nch, ch0 + a.cps);
    const int nloc = max(ch1 - ch0, 0);     // a segment past the end is an identity step
    const int rw = 16 * w + jl;             // this lane's output row

    // state tile: key rows 16 (2 w + ib) + 4 g + j, columns c0 + colmap(ct, jl)
    f32x4_t S[2][NVT];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) S[ib][ct] = zero4();
    float4* const slots = reinterpret_cast<float4*>(a.dS) +
                          (size_t(seq) * a.nseg * a.ntiles + tile) * (DK * VT / 4);
    const size_t slot_stride = size_t(a.ntiles) * (DK * VT / 4);
    auto S0_elem = [&](int ib, int ct, int j) {
        const int i = 16 * (2 * w + ib) + 4 * g + j, c = c0 + colmap<NVT>(ct, jl);
        return a.S0[size_t(seq) * DK * DV + size_t(i) * DV + c];
    };
    float aprod = 1.f;   // product of the chunk decays (summary)

    // Every load is unconditional: the resources cover the sequence, so a prefetch past
    // its end reads zeros (and is never processed past the segment's chunks).
    const uint32_t len = uint32_t(sp.len);
    const rsrc_t rk = make_rsrc(a.k + tok0 * DK, len * DK * 2u);
    const rsrc_t rq = make_rsrc(a.q + tok0 * DK, len * DK * 2u);
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, len * uint32_t(DV) * 2u);
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t rg = make_rsrc(static_cast<const char*>(a.g) + tok0 * GS, len * GS);
    const uint32_t obytes = len * uint32_t(DV) * 2u;
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

    auto load = [&](SsdRegs<KV>& R, int lc) {
        const uint32_t t0 = uint32_t(ch0 + lc) * C;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int id = tid + NT * x, r = id >> 4, col = (id & 15) * 8;
            R.k[x] = buf_ld16(rk, ((t0 + r) * DK + col) * 2u);
        }
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            // 64 rows x VT columns in 16-byte pieces, VT / 8 per row; with VT = 16 the
            // upper half of the threads reads past the range (zeros, unused)
            const int id = tid + NT * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
            const uint32_t off = VT >= 32 || id < C * VT / 8 ? ((t0 + r) * uint32_t(DV) + c0 + col) * 2u : obytes;
            R.v[x] = buf_ld16(rv, off);
        }
        if (OUT) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                R.qf[kk] = buf_ld16(rq, ((t0 + uint32_t(rw)) * DK + uint32_t(32 * kk + 8 * g)) * 2u);
        }
        R.a = buf_ld_gate<GB>(rg, t0 + uint32_t(lane));
        __builtin_amdgcn_sched_barrier(0);
    };
    // staging of chunk lc into buffer buf: K as given, the decays' running sum, V and the
    // scaled V^ = 2^{c_last - c_s} V
    auto stage = [&](const SsdRegs<KV>& R, int lc, int buf) {
        const int t0 = (ch0 + lc) * C;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int id = tid + NT * x, r = id >> 4, col = (id & 15) * 8;
            *reinterpret_cast<uint4*>(sm.k[buf] + r * PQ + col) = R.k[x];
        }
        // every wave forms the chunk's running decay sum (lane = token; padding rows
        // are identity steps)
        const float av = t0 + lane < sp.len ? fmaxf(gate_val<GB>(R.a), kDecayMin) : 1.f;
        const float cs = wave_inclusive_scan(__builtin_amdgcn_logf(av));
        const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
        if (w == 0) sm.c[buf][lane] = cs;
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            const int id = tid + NT * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
            if (VT >= 32 || id < C * VT / 8) {
                *reinterpret_cast<uint4*>(sm.v[buf] + r * PV + col) = R.v[x];
                const float f = __builtin_amdgcn_exp2f(clast - __shfl(cs, r, 64));
                const uint4 u = R.v[x];
                const uint32_t in[4] = {u.x, u.y, u.z, u.w};
                uint32_t outw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    outw[e] = pack_bf16x2(__uint_as_float(in[e] << 16) * f,
                                          __uint_as_float(in[e] & 0xffff0000u) * f);
                *reinterpret_cast<uint4*>(sm.vh[buf] + r * PV + col) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
            }
        }
    };

    auto process = [&](const SsdRegs<KV>& R, const SsdRegs<KV>& Rn, SsdRegs<KV>& Rl, int lc, int cur) {
        load(Rl, lc + 2);
        const uint16_t* kc = sm.k[cur];
        const float* cc = sm.c[cur];
        // the chunk's decay sums and the state update's operands, read before any LDS write
        // of this chunk: the compiler keeps LDS reads behind LDS writes it cannot tell
        // apart, so read later each would wait a round trip of its own
        float4 c4[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) c4[sb] = *reinterpret_cast<const float4*>(cc + 16 * sb + 4 * g);
        const float cr = cc[rw], clast = cc[C - 1];
        bf16x8_t vf[2][NVT], ktf[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) vf[kk][ct] = frag_kr_cols<NVT>(sm.vh[cur], PV, 32 * kk, 0, ct, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i0 = 16 * (2 * w + ib);
            ktf[ib][0] = frag_kr(kc, PQ, 0, i0, lane);
            ktf[ib][1] = frag_kr(kc, PQ, 32, i0, lane);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep these reads issued here
        if (OUT) {
            // score tiles P^T[s][r] for this wave's rows r = 16 w + j (s <= r): A = K rows
            // s, B = q's fragments, then the decay 2^{c_r - c_s} and the causal mask. Every
            // wave forms all four tiles (the masked ones come out zero): the wave with the
            // most rows sets the chunk's length either way, and without a branch on the wave
            // index the compiler schedules the whole chunk as one block.
            f32x4_t pt[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    pt[sb] = mfma16(frag_kc(kc, PQ, 16 * sb, 32 * kk, lane),
                                    __builtin_bit_cast(bf16x8_t, R.qf[kk]), pt[sb]);
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const float csv[4] = {c4[sb].x, c4[sb].y, c4[sb].z, c4[sb].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * sb + 4 * g + e;
                    pt[sb][e] = s <= rw ? __builtin_amdgcn_exp2f(cr - csv[e]) * pt[sb][e] : 0.f;
                }
            }
            const bf16x8_t pf0 = pack_pk(pt[0], pt[1]), pf1 = pack_pk(pt[2], pt[3]);
            const float er = __builtin_amdgcn_exp2f(cr);   // the state part of row rw
            const uint16_t* vv = sm.v[cur];
            // O^T = 2^{c_r} S^T q^T + V^T P^T for rows 16 w ..; 4 NVT contiguous columns
            // per lane
            bf16x8_t sfr[NVT][DK / 32], pv[2][NVT];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) sfr[ct][kk] = frag_st<NVT>(sm.st[cur], PQ, 0, ct, 32 * kk, lane);
                pv[0][ct] = frag_kr_cols_pk<NVT>(vv, PV, 0, 0, ct, lane);
                pv[1][ct] = frag_kr_cols_pk<NVT>(vv, PV, 1, 0, ct, lane);
            }
            uint2 ow[NVT];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    o_ = mfma16(sfr[ct][kk], __builtin_bit_cast(bf16x8_t, R.qf[kk]), o_);
                o_ *= er;
                o_ = mfma16(pv[0][ct], pf0, o_);
                o_ = mfma16(pv[1][ct], pf1, o_);   // pf1 is zero for w < 2
                ow[ct].x = pack_bf16x2(o_[0], o_[1]);
                ow[ct].y = pack_bf16x2(o_[2], o_[3]);
            }
            const uint32_t orow = ((uint32_t(ch0 + lc) * C + rw) * uint32_t(DV) + c0 + 4 * NVT * g) * 2u;
            if constexpr (NVT == 4) {
                buf_st16_out(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
                buf_st16_out(ro, orow + 16u, make_uint4(ow[2].x, ow[2].y, ow[3].x, ow[3].y));
            } else if constexpr (NVT == 2) {
                buf_st16_out(ro, orow, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
            } else {
                buf_st8(ro, orow, ow[0]);
            }
        }
        // S = 2^{c_last} S + K^T V^ (key rows 32 w ..)
        const float al = __builtin_amdgcn_exp2f(clast);
        if (!OUT) aprod *= al;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const int i0 = 16 * (2 * w + ib);
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * al;
                s_ = mfma16(ktf[ib][0], vf[0][ct], s_);
                s_ = mfma16(ktf[ib][1], vf[1][ct], s_);
                S[ib][ct] = s_;
                if (OUT) store_st<NVT>(sm.st[cur ^ 1], PQ, i0, 0, ct, s_, lane);
            }
        }
        stage(Rn, lc + 1, cur ^ 1);
        lds_barrier();
    };

    // three register sets rotate: each chunk's loads go out two chunks before it is
    // processed (a prefetch past the segment is never processed)
    SsdRegs<KV> RA, RB, RC;
    load(RA, 0);
    load(RB, 1);
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
            // state entering segment seg, from the summaries of the segments before it,
            // newest first, four summaries per batch of loads
            float dcur = 1.f;
            const float* Abase = a.A + size_t(seq) * (a.nseg - 1);
            for (int m = seg - 1; m >= 0; m -= 4) {
                float4 ds[4][2][NVT];
                float am[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int mm = max(m - u, 0);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                        for (int ct = 0; ct < NVT; ++ct)
                            ds[u][ib][ct] = slots[(mm + 1) * slot_stride + (ib * NVT + ct) * NT + tid];
                    am[u] = Abase[mm];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (m - u < 0) break;
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                        for (int ct = 0; ct < NVT; ++ct) {
                            S[ib][ct][0] += dcur * ds[u][ib][ct].x;
                            S[ib][ct][1] += dcur * ds[u][ib][ct].y;
                            S[ib][ct][2] += dcur * ds[u][ib][ct].z;
                            S[ib][ct][3] += dcur * ds[u][ib][ct].w;
                        }
                    dcur *= am[u];
                }
            }
            if (a.S0) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int ct = 0; ct < NVT; ++ct) {
                        const float4 x = slots[(ib * NVT + ct) * NT + tid];
                        S[ib][ct][0] += dcur * x.x;
                        S[ib][ct][1] += dcur * x.y;
                        S[ib][ct][2] += dcur * x.z;
                        S[ib][ct][3] += dcur * x.w;
                    }
            }
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                store_st<NVT>(sm.st[0], PQ, 16 * (2 * w + ib), 0, ct, S[ib][ct], lane);
    }
    stage(RA, 0, 0);
    lds_barrier();
    for (int lc = 0; lc < nloc; lc += 3) {
        process(RA, RB, RC, lc, lc & 1);
        if (lc + 1 >= nloc) break;
        process(RB, RC, RA, lc + 1, (lc + 1) & 1);
        if (lc + 2 >= nloc) break;
        process(RC, RA, RB, lc + 2, lc & 1);
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
        if (tile == 0 && tid == 0) a.A[size_t(seq) * (a.nseg - 1) + seg] = aprod;
    }
}

struct WsLayout {
    size_t dS, A, total;
};
// value columns per workgroup (as for GLA's chain: 64 at d_v = 64, 32 at d_v = 128)
int pick_nvt(int dv) { return dv == 128 ? 2 : dv >= 64 ? 4 : dv / 16; }
WsLayout ws_layout(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t nsum = size_t(p.segments > 1 ? p.segments - 1 : 0);
    const size_t nslot = p.segments > 1 ? size_t(p.segments) : 0;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout L{};
    L.dS = 0;
    L.A = al(nseq * nslot * DK * size_t(p.dv) * 4);
    L.total = L.A + al(nseq * nsum * 4);
    return L;
}

template <bool GB, int NVT>
hipError_t launch_nvt(const Problem& p) {
    constexpr int VT = 16 * NVT;
    const WsLayout L = ws_layout(p);
    SsdArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.g = p.g;
    a.S0 = p.S0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    a.dS = reinterpret_cast<float*>(ws + L.dS);
    a.A = reinterpret_cast<float*>(ws + L.A);
    a.N = p.N;
    a.cu = p.cu;
    a.H = p.H;
    a.L = p.L;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    const int nchunks = (p.L + C - 1) / C;
    a.nseg = p.segments;
    a.cps = (nchunks + a.nseg - 1) / a.nseg;
    a.DV = p.dv;
    a.ntiles = p.dv / VT;
    const size_t smem = sizeof(SsdSmem<VT>);
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_chain_kernel<false, NVT, GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        ssd_chain_kernel<false, NVT, GB>
            <<<dim3(xcd_grid(a.ntiles * (a.nseg - 1), a.nseq)), dim3(NT), smem, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ssd_chain_kernel<true, NVT, GB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    ssd_chain_kernel<true, NVT, GB>
        <<<dim3(xcd_grid(a.ntiles * a.nseg, a.nseq)), dim3(NT), smem, p.stream>>>(a);
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

size_t ssd_mfma_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

hipError_t launch_prefill_ssd_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24)) return hipErrorInvalidValue;
    if (p.segments > 1 && !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's q / k / v / o rows
    if (size_t(p.L) * size_t(DK) * 4 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    return p.gate_bf16 ? launch_gb<true>(p) : launch_gb<false>(p);
}

}  // namespace la
