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
// cut into four 16-row blocks; row block b uses the reference rho_b = B at its row 7:
// q~_r = q_r exp(B_r - rho_b), k~_s = k_s exp(rho_b - B_s) within the block, and an
// off-diagonal block pair takes the bounded factor exp(rho_rb - rho_sb) <= 1 on one
// side. Gates are clamped at g >= exp(-10) (a gate below that keeps less than 4.5e-5
// of the state, so the clamp changes no result beyond bf16 rounding), which keeps
// every factor within [exp(-80), exp(80)], inside fp32's normal range.
//
// Mamba-2's SSD (one decay per token and head) has kernels of its own
// (prefill_ssd_mfma.hip): with one decay per row every factor is bounded by itself, so it
// needs no prep pass.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 8;     // pitch of [*][128] bf16 tiles

// Workspace of one chunk, written by prep (bytes), each matrix in MFMA fragment order
// so that a wave reads its fragment as one contiguous kilobyte: q^ (piece (rb, kk, lane =
// 16 g + j) = row 16 rb + j, key columns 32 kk + 4 g .. + 3 then 32 kk + 16 + 4 g .. + 3:
// the key order of the S^T fragments the forward packs straight from its state
// registers), k^ transposed (piece (ib, kk,
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
    const int32_t* cu;   // packed variable-length batch, or null
    int H, L;            // heads; longest sequence (chunk counts are sized for it)
};

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per chunk. Wave w owns the 8-row group rows 8 w .. 8 w + 7
// (row block b = w / 2, its lower half for even w) and lane l the key columns 2 l,
// 2 l + 1. Every gate factor is a product of clamped gates (g >= exp(-10), the clamp
// above): the wave's own running products down its 8 rows (inclusive prefix pp,
// exclusive suffix ss) and the eight group totals T_h, shared through LDS. Row block
// b's reference rho_b = B at its row 7 is the last row of its lower group, so
//   lower group: exp(rho_b - B_r) = ss_r,  upper group: exp(B_r - rho_b) = pp_r,
// each in [exp(-80), 1], the other of the pair one reciprocal; q^ = q Pre pp and
// k^ = k ss Suf with Pre / Suf the products of the groups before / after (these two
// may underflow to zero, exactly where the true factor leaves fp32's range). An
// off-diagonal score block (rb, sb < rb) needs one of its operands rescaled by
// exp(rho_rb - rho_sb) <= 1, the product of groups 2 sb + 1 .. 2 rb: the rescaled
// copy of block sb's k~ for the pairs (0,1) (0,2) (1,2) (2,3), and of block rb's q~
// for (0,3) (1,3), so no wave writes more than two copies.
constexpr int NTP = 512;
constexpr float kGateMin = 4.539993e-05f;   // exp(-10)

__host__ __device__ constexpr bool pair_on_q(int sb, int rb) { return rb == 3 && sb <= 1; }

struct __align__(16) PrepSmem {
    __align__(16) uint16_t qo[C * PQ];      // q~, own row block's reference
    __align__(16) uint16_t ko[C * PQ];      // k~, own row block's reference
    __align__(16) uint16_t pc[6][16 * PQ];  // rescaled copy for each off-diagonal pair
    __align__(16) float T[8][DK];           // gate product of each 8-row group
    // q^ in the workspace's fragment order: every lane forms 4-byte pieces scattered over
    // the chunk's q^ block, so they are gathered here and written out in whole 16-byte
    // pieces (scattered 4-byte stores to memory cost far more than the same bytes whole)
    __align__(16) uint16_t qh[C * DK];
};
static_assert(2 * sizeof(PrepSmem) <= 163840, "two prep workgroups per compute unit");

template <bool GB>
__global__ __launch_bounds__(NTP) void gla_prep_kernel(GlaArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    // all chunks of a sequence on one XCD, where its later kernels run too
    const XcdMap mp = xcd_map(blockIdx.x, a.nchunks, a.nseq);
    if (!mp.valid) return;
    const size_t seq = size_t(mp.seq);
    const int ch = mp.tile;
    const int t0 = ch * C;
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    if (t0 >= sp.len) return;   // past this sequence's end: nothing reads this chunk
    const int rg = w, b = w >> 1;
    const bool upper = (w & 1) != 0;
    const int col = 2 * lane;

    // rows past the end of the sequence read as zero
    const uint32_t rows_left = uint32_t(sp.len - t0);
    const rsrc_t rq = make_rsrc(a.q + (tok0 + t0) * DK, rows_left * DK * 2u);
    const rsrc_t rk = make_rsrc(a.k + (tok0 + t0) * DK, rows_left * DK * 2u);
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t rg_ = make_rsrc(static_cast<const char*>(a.g) + (tok0 + t0) * DK * GS,
                                 rows_left * DK * GS);
    uint32_t qv[8], kv[8], gv[GB ? 8 : 16];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t e = uint32_t((8 * rg + r) * DK + col);
        qv[r] = buf_ld4(rq, e * 2u);
        kv[r] = buf_ld4(rk, e * 2u);
        if constexpr (GB) {
            gv[r] = buf_ld4(rg_, e * 2u);
        } else {
            const uint2 x = buf_ld8(rg_, e * 4u);
            gv[2 * r] = x.x;
            gv[2 * r + 1] = x.y;
        }
    }
    float pp[8][2], ss[8][2];
    {
        float gf[8][2];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float g0, g1;
            if constexpr (GB) {
                g0 = __uint_as_float(gv[r] << 16);
                g1 = __uint_as_float(gv[r] & 0xffff0000u);
            } else {
                g0 = __uint_as_float(gv[2 * r]);
                g1 = __uint_as_float(gv[2 * r + 1]);
            }
            const bool live = uint32_t(8 * rg + r) < rows_left;   // padding rows: identity steps
            gf[r][0] = live ? fmaxf(g0, kGateMin) : 1.f;
            gf[r][1] = live ? fmaxf(g1, kGateMin) : 1.f;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            pp[0][c] = gf[0][c];
#pragma unroll
            for (int r = 1; r < 8; ++r) pp[r][c] = pp[r - 1][c] * gf[r][c];
            ss[7][c] = 1.f;
#pragma unroll
            for (int r = 6; r >= 0; --r) ss[r][c] = ss[r + 1][c] * gf[r + 1][c];
        }
    }
    *reinterpret_cast<float2*>(&sm.T[rg][col]) = make_float2(pp[7][0], pp[7][1]);
    lds_barrier();

    float Tv[8][2];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        const float2 t = *reinterpret_cast<const float2*>(&sm.T[hh][col]);
        Tv[hh][0] = t.x;
        Tv[hh][1] = t.y;
    }
    // products of the groups before / after this one, and the pair factors: this wave
    // rescales k~ for the k-side pairs (b, rb > b) and q~ for the q-side pairs (sb, b)
    float pre[2], suf[2], fk[4][2], fq[4][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        pre[c] = 1.f;
        suf[c] = 1.f;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            if (hh < rg) pre[c] *= Tv[hh][c];
            if (hh > rg) suf[c] *= Tv[hh][c];
        }
#pragma unroll
        for (int o = 0; o < 4; ++o) {   // exp(rho_o - rho_b) (o > b), exp(rho_b - rho_o) (o < b)
            const int lo = o < b ? o : b, hi = o < b ? b : o;
            float f = 1.f;
#pragma unroll
            for (int hh = 1; hh < 7; ++hh)
                if (hh >= 2 * lo + 1 && hh <= 2 * hi) f *= Tv[hh][c];
            fk[o][c] = f;
            fq[o][c] = f;
        }
    }
    unsigned char* wsc = a.ws + (seq * a.nchunks + ch) * size_t(kWsChunk);
    if (rg == 0 && lane < DK / 2) {
        *reinterpret_cast<float2*>(wsc + kWsA + col * 4) = make_float2(Tv[0][0] * suf[0], Tv[0][1] * suf[1]);
    }
    float kh[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int rr = 8 * rg + r;
        const float q0 = __uint_as_float(qv[r] << 16), q1 = __uint_as_float(qv[r] & 0xffff0000u);
        const float k0 = __uint_as_float(kv[r] << 16), k1 = __uint_as_float(kv[r] & 0xffff0000u);
        float e0, e1, i0, i1;
        if (upper) {
            e0 = pp[r][0]; e1 = pp[r][1];
            i0 = __builtin_amdgcn_rcpf(e0); i1 = __builtin_amdgcn_rcpf(e1);
        } else {
            i0 = ss[r][0]; i1 = ss[r][1];
            e0 = __builtin_amdgcn_rcpf(i0); e1 = __builtin_amdgcn_rcpf(i1);
        }
        const float qt0 = q0 * e0, qt1 = q1 * e1, kt0 = k0 * i0, kt1 = k1 * i1;
        *reinterpret_cast<uint32_t*>(sm.qo + rr * PQ + col) = pack_bf16x2(qt0, qt1);
        *reinterpret_cast<uint32_t*>(sm.ko + rr * PQ + col) = pack_bf16x2(kt0, kt1);
        const int pr = rr & 15;
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            if (o > b && !pair_on_q(b, o))
                *reinterpret_cast<uint32_t*>(sm.pc[pair_index(b, o)] + pr * PQ + col) =
                    pack_bf16x2(kt0 * fk[o][0], kt1 * fk[o][1]);
            if (o < b && pair_on_q(o, b))
                *reinterpret_cast<uint32_t*>(sm.pc[pair_index(o, b)] + pr * PQ + col) =
                    pack_bf16x2(qt0 * fq[o][0], qt1 * fq[o][1]);
        }
        // q^ in fragment order: row rr, columns col, col + 1 are one slot pair of the
        // piece of lane group gg (key kc = 4 gg + e or 16 + 4 gg + e goes to slot e or 4 + e)
        const int kk = col >> 5, kc = col & 31, gg = (kc & 15) >> 2;
        const int slot = (kc & 3) + (kc >= 16 ? 4 : 0);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(sm.qh) +
                                     (((rr >> 4) * 4 + kk) * 64 + 16 * gg + pr) * 16 + slot * 2) =
            pack_bf16x2(q0 * (pre[0] * pp[r][0]), q1 * (pre[1] * pp[r][1]));
        kh[r][0] = k0 * (ss[r][0] * suf[0]);
        kh[r][1] = k1 * (ss[r][1] * suf[1]);
    }
    // k^ transposed: this thread's 8 tokens of key i are one fragment piece
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int i = col + c;
        float f[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) f[r] = kh[r][c];
        *reinterpret_cast<uint4*>(wsc + kWsK + (((i >> 4) * 2 + (rg >> 2)) * 64 + 16 * (rg & 3) + (i & 15)) * 16) =
            pack8(f);
    }
    lds_barrier();
    // q^ to the workspace in whole 16-byte pieces, coalesced
#pragma unroll
    for (int x = 0; x < C * DK * 2 / 16 / NTP; ++x) {
        const int pz = tid + NTP * x;
        *reinterpret_cast<uint4*>(wsc + kWsQ + pz * 16) =
            *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(sm.qh) + pz * 16);
    }
    // P: ten lower tiles, D'[s][r] = sum_i K~_si Q~_ri over key block sb and row block rb,
    // stored straight from the accumulators as half pieces; the two upper half pieces
    // the forward kernel reads, (0, 1) and (2, 3), are written as zeros. Waves 0 and 1
    // take two tiles, the others one.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int ti = w + 8 * tt;
        if (ti >= 10) continue;
        const int rb = ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3;
        const int sb = ti - (rb * (rb + 1)) / 2;
        const uint16_t* At = sm.ko;
        const uint16_t* Bt = sm.qo;
        int ar = 16 * sb, br = 16 * rb;
        if (sb < rb) {
            if (pair_on_q(sb, rb)) { Bt = sm.pc[pair_index(sb, rb)]; br = 0; }
            else { At = sm.pc[pair_index(sb, rb)]; ar = 0; }
        }
        f32x4_t acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            acc = mfma16(frag_kc(At, PQ, ar, 32 * kk, lane), frag_kc(Bt, PQ, br, 32 * kk, lane), acc);
        const int r = 16 * rb + jl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s_ = 16 * sb + 4 * g + j;
            acc[j] = s_ <= r ? acc[j] : 0.f;
        }
        unsigned char* piece = wsc + kWsP + ((rb * 2 + (sb >> 1)) * 64 + lane) * 16;
        *reinterpret_cast<uint2*>(piece + (sb & 1) * 8) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        if (sb == rb && (rb & 1) == 0) *reinterpret_cast<uint2*>(piece + 8) = make_uint2(0, 0);
    }
}

// ---------------------------------------------------------------------------
// summary (OUT = false) and forward (OUT = true): the chunk walk of one segment
// ---------------------------------------------------------------------------
// S^T is kept in fragment order: piece (kk, ct, lane = 16 g + L) holds column
// colmap(ct, L) of the tile and key rows 32 kk + 4 g .. + 3, 32 kk + 16 + 4 g .. + 3, which
// is what lane (g, L) of wave kk holds in its two state tiles, so each lane writes one
// contiguous 16-byte piece and each reader loads one.
template <int VT>
struct __align__(16) ChainSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint16_t v[2][C * PV];          // V [s][c]
    __align__(16) uint4 st[2][4 * (VT / 16) * 64];  // S^T fragments, bf16 (forward only)
    __align__(16) float a[2][DK];                 // chunk decay exp(B_last)
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
    const SeqSpan sp = seq_span(seq, a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nch = (sp.len + C - 1) / C;   // this sequence's chunks
    const int ch0 = seg * a.cps, ch1 = min(nch, ch0 + a.cps);
    const int nloc = max(ch1 - ch0, 0);     // a segment past the end is an identity step
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
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, uint32_t(sp.len) * uint32_t(DV) * 2u);
    const uint32_t obytes = uint32_t(sp.len) * uint32_t(DV) * 2u;
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

    // A chunk's loads (lc: chunk index within the segment) go out in two parts, at the
    // start and in the middle of the processing of the chunk three before it, so that the
    // memory unit's queue is not handed all of them at once; each part stays in program
    // order (the memory-counter waits before a chunk is used count the loads after it).
    auto load_part = [&](ChainRegs<KV>& R, int lc, int part) {
        const uint32_t cb = uint32_t(lc) * kWsChunk;
        const uint32_t t0 = uint32_t(ch0 + lc) * C;
        if (part == 0) {
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    R.kt[2 * ib + kk] =
                        buf_ld16(rw_, cb + kWsK + uint32_t(((2 * w + ib) * 2 + kk) * 64 + lane) * 16u);
            R.ast = buf_ld16(rw_, tid < DK / 4 ? cb + kWsA + uint32_t(tid) * 16u
                                               : uint32_t(nloc) * kWsChunk);
            __builtin_amdgcn_sched_barrier(0);
            return;
        }
#pragma unroll
        for (int x = 0; x < KV; ++x) {
            // V pieces: 64 rows x VT columns in 16-byte pieces, VT / 8 per row; with
            // VT = 16 the upper half of the threads reads past the range (zeros, unused)
            const int id = tid + NT * x, r = id / (VT / 8), col = (id % (VT / 8)) * 8;
            const uint32_t off = VT >= 32 || id < C * VT / 8
                                     ? ((t0 + r) * uint32_t(DV) + c0 + col) * 2u : obytes;
            R.vst[x] = buf_ld16(rv, off);
        }
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
    auto load_chunk = [&](ChainRegs<KV>& R, int lc) {
        load_part(R, lc, 0);
        load_part(R, lc, 1);
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

    auto process = [&](const ChainRegs<KV>& R, const ChainRegs<KV>& Rn, ChainRegs<KV>& Rl, int lc,
                       int cur) {
        load_part(Rl, lc + 3, 0);
        const uint16_t* vv = sm.v[cur];
        // Every LDS operand of the chunk is read first, so that the reads overlap one
        // another instead of each waiting in front of its own product.
        constexpr int NS = OUT ? 4 : 1;
        bf16x8_t sfr[NS][NVT], vpk[NS / 2 + 1][NVT], vf[2][NVT];
        f32x4_t av[2];
        if (OUT) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct)
                    sfr[kk][ct] = __builtin_bit_cast(bf16x8_t, sm.st[cur][(kk * NVT + ct) * 64 + lane]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ct = 0; ct < NVT; ++ct) vpk[kk][ct] = frag_kr_cols_pk<NVT>(vv, PV, kk, 0, ct, lane);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) vf[kk][ct] = frag_kr_cols<NVT>(vv, PV, 32 * kk, 0, ct, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const float4 a4 = *reinterpret_cast<const float4*>(sm.a[cur] + 16 * (2 * w + ib) + 4 * g);
            av[ib] = f32x4_t{a4.x, a4.y, a4.z, a4.w};
        }
        // S = diag(a) S + K^^T V (key rows 32 w ..)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            if (!OUT) {
#pragma unroll
                for (int j = 0; j < 4; ++j) aprod[ib][j] *= av[ib][j];
            }
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * av[ib];
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kt[2 * ib]), vf[0][ct], s_);
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kt[2 * ib + 1]), vf[1][ct], s_);
                S[ib][ct] = s_;
            }
        }
        if (OUT) {
            // O^T = S^T q^^T + V^T P^T for rows 16 w ..; 4 NVT contiguous columns per lane
            uint2 ow[NVT];
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t o_ = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    o_ = mfma16(sfr[kk][ct], __builtin_bit_cast(bf16x8_t, R.qf[kk]), o_);
                o_ = mfma16(vpk[0][ct], __builtin_bit_cast(bf16x8_t, R.pf[0]), o_);
                if (nk > 1) o_ = mfma16(vpk[1][ct], __builtin_bit_cast(bf16x8_t, R.pf[1]), o_);
                ow[ct].x = pack_bf16x2(o_[0], o_[1]);
                ow[ct].y = pack_bf16x2(o_[2], o_[3]);
            }
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                sm.st[cur ^ 1][(w * NVT + ct) * 64 + lane] =
                    __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));
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
        load_part(Rl, lc + 3, 1);
        stage(Rn, cur ^ 1);
        lds_barrier();
    };

    // four register sets rotate: each chunk's loads go out three chunks before it is
    // processed (a prefetch past the segment reads zeros and is never processed)
    ChainRegs<KV> RA, RB, RC, RD;
    load_chunk(RA, 0);
    load_chunk(RB, 1);
    load_chunk(RC, 2);
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
            // S_in = sum_m (prod_{l > m} A_l) dS_m + (prod_l A_l) S0, newest first, four
            // summaries per batch of loads
            float dcur[2][4];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int j = 0; j < 4; ++j) dcur[ib][j] = 1.f;
            const float* Abase = a.A + size_t(seq) * (a.nseg - 1) * DK + 16 * (2 * w) + 4 * g;
            for (int m = seg - 1; m >= 0; m -= 4) {
                float4 ds[4][2][NVT], am[4][2];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
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
                for (int u = 0; u < 4; ++u) {
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
        for (int ct = 0; ct < NVT; ++ct)
            sm.st[0][(w * NVT + ct) * 64 + lane] = __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));
    }
    stage(RA, 0);
    lds_barrier();
    for (int lc = 0; lc < nloc; lc += 4) {
        process(RA, RB, RD, lc, 0);
        if (lc + 1 >= nloc) break;
        process(RB, RC, RA, lc + 1, 1);
        if (lc + 2 >= nloc) break;
        process(RC, RD, RB, lc + 2, 0);
        if (lc + 3 >= nloc) break;
        process(RD, RA, RC, lc + 3, 1);
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
    const size_t nchunks = size_t((p.L + C - 1) / C);
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

// Value columns per workgroup: 64 for d_v = 64 (one tile per sequence), but 32 for
// d_v = 128: four smaller tiles per sequence put two workgroups on each CU, whose
// latencies overlap, which measured faster than two 64-column tiles at one per CU even
// though every tile re-reads the chunk's q^, k^T and P.
int pick_nvt(int dv) { return dv == 128 ? 2 : dv >= 64 ? 4 : dv / 16; }

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
    a.cu = p.cu;
    a.H = p.H;
    a.L = p.L;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    a.nchunks = (p.L + C - 1) / C;
    a.nseg = p.segments;
    a.cps = (a.nchunks + a.nseg - 1) / a.nseg;
    a.DV = p.dv;
    a.ntiles = p.dv / VT;
    hipError_t e;
    {
        const size_t blocks = size_t(xcd_grid(a.nchunks, (a.nseq + 7) & ~7));
        if (size_t(a.nseq + 7) * size_t(a.nchunks) > 0x7fffffffull) return hipErrorInvalidValue;
        const size_t smem = sizeof(PrepSmem);
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gla_prep_kernel<GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        gla_prep_kernel<GB><<<dim3(unsigned(blocks)), dim3(NTP), smem, p.stream>>>(a);
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
    const size_t nchunks = size_t((p.L + C - 1) / C);
    const size_t units = nseq * ntiles;
    size_t want = (256 + units - 1) / units;
    // a packed batch: cut the longest sequence into pieces about the mean length, so that
    // it does not outlast the others (B sequences share the N tokens of each head)
    if (p.packed && p.N > 0) {
        const size_t even = (size_t(p.L) * size_t(p.B) + size_t(p.N) - 1) / size_t(p.N);
        if (even > want) want = even;
    }
    const size_t cap = nchunks / 2;
    if (want > cap) want = cap;
    return want < 1 ? 1 : int(want);
}

hipError_t launch_prefill_gla_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24) || !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's v / o rows and its chunk workspace
    if (size_t(p.L) * size_t(DK) * 4 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    if (size_t((p.L + C - 1) / C) * kWsChunk >= (size_t(1) << 31)) return hipErrorInvalidValue;
    return p.gate_bf16 ? launch_gb<true>(p) : launch_gb<false>(p);
}

}  // namespace la
