// Chunked prefill for Kimi Delta Attention on bf16 MFMA (d_k = 128, chunk C = 64).
//
// Method ("状态空间与线性注意力", section KDA, rewritten per chunk). With the entering
// state S (key-major, fp32), local rows r, s = 0..C-1 and the per-channel cumulative
// retention G_r = prod_{m<=r} alpha_m (a d_k vector), unrolling Sbar = Diag(alpha) S,
// S' = Sbar + beta k (v - Sbar^T k)^T token by token gives, with K~ = G * K,
// Q~ = G * Q, K^ = (G_last / G) * K and the decay-weighted products
//   (K~ K-)_rs = sum_i k_ri k_si G_ri / G_si,  (Q~ K-)_rs likewise  (s <= r):
//   L = stril(diag(beta) K~ K-^T),  T = (I + L)^{-1}
//   U = T diag(beta) (V - K~ S),  O = Q~ S + tril(Q~ K-^T) U
//   S <- Diag(G_last) S + K^^T U.
// The ratios G_r / G_s come from products of the clamped retentions (alpha >= e^-10,
// the same bound as the GLA kernels; the bounded log-decay of the page, alpha >
// e^-5, never reaches it): per 16-row block b a reference row rho_b (row 7 of the
// block), k~_s = k_s G_rho / G_s and q~_r = q_r G_r / G_rho for the diagonal block,
// and the bounded factor G_rho_rb / G_rho_sb <= 1 on the key side of an off-diagonal
// block, so every factor stays within [e^-80, e^80].
//
// Two kernels:
//   prep     one workgroup of 8 waves per (sequence, chunk), fully parallel: Q~, K~ and
//            K^^T in MFMA fragment order, the masked score tile P, T and G_last, all
//            to the workspace. Waves 0..3 build L and invert it (diagonal 16 x 16
//            blocks by fp32 forward substitution, the rest by bf16 block products)
//            while waves 4..7 form P.
//   forward  one workgroup per (sequence, 32-column value tile): walks the chunks with
//            its fp32 state tile in MFMA accumulators. Every per-chunk operand comes
//            straight into registers in fragment layout, two chunks ahead; only X, U
//            and the bf16 copy of S^T go through LDS. Three barriers per chunk:
//            (S^T Q~^T, S^T K~^T) -> X | U = T X | O = Q~ S + P U and the state
//            update.
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NTP = 512;       // prep: 8 waves
constexpr int NTF = 256;       // forward: 4 waves
constexpr int PQ = DK + 8;     // pitch of [*][128] bf16 tiles
constexpr int PC = C + 8;      // pitch of [*][64] bf16 tiles (rows 16-byte aligned)
constexpr int PD = 16;         // pitch of the fp32 16 x 16 diagonal L blocks
constexpr int PY = 32 + 8;     // pitch of the bf16 32-row scratch tiles
constexpr float kGateMin = 4.539993e-05f;   // exp(-10)

// Workspace of one chunk (bytes), each matrix in MFMA fragment order (a 16-byte piece
// per lane, a wave's fragment one contiguous kilobyte):
//   Q~, K~: piece (rb, kk, lane = 16 g + j) = row 16 rb + j, keys 32 kk + 4 g .. + 3 then
//           32 kk + 16 + 4 g .. + 3 (the key order of the S^T fragments the forward
//           packs straight from its state registers);
//   K^^T:   piece (ib, kk, lane) = key 16 ib + j, tokens 32 kk + 8 g .. + 7;
//   P:      piece (rb, kk, lane) = row 16 rb + j, tokens 32 kk + 4 g .. + 3, then
//           32 kk + 16 + 4 g .. + 3 (the order the matrix cores return the tile);
//   T:      piece (rb, kk, lane) = row 16 rb + j, columns 32 kk + 8 g .. + 7;
//   a:      G_last, fp32 [128].
constexpr uint32_t kWsQ = 0, kWsK = 16384, kWsKh = 32768, kWsP = 49152, kWsT = 57344,
                   kWsA = 65536, kWsChunk = 66048;

__host__ __device__ constexpr int pair_index(int b, int bb) {   // (0,1)..(2,3) -> 0..5
    return b == 0 ? bb - 1 : b == 1 ? bb + 1 : 5;
}

struct KdaArgs {
    const uint16_t *q, *k, *v;
    const void *alpha, *beta;
    const float* S0;
    uint16_t* o;
    float* S;
    unsigned char* ws;
    int N, nseq, ntiles, nchunks;
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

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
// Wave w owns rows 8 w .. 8 w + 7 (row block b = w / 2, its lower half for even w)
// and lane l the key columns 2 l, 2 l + 1; the running products of its rows' clamped
// retentions (inclusive prefix pp, exclusive suffix ss) and the group totals give
// every factor: lower group G_rho / G_r = ss_r, upper group G_r / G_rho = pp_r (each in
// [e^-80, 1]), the other of the pair one reciprocal; G_r = Pre pp_r and G_last / G_r =
// ss_r Suf with Pre / Suf the products of the groups before / after.
// 80 KiB, so that two workgroups share a CU: the off-diagonal key fragments are
// rescaled as they are read (from the per-pair factor table fe) instead of being stored
// as copies, and the inverse's scratch reuses q~, which is dead by then.
struct __align__(16) PrepSmem {
    union {
        __align__(16) uint16_t qo[C * PQ];  // q~ (own row block's reference)
        struct {
            __align__(16) uint16_t ya[2][32 * PY];  // level-a scratch (rows 0..15 used)
            __align__(16) uint16_t yb[32 * PY];     // level-b scratch
        } y;
    } u;
    __align__(16) uint16_t ko[C * PQ];      // k- side: k_s G_rho / G_s
    __align__(16) uint16_t kr[C * PQ];      // k~ row side: k_r G_r / G_rho
    __align__(16) uint16_t t[C * PC];       // T [r][s]
    __align__(16) uint16_t lo[C * PC];      // off-diagonal blocks of L [r][s]
    __align__(16) float ld[4][16 * PD];     // diagonal blocks of L, fp32
    __align__(16) float T[8][DK];           // retention product of each 8-row group
    __align__(16) float fe[6][DK];          // G_rho_rb / G_rho_sb per key, pair (sb, rb)
};
static_assert(sizeof(PrepSmem) <= 80 * 1024, "two prep workgroups per CU");

template <bool GB>
__global__ __launch_bounds__(NTP) void kda_prep_kernel(KdaArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const XcdMap mp = xcd_map(blockIdx.x, a.nchunks, a.nseq);
    if (!mp.valid) return;
    const size_t seq = size_t(mp.seq);
    const int ch = mp.tile;
    const int t0 = ch * C;
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    if (t0 >= sp.len) return;   // past this sequence's end: the forward reads zeros instead
    const int rg = w, b = w >> 1;
    const bool upper = (w & 1) != 0;
    const int col = 2 * lane;

    // rows past the end of the sequence read as zero
    const uint32_t rows_left = uint32_t(sp.len - t0);
    const rsrc_t rq = make_rsrc(a.q + (tok0 + t0) * DK, rows_left * DK * 2u);
    const rsrc_t rk = make_rsrc(a.k + (tok0 + t0) * DK, rows_left * DK * 2u);
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t ra = make_rsrc(static_cast<const char*>(a.alpha) + (tok0 + t0) * DK * GS,
                                rows_left * DK * GS);
    const rsrc_t rb_ = make_rsrc(static_cast<const char*>(a.beta) + (tok0 + t0) * GS, rows_left * GS);
    uint32_t qv[8], kv[8], gv[GB ? 8 : 16];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t e = uint32_t((8 * rg + r) * DK + col);
        qv[r] = buf_ld4(rq, e * 2u);
        kv[r] = buf_ld4(rk, e * 2u);
        if constexpr (GB) {
            gv[r] = buf_ld4(ra, e * 2u);
        } else {
            const uint2 x = buf_ld8(ra, e * 4u);
            gv[2 * r] = x.x;
            gv[2 * r + 1] = x.y;
        }
    }
    // beta of rows 16 bb + jl, for the waves that form L (zero past the end)
    float bet[4] = {0.f, 0.f, 0.f, 0.f};
    if (w < 4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) bet[bb] = gate_val<GB>(buf_ld_gate<GB>(rb_, uint32_t(16 * bb + jl)));
    }
    if (w >= 4) {
        // zero the six upper blocks of T (the level-a scratch needs none: its rows 16..31
        // only reach lanes whose fragment is replaced by zeros)
        const int x = w - 4;
        const int ub[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};
        const int r = lane >> 2, cc = (lane & 3) * 4;
        for (int y = x; y < 6; y += 4)
            *reinterpret_cast<uint2*>(sm.t + (16 * ub[y][0] + r) * PC + 16 * ub[y][1] + cc) =
                make_uint2(0, 0);
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
    // products of the groups before / after this one
    float pre[2], suf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        pre[c] = 1.f;
        suf[c] = 1.f;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            if (hh < rg) pre[c] *= Tv[hh][c];
            if (hh > rg) suf[c] *= Tv[hh][c];
        }
    }
    if (rg == 1) {
        // pair factors G_rho_rb / G_rho_sb = product of groups 2 sb + 1 .. 2 rb
#pragma unroll
        for (int sb = 0; sb < 3; ++sb) {
            float run[2] = {1.f, 1.f};
#pragma unroll
            for (int rb = sb + 1; rb < 4; ++rb) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    if (2 * rb - 1 > 2 * sb) run[c] *= Tv[2 * rb - 1][c];
                    run[c] *= Tv[2 * rb][c];
                }
                *reinterpret_cast<float2*>(&sm.fe[pair_index(sb, rb)][col]) = make_float2(run[0], run[1]);
            }
        }
    }
    unsigned char* wsc = a.ws + (seq * a.nchunks + ch) * size_t(kWsChunk);
    if (rg == 0)
        *reinterpret_cast<float2*>(wsc + kWsA + col * 4) = make_float2(Tv[0][0] * suf[0], Tv[0][1] * suf[1]);
    float kh[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int rr = 8 * rg + r, pr = rr & 15;
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
        const float kt0 = k0 * i0, kt1 = k1 * i1;
        *reinterpret_cast<uint32_t*>(sm.u.qo + rr * PQ + col) = pack_bf16x2(q0 * e0, q1 * e1);
        *reinterpret_cast<uint32_t*>(sm.kr + rr * PQ + col) = pack_bf16x2(k0 * e0, k1 * e1);
        *reinterpret_cast<uint32_t*>(sm.ko + rr * PQ + col) = pack_bf16x2(kt0, kt1);
        // Q~ and K~ in fragment order: row rr, columns col, col + 1 are one slot pair of the
        // piece of lane group gg (key kc = 4 gg + e or 16 + 4 gg + e goes to slot e or 4 + e)
        const int kk = col >> 5, kc = col & 31, gg = (kc & 15) >> 2;
        const int slot = (kc & 3) + (kc >= 16 ? 4 : 0);
        const uint32_t piece = (((rr >> 4) * 4 + kk) * 64 + 16 * gg + pr) * 16 + slot * 2;
        const float G0 = pre[0] * pp[r][0], G1 = pre[1] * pp[r][1];
        *reinterpret_cast<uint32_t*>(wsc + kWsQ + piece) = pack_bf16x2(q0 * G0, q1 * G1);
        *reinterpret_cast<uint32_t*>(wsc + kWsK + piece) = pack_bf16x2(k0 * G0, k1 * G1);
        kh[r][0] = k0 * (ss[r][0] * suf[0]);
        kh[r][1] = k1 * (ss[r][1] * suf[1]);
    }
    // K^ transposed: this thread's 8 tokens of key i are one fragment piece
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int i = col + c;
        float f[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) f[r] = kh[r][c];
        *reinterpret_cast<uint4*>(wsc + kWsKh + (((i >> 4) * 2 + (rg >> 2)) * 64 + 16 * (rg & 3) + (i & 15)) * 16) =
            pack8(f);
    }
    lds_barrier();

    // key-side fragment of tile (rb, sb), keys 32 kk ..: the own-reference k- rows of
    // block sb, rescaled to row block rb's reference for sb < rb (a factor <= 1)
    auto key_frag = [&](int rb, int sb, int kk) -> bf16x8_t {
        const bf16x8_t f = frag_kc(sm.ko, PQ, 16 * sb, 32 * kk, lane);
        if (sb == rb) return f;
        const float* fp = sm.fe[pair_index(sb, rb)] + 32 * kk + 8 * g;
        const float4 f0 = *reinterpret_cast<const float4*>(fp);
        const float4 f1 = *reinterpret_cast<const float4*>(fp + 4);
        float x[8];
        unpack8(__builtin_bit_cast(uint4, f), x);
        x[0] *= f0.x; x[1] *= f0.y; x[2] *= f0.z; x[3] *= f0.w;
        x[4] *= f1.x; x[5] *= f1.y; x[6] *= f1.z; x[7] *= f1.w;
        return __builtin_bit_cast(bf16x8_t, pack8(x));
    };
    if (w == 0) {
        // diagonal blocks of L (fp32): D'[s][r] = beta_r sum_i k-_si k~_ri, s < r
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            f32x4_t d = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                d = mfma16(frag_kc(sm.ko, PQ, 16 * bb, 32 * kk, lane),
                           frag_kc(sm.kr, PQ, 16 * bb, 32 * kk, lane), d);
            const int r = 16 * bb + jl;
            const float br = bet[bb];
            float4 val;
            float* vv = reinterpret_cast<float*>(&val);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * bb + 4 * g + j;
                vv[j] = s < r ? br * d[j] : 0.f;
            }
            *reinterpret_cast<float4*>(sm.ld[bb] + jl * PD + 4 * g) = val;
        }
        wave_lds_sync();
        // forward substitution, lane = 16 bb + column jc: T_bb[:, jc]
        const int bb = g, jc = jl;
        const float* Lb = sm.ld[bb];
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
        for (int r = 0; r < 16; ++r) sm.t[(16 * bb + r) * PC + 16 * bb + jc] = f32_to_bf16(tc[r]);
    } else if (w < 4) {
        // waves 1..3: the six off-diagonal L blocks (bf16) -> lo[r][s]
        for (int task = w - 1; task < 6; task += 3) {
            const int rb = task < 1 ? 1 : task < 3 ? 2 : 3;
            const int sb = task - (rb * (rb - 1)) / 2;
            f32x4_t d = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                d = mfma16(key_frag(rb, sb, kk), frag_kc(sm.kr, PQ, 16 * rb, 32 * kk, lane), d);
            const float br = rb == 1 ? bet[1] : rb == 2 ? bet[2] : bet[3];
            store_dT(sm.lo, PC, 16 * sb, 16 * rb, d * br, lane);
        }
    } else {
        // waves 4..7: the ten lower score tiles, D'[s][r] = sum_i k-_si q~_ri (s <= r),
        // stored from the accumulators as half pieces; the two upper half pieces the
        // forward kernel reads, (0, 1) and (2, 3), are written as zeros
        for (int ti = w - 4; ti < 10; ti += 4) {
            const int rb = ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3;
            const int sb = ti - (rb * (rb + 1)) / 2;
            f32x4_t acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                acc = mfma16(key_frag(rb, sb, kk), frag_kc(sm.u.qo, PQ, 16 * rb, 32 * kk, lane), acc);
            const int r = 16 * rb + jl;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = 16 * sb + 4 * g + j <= r ? acc[j] : 0.f;
            unsigned char* piece = wsc + kWsP + ((rb * 2 + (sb >> 1)) * 64 + lane) * 16;
            *reinterpret_cast<uint2*>(piece + (sb & 1) * 8) =
                make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
            if (sb == rb && (rb & 1) == 0) *reinterpret_cast<uint2*>(piece + 8) = make_uint2(0, 0);
        }
    }
    lds_barrier();
    // level a: T_10 = -T_11 L_10 T_00 (wave 1), T_32 = -T_33 L_32 T_22 (wave 2)
    if (w == 1 || w == 2) {
        const int i = w == 1 ? 1 : 3, j = i - 1;
        uint16_t* y = sm.u.y.ya[w - 1];
        f32x4_t d = mfma16(k16(frag_kr(sm.t, PC, 16 * j, 16 * j, lane), lane),
                           k16(frag_kc(sm.lo, PC, 16 * i, 16 * j, lane), lane), zero4());
        store_dT(y, PY, 0, 0, d, lane);
        wave_lds_sync();
        d = mfma16(k16(frag_kr(y, PY, 0, 0, lane), lane),
                   k16(frag_kc(sm.t, PC, 16 * i, 16 * i, lane), lane), zero4());
        store_dT(sm.t, PC, 16 * j, 16 * i, -d, lane);
    }
    lds_barrier();
    // level b: Y = L[32:64, 0:32] A^{-1}, tile (rb, jb) per wave
    if (w < 4) {
        const int jb = w & 1, rb = w >> 1;
        const f32x4_t d = mfma16(frag_kr(sm.t, PC, 0, 16 * jb, lane),
                                 frag_kc(sm.lo, PC, 32 + 16 * rb, 0, lane), zero4());
        store_dT(sm.u.y.yb, PY, 16 * jb, 16 * rb, d, lane);
    }
    lds_barrier();
    // level c: T[32:64, 0:32] = -B^{-1} Y
    if (w < 4) {
        const int jb = w & 1, rb = w >> 1;
        const f32x4_t d = mfma16(frag_kr(sm.u.y.yb, PY, 0, 16 * jb, lane),
                                 frag_kc(sm.t, PC, 32 + 16 * rb, 32, lane), zero4());
        store_dT(sm.t, PC, 16 * jb, 32 + 16 * rb, -d, lane);
    }
    lds_barrier();
    // T in fragment order: one 16-byte piece per thread
    {
        const int rb = tid >> 7, kk = (tid >> 6) & 1, l = tid & 63;
        const int off = (16 * rb + (l & 15)) * PC + 32 * kk + 8 * (l >> 4);
        *reinterpret_cast<uint4*>(wsc + kWsT + tid * 16) = *reinterpret_cast<const uint4*>(sm.t + off);
    }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// The bf16 copy of the state is kept as S^T fragments: piece (kk, ct, lane = 16 g + L)
// holds column colmap(ct, L) and key rows 32 kk + 4 g .. + 3, 32 kk + 16 + 4 g .. + 3, which
// is what lane (g, L) of wave kk holds in its two state tiles, so each lane writes one
// contiguous 16-byte piece and each reader loads one.
template <int VT>
struct __align__(16) FwdSmem {
    static constexpr int PV = VT + 8;
    __align__(16) uint4 st[4 * (VT / 16) * 64];   // S^T fragments, bf16
    __align__(16) uint16_t x[C * PV];            // X [s][c]
    __align__(16) uint16_t u[C * PV];            // U [s][c]
};

// Per-chunk operands of one wave (row block rb = w): rows 16 rb + j of Q~, K~, T and P,
// key blocks 2 rb, 2 rb + 1 of K^^T, this thread's V piece, G_last of its state rows
// and beta of its row.
template <int NVT>
struct ChunkRegs {
    uint4 q[4], k[4], kh[4], t[2], p[2];
    uint2 v[NVT];
    float4 a[2];
    uint32_t b;
};

template <int NVT, bool GB>
__global__ __launch_bounds__(NTF) void kda_fwd_kernel(KdaArgs a) {
    constexpr int VT = 16 * NVT;
    constexpr int PV = FwdSmem<VT>::PV;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FwdSmem<VT>& sm = *reinterpret_cast<FwdSmem<VT>*>(smem_raw);

    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles, a.nseq);
    if (!mp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int rb = w, g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT;
    const int c0 = mp.tile * VT;
    const size_t seq = size_t(mp.seq);
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nchunks = (sp.len + C - 1) / C;   // this sequence's chunks
    const int rw = 16 * rb + jl;
    const int nk = rb < 2 ? 1 : 2;   // T and P vanish for s >= 16 (rb + 1)

    // state tiles: key blocks 2 rb + ib, column tiles ct (D layout)
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
    for (int ct = 0; ct < NVT; ++ct)
        sm.st[(rb * NVT + ct) * 64 + lane] = __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));

    const rsrc_t rw_ = make_rsrc(a.ws + seq * size_t(a.nchunks) * kWsChunk, uint32_t(nchunks) * kWsChunk);
    const uint32_t vbytes = uint32_t(sp.len) * uint32_t(DV) * 2u;
    const rsrc_t rv = make_rsrc(a.v + tok0 * DV, vbytes);
    const rsrc_t ro = make_rsrc(a.o + tok0 * DV, vbytes);
    constexpr uint32_t GS = GB ? 2u : 4u;
    const rsrc_t rbeta = make_rsrc(static_cast<const char*>(a.beta) + tok0 * GS, uint32_t(sp.len) * GS);

    // a chunk's loads go out in three parts over the processing of the chunk two before
    // it (each part in program order: the memory-counter waits count the loads after it)
    auto load_part = [&](ChunkRegs<NVT>& R, int ch, int part) {
        const uint32_t cb = uint32_t(ch) * kWsChunk;
        const uint32_t lq = uint32_t((rb * 4) * 64 + lane) * 16u;
        if (part == 0) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) R.q[kk] = buf_ld16(rw_, cb + kWsQ + lq + 1024u * kk);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) R.k[kk] = buf_ld16(rw_, cb + kWsK + lq + 1024u * kk);
            R.b = buf_ld_gate<GB>(rbeta, uint32_t(ch * C + rw));
        } else if (part == 1) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                R.t[kk] = buf_ld16(rw_, cb + kWsT + uint32_t((rb * 2 + kk) * 64 + lane) * 16u);
            const uint32_t ov = ((uint32_t(ch * C) + rw) * uint32_t(DV) + c0 + colmap<NVT>(0, 4 * g)) * 2u;
            if constexpr (NVT == 2) {
                const uint4 v4 = buf_ld16(rv, ov);
                R.v[0] = make_uint2(v4.x, v4.y);
                R.v[1] = make_uint2(v4.z, v4.w);
            } else {
                R.v[0] = buf_ld8(rv, ov);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                R.p[kk] = buf_ld16(rw_, cb + kWsP + uint32_t((rb * 2 + kk) * 64 + lane) * 16u);
#pragma unroll
            for (int x = 0; x < 4; ++x)
                R.kh[x] = buf_ld16(rw_, cb + kWsKh + uint32_t(((2 * rb) * 2 + x) * 64 + lane) * 16u);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
                R.a[ib] = __builtin_bit_cast(float4, buf_ld16(rw_, cb + kWsA + uint32_t(16 * (2 * rb + ib) + 4 * g) * 4u));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_chunk = [&](ChunkRegs<NVT>& R, int ch) {
        load_part(R, ch, 0);
        load_part(R, ch, 1);
        load_part(R, ch, 2);
    };

    auto process = [&](const ChunkRegs<NVT>& R, ChunkRegs<NVT>& Rl, int ch) {
        load_part(Rl, ch + 2, 0);
        const uint32_t t0 = uint32_t(ch) * C;
        const float br = gate_val<GB>(R.b);   // 0 past the end
        // ---- (S^T Q~^T) and (S^T K~^T) for rows 16 rb ..: D[c][r]
        f32x4_t oq[NVT], ks[NVT];
        bf16x8_t sf[DK / 32][NVT];   // every S^T fragment first, so that the reads overlap
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct)
                sf[kk][ct] = __builtin_bit_cast(bf16x8_t, sm.st[(kk * NVT + ct) * 64 + lane]);
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) { oq[ct] = zero4(); ks[ct] = zero4(); }
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                oq[ct] = mfma16(sf[kk][ct], __builtin_bit_cast(bf16x8_t, R.q[kk]), oq[ct]);
                ks[ct] = mfma16(sf[kk][ct], __builtin_bit_cast(bf16x8_t, R.k[kk]), ks[ct]);
            }
        }
        // ---- X[s][c] = beta_s (v_s,c - (S^T k~_s)_c), s = 16 rb + j
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            const uint2 vv = R.v[ct];
            const float vf[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                                 __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
            f32x4_t x_;
#pragma unroll
            for (int j = 0; j < 4; ++j) x_[j] = br * (vf[j] - ks[ct][j]);
            store_rows<NVT>(sm.x, PV, 0, ct, 16 * rb, x_, lane);
        }
        lds_barrier();
        load_part(Rl, ch + 2, 1);
        // ---- U^T = X^T T^T for rows 16 rb .. (every X fragment read before the first U
        // row is written: the compiler keeps LDS reads behind LDS writes it cannot tell
        // apart, which would make each column tile's reads a round trip of its own)
        bf16x8_t xf[2][NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            xf[0][ct] = frag_kr_cols<NVT>(sm.x, PV, 0, 0, ct, lane);
            if (nk > 1) xf[1][ct] = frag_kr_cols<NVT>(sm.x, PV, 32, 0, ct, lane);
        }
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t u_ = mfma16(xf[0][ct], __builtin_bit_cast(bf16x8_t, R.t[0]), zero4());
            if (nk > 1) u_ = mfma16(xf[1][ct], __builtin_bit_cast(bf16x8_t, R.t[1]), u_);
            store_rows<NVT>(sm.u, PV, 0, ct, 16 * rb, u_, lane);
        }
        lds_barrier();
        load_part(Rl, ch + 2, 2);
        // ---- O^T = (S^T Q~^T) + U^T P^T -> o rows 16 rb .. (every U fragment of this
        // and of the state update read first)
        bf16x8_t pu[2][NVT], uf[2][NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            pu[0][ct] = frag_kr_cols_pk<NVT>(sm.u, PV, 0, 0, ct, lane);
            if (nk > 1) pu[1][ct] = frag_kr_cols_pk<NVT>(sm.u, PV, 1, 0, ct, lane);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) uf[kk][ct] = frag_kr_cols<NVT>(sm.u, PV, 32 * kk, 0, ct, lane);
        uint2 ow[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) {
            f32x4_t o_ = mfma16(pu[0][ct], __builtin_bit_cast(bf16x8_t, R.p[0]), oq[ct]);
            if (nk > 1) o_ = mfma16(pu[1][ct], __builtin_bit_cast(bf16x8_t, R.p[1]), o_);
            ow[ct].x = pack_bf16x2(o_[0], o_[1]);
            ow[ct].y = pack_bf16x2(o_[2], o_[3]);
        }
        {
            const uint32_t oo = ((t0 + rw) * uint32_t(DV) + c0 + colmap<NVT>(0, 4 * g)) * 2u;
            if constexpr (NVT == 2) buf_st16_out(ro, oo, make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
            else buf_st8(ro, oo, ow[0]);
        }
        // ---- S = Diag(G_last) S + K^^T U (key rows 32 rb ..), bf16 copy to st
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            const f32x4_t av = {R.a[ib].x, R.a[ib].y, R.a[ib].z, R.a[ib].w};
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                f32x4_t s_ = S[ib][ct] * av;
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kh[2 * ib]), uf[0][ct], s_);
                s_ = mfma16(__builtin_bit_cast(bf16x8_t, R.kh[2 * ib + 1]), uf[1][ct], s_);
                S[ib][ct] = s_;
            }
        }
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
            sm.st[(rb * NVT + ct) * 64 + lane] = __builtin_bit_cast(uint4, pack_pk(S[0][ct], S[1][ct]));
        lds_barrier();
    };

    // three register sets rotate so that each chunk's loads are issued two chunks ahead;
    // whole triples only: a chunk past the end reads zeros (beta = 0, T = P = 0, G = 0
    // keeps nothing), so it stores nothing and its state update is discarded below
    ChunkRegs<NVT> RA, RB, RC;
    load_chunk(RA, 0);
    load_chunk(RB, 1);
    lds_barrier();
    f32x4_t Sfin[2][NVT];   // the state after the sequence's last chunk (S0 if it has none)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) Sfin[ib][ct] = S[ib][ct];
    for (int ch = 0; ch < nchunks; ch += 3) {
        process(RA, RC, ch);
        if (ch + 1 == nchunks) { for (int ib = 0; ib < 2; ++ib) for (int ct = 0; ct < NVT; ++ct) Sfin[ib][ct] = S[ib][ct]; }
        process(RB, RA, ch + 1);
        if (ch + 2 == nchunks) { for (int ib = 0; ib < 2; ++ib) for (int ct = 0; ct < NVT; ++ct) Sfin[ib][ct] = S[ib][ct]; }
        process(RC, RB, ch + 2);
        if (ch + 3 == nchunks) { for (int ib = 0; ib < 2; ++ib) for (int ct = 0; ct < NVT; ++ct) Sfin[ib][ct] = S[ib][ct]; }
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * (2 * rb + ib) + 4 * g + j, c = colmap<NVT>(ct, jl);
                a.S[seq * DK * DV + size_t(i) * DV + c0 + c] = Sfin[ib][ct][j];
            }
}

template <bool GB>
hipError_t launch_gb(const Problem& p) {
    KdaArgs a{};
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.alpha = p.g;
    a.beta = p.beta;
    a.S0 = p.S0;
    a.o = static_cast<uint16_t*>(p.o);
    a.S = p.S;
    a.ws = static_cast<unsigned char*>(p.ws);
    a.N = p.N;
    a.nseq = int(size_t(p.B) * size_t(p.H));
    a.nchunks = (p.L + C - 1) / C;
    a.cu = p.cu;
    a.H = p.H;
    a.L = p.L;
    const bool wide = p.dv >= 32;
    a.ntiles = p.dv / (wide ? 32 : 16);
    {
        const size_t smem = sizeof(PrepSmem);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_prep_kernel<GB>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        const size_t blocks = size_t(xcd_grid(a.nchunks, a.nseq));
        if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
        kda_prep_kernel<GB><<<dim3(unsigned(blocks)), dim3(NTP), smem, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (wide) {
        const size_t smem = sizeof(FwdSmem<32>);
        kda_fwd_kernel<2, GB><<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(NTF), smem, p.stream>>>(a);
    } else {
        const size_t smem = sizeof(FwdSmem<16>);
        kda_fwd_kernel<1, GB><<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(NTF), smem, p.stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

bool kda_mfma_supported(int dk, int dv, bool io_bf16) {
    return io_bf16 && dk == DK && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

size_t kda_mfma_workspace_bytes(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    const size_t nchunks = size_t((p.L + C - 1) / C);
    return nseq * nchunks * kWsChunk;
}

hipError_t launch_prefill_kda_mfma(const Problem& p) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if (nseq > (1u << 24) || !p.ws) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: one sequence's v / o rows and its chunk workspace
    if (size_t(p.L) * DK * 4 >= (size_t(1) << 31)) return hipErrorInvalidValue;
    if (size_t((p.L + C - 1) / C) * kWsChunk >= (size_t(1) << 31)) return hipErrorInvalidValue;
    return p.gate_bf16 ? launch_gb<true>(p) : launch_gb<false>(p);
}

}  // namespace la
