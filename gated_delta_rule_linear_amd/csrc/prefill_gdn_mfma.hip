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
//   forward  one workgroup per (sequence, value tile of 16 or 32 columns): chain waves
//            that each carry 16 columns of the fp32 state through the chunks in
//            registers (columns of S never mix, so a chain needs no other wave's
//            results), and two output waves one chunk behind that form the causal
//            score tiles P_rs = exp(c_r - c_s) q_r.k_s (s <= r) and the outputs
//            O = gamma (S^T q) + P U from the copies of S and U the chains leave in LDS.
//            One barrier per chunk; the tiles of one sequence share an XCD so their
//            q / k / T reads hit the same L2.
//
// Fragments whose K index runs along tile rows use the LDS transpose read; result
// tiles are written to LDS with 8-byte stores.
#include <type_traits>

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
    // T in fragment order with the column slots of a pair of matrix-core result tiles:
    // 16-byte piece (rb, kk, lane = 16 g + j) holds row 16 rb + j, columns 32 kk + 4 g ..
    // + 3 then 32 kk + 16 + 4 g .. + 3, so that a forward wave reads its A fragment as one
    // contiguous kilobyte and multiplies it with a B fragment packed straight from two of
    // its own result tiles
    uint16_t* Tg = a.T + (seq * a.nchunks + ch) * size_t(C * C);
#pragma unroll
    for (int x2 = 0; x2 < 2; ++x2) {
        const int x = tid + NT * x2, rb = x >> 7, kk = (x >> 6) & 1, l = x & 63;
        const int off = (16 * rb + (l & 15)) * PC + 32 * kk + 4 * (l >> 4);
        const uint2 lo = *reinterpret_cast<const uint2*>(sm.t + off);
        const uint2 hi = *reinterpret_cast<const uint2*>(sm.t + off + 16);
        *reinterpret_cast<uint4*>(Tg + 8 * x) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// ---------------------------------------------------------------------------
// forward kernel
// ---------------------------------------------------------------------------
// One workgroup per (sequence, VT = 16 NCW value columns): NCW chain waves and two
// output waves, one workgroup barrier per chunk.
//
// A chain wave owns 16 value columns of the state for all 128 key rows, as eight fp32
// 16 x 16 result tiles in registers (lane 16 g + j: key rows 16 ib + 4 g .. + 3 of
// column j). Columns of S never mix, so its walk over the chunks needs nothing from
// another wave but the chunk's staged operands. For chunk c:
//   S^T (bf16, the state entering the chunk) -> LDS, for the output waves
//   KS = K S                       (A: rows of K; B: S packed from its own tiles)
//   X = beta (V - gamma KS)        (V read in the result-tile layout)
//   U = T X                        (A: T in the order the prep stored it)
//   U^T (bf16) -> LDS, for the output waves
//   S <- gamma_last S + K^T (d U),  d_r = exp(c_last - c_r)   (A: K^T by transpose reads)
// Every B fragment is packed straight from two result tiles, so its K slots come in the
// order the matrix cores return them (rows 4 g .. + 3 of the lower tile, then of the
// upper one), and each matching A fragment is read in that slot order.
//
// The two output waves run one chunk behind: wave p takes the row blocks {0, 3} (p = 0)
// or {1, 2} (p = 1), five causal score tiles each. In the iteration of chunk c they form
// the score tiles P^T_{c-1} = (K Q^T) o D of their rows (D_sr = exp(c_r - c_s), s <= r)
// and write O_{c-1}^T = gamma (S^T Q^T) + U^T P^T from the copies the chain waves left in
// LDS.
//
// The chunk operands that several waves share (K, T) go from global memory straight into
// LDS (buffer loads with an LDS destination, 16 bytes per lane), two chunks ahead, into a
// ring of four slots, every wave copying its share; each wave waits for its own copies of
// the next chunk before the barrier that ends the current one. A chain wave loads its
// value columns straight into registers in the result-tile layout, also two chunks ahead. Every slot is an LDS object of its
// own and the chunk loop is unrolled by four, so the compiler sees which slot each access
// touches and never waits on a copy in flight to another slot. Per-sequence buffer
// resources make every load past the end of the sequence read zero and drop every store
// past it, so ragged tails need no branches.

typedef __attribute__((address_space(3))) void lds_void_t;
// 16 bytes per lane from a buffer straight into LDS at lds + 16 lane (lds wave-uniform).
__device__ __forceinline__ void dma16(rsrc_t r, const uint16_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, 0, 0, 0);
}
// A fragment of the transpose of a row-major [K rows][columns] bf16 tile: M = columns
// n0 .. n0 + 15, K = rows 32 kk .. + 31 in the pair-of-tiles slot order (LDS transpose
// reads: lane L of a 16-lane group addresses row L / 4 of a 4-row block).
__device__ __forceinline__ bf16x8_t frag_tr_pk(const uint16_t* t, int pitch, int kk, int n0,
                                               int lane) {
    const int g = lane >> 4, L = lane & 15;
    const uint16_t* p = t + (32 * kk + 4 * g + (L >> 2)) * pitch + n0 + 4 * (L & 3);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 16 * pitch));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}
// A fragment over K = 32 kk .. + 31 of row `row` of a padded row-major bf16 tile, pair-of-
// tiles slot order.
__device__ __forceinline__ bf16x8_t frag_row_pk(const uint16_t* t, int pitch, int row, int kk,
                                                int lane) {
    const uint16_t* p = t + row * pitch + 32 * kk + 4 * (lane >> 4);
    const uint2 lo = *reinterpret_cast<const uint2*>(p);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ uint2 pack4(f32x4_t d) {
    return make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
}
// s_waitcnt vmcnt(N) (other counters left alone), through the builtin so that the
// compiler's own wait placement knows of it
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int NCW>
struct FwdShape {
    static constexpr int VT = 16 * NCW;
    static constexpr int NW = NCW + 2;                 // waves per workgroup
    // the padded K tile is 64 rows of 17 16-byte pieces (16 of data, one of padding):
    // 17 blocks of 1 KiB; each wave issues KDMA of them (some twice, so that every wave
    // issues the same number)
    static constexpr int KBLK = C * (PQ / 8) / 64;
    static constexpr int KDMA = (KBLK + NW - 1) / NW;
    // T of a chunk is 8 blocks of 1 KiB, split over all waves the same way
    static constexpr int TDMA = (8 + NW - 1) / NW;
    static constexpr int VLD = 16;                     // 2-byte value loads per lane
    // vector-memory operations a wave issues per iteration before the barrier's wait
    // (loads only; the output waves' stores are not counted, so the wait is at least as
    // strict as needed)
    static constexpr int VM_CHAIN = KDMA + TDMA + VLD + 2;
    static constexpr int VM_OUT = KDMA + TDMA + 8 + 1;
    // two iterations of copies in flight stay within the 6-bit vector-memory counter
    static_assert(2 * VM_CHAIN <= 63 && 2 * VM_OUT <= 63, "vmcnt range");
};
static_assert(PQ % 8 == 0 && C * (PQ / 8) % 64 == 0, "padded K rows in whole 1 KiB blocks");

template <int J>
using Ic = std::integral_constant<int, J>;

// One chunk's operands that several waves read: K [s][i] (padded rows) and T in fragment
// order, copied straight from global memory.
struct __align__(16) ChunkSmem {
    __align__(16) uint16_t k[C * PQ];
    __align__(16) uint16_t t[C * C];
};

template <int NCW, bool GB>
__global__ __launch_bounds__(64 * (NCW + 2)) void gdn_fwd_kernel(GdnArgs a) {
    using Sh = FwdShape<NCW>;
    constexpr int VT = Sh::VT, NW = Sh::NW;
    // a ring of four chunks (slot = chunk mod 4), each slot one LDS object holding the
    // chunk's K and T
    __shared__ ChunkSmem sl0, sl1, sl2, sl3;
    __shared__ __align__(16) uint16_t st0[VT * PQ], st1[VT * PQ];   // S^T [col][i]
    __shared__ __align__(16) uint16_t ut0[VT * PC], ut1[VT * PC];   // U^T [col][s]
    __shared__ __align__(16) float gs[NCW + 2][3][C];               // per-wave gate factors
    auto slot_ = [&](auto I) -> ChunkSmem& {
        constexpr int s = decltype(I)::value & 3;
        if constexpr (s == 0) return sl0; else if constexpr (s == 1) return sl1;
        else if constexpr (s == 2) return sl2; else return sl3;
    };
    auto ks_ = [&](auto I) -> uint16_t* { return slot_(I).k; };
    auto ts_ = [&](auto I) -> uint16_t* { return slot_(I).t; };
    auto sts_ = [&](auto I) -> uint16_t* {
        if constexpr ((decltype(I)::value & 1) == 0) return st0; else return st1;
    };
    auto uts_ = [&](auto I) -> uint16_t* {
        if constexpr ((decltype(I)::value & 1) == 0) return ut0; else return ut1;
    };

    const XcdMap mp = xcd_map(blockIdx.x, a.ntiles, a.nseq);
    if (!mp.valid) return;
    const int lane = threadIdx.x & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    const int DV = a.ntiles * VT;
    const int c0 = mp.tile * VT;                 // first column of the tile
    const size_t seq = size_t(mp.seq);
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int nchunks = (sp.len + C - 1) / C;
    // one iteration per chunk plus one for the output waves, in whole groups of four; a
    // chunk past the end reads zeros and leaves the state unchanged
    const int niter = ((nchunks + 1 + 3) / 4) * 4;

    constexpr uint32_t GS = GB ? 2u : 4u;

    // this wave's 1 KiB blocks of the padded K tile: piece p = 64 b + lane is row p / 17,
    // 16-byte chunk p % 17 (chunk 16 is padding, filled with chunk 0); a wave may repeat a
    // block of another so that every wave issues the same number. The global offsets
    // within a chunk are fixed per lane.
    // Each copy's per-lane offset is fixed for the whole walk (registers never rewritten
    // while a copy that names them may still be in flight); the chunk is selected by the
    // buffer resource, built per chunk from scalars with the bytes left in the sequence
    // (none past its end, so those copies fill zeros).
    uint32_t koff[Sh::KDMA];
#pragma unroll
    for (int x = 0; x < Sh::KDMA; ++x) {
        const int b = (w + NW * x) % Sh::KBLK, pz = 64 * b + lane;
        const int row = pz / (PQ / 8), ck = pz % (PQ / 8);
        koff[x] = uint32_t(row * DK + (ck < DK / 8 ? ck : 0) * 8) * 2u;
    }
    auto rows_left = [&](int ch) { return uint32_t(max(0, sp.len - ch * C)); };
    // resources over one chunk (and what follows it in the sequence) of a token-major array
    auto gate_rsrc = [&](const void* base, int ch) {
        return make_rsrc(static_cast<const char*>(base) + (tok0 + size_t(ch) * C) * GS, rows_left(ch) * GS);
    };
    const uint32_t goff = uint32_t(lane) * GS;   // lane = token
    // copies of K of chunk ch into kb
    auto dma_k = [&](uint16_t* kb, int ch) {
        const rsrc_t r = make_rsrc(a.k + (tok0 + size_t(ch) * C) * DK, rows_left(ch) * DK * 2u);
#pragma unroll
        for (int x = 0; x < Sh::KDMA; ++x) {
            const int b = (w + NW * x) % Sh::KBLK;
            dma16(r, kb + b * 512, koff[x]);
        }
    };
    // this wave's 1 KiB blocks of T of a chunk (stored in fragment order by the prep)
    uint32_t toff[Sh::TDMA];
#pragma unroll
    for (int x = 0; x < Sh::TDMA; ++x) toff[x] = uint32_t((w + NW * x) % 8) * 1024u + lane * 16u;
    auto dma_t = [&](uint16_t* tb_, int ch) {
        const rsrc_t r1 = make_rsrc(a.T + (seq * size_t(a.nchunks) + size_t(ch)) * (C * C),
                                    ch < nchunks ? C * C * 2u : 0u);
#pragma unroll
        for (int x = 0; x < Sh::TDMA; ++x) dma16(r1, tb_ + ((w + NW * x) % 8) * 512, toff[x]);
    };
    float (*gw)[C] = gs[w];

    if (w < NCW) {
        // =========================== chain wave ===========================
        const int cb = 16 * w;   // first column of this wave within the tile
        f32x4_t S[8];
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g + e;
                S[ib][e] = a.S0 ? a.S0[seq * DK * DV + size_t(i) * DV + c0 + cb + jl] : 0.f;
            }
        // this lane's value column cb + j of token rows 4 g + e (+ 16 tb), the result-tile
        // layout of KS, straight from global memory
        const uint32_t voff = ((4 * g) * uint32_t(DV) + c0 + cb + jl) * 2u;
        struct VSet { uint32_t v[4][4]; };
        auto load_v = [&](VSet& V, int ch) {
            const rsrc_t r2 = make_rsrc(a.v + (tok0 + size_t(ch) * C) * DV,
                                        rows_left(ch) * uint32_t(DV) * 2u);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    V.v[tb][e] = __builtin_amdgcn_raw_buffer_load_b16(
                        r2, voff + uint32_t((16 * tb + e) * DV * 2), 0, 0);
        };
        VSet VS[4];
        struct Gate { uint32_t ga, gb; };
        auto load_g = [&](Gate& G, int ch) {
            G.ga = buf_ld_gate_off<GB>(gate_rsrc(a.alpha, ch), goff);
            G.gb = buf_ld_gate_off<GB>(gate_rsrc(a.beta, ch), goff);
        };
        Gate G[4];

        auto step = [&](auto J, int ch) {
            constexpr int j = decltype(J)::value;
            dma_k(ks_(Ic<j + 2>{}), ch + 2);
            dma_t(ts_(Ic<j + 2>{}), ch + 2);
            load_v(VS[(j + 2) & 3], ch + 2);
            load_g(G[(j + 2) & 3], ch + 2);
            __builtin_amdgcn_sched_barrier(0);
            const Gate& Gc = G[j];
            const int n = min(C, sp.len - ch * C);
            const uint16_t* kc = ks_(J);
            const uint16_t* tc = ts_(J);
            // per-token gate factors (lane = token; padding rows are identity steps)
            const float lg = lane < n ? fast_log(gate_val<GB>(Gc.ga)) : 0.f;
            const float cum = wave_inclusive_scan(lg);
            const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 63));
            gw[0][lane] = fast_exp(cum);            // gamma_r
            gw[1][lane] = fast_exp(clast - cum);    // d_r
            gw[2][lane] = lane < n ? gate_val<GB>(Gc.gb) : 0.f;
            // S as B fragments (keys in pair-of-tiles slot order), and S^T entering the chunk
            // for the output waves from the same packed words
            bf16x8_t Sb[4];
            uint16_t* stc = sts_(J);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Sb[kk] = pack_pk(S[2 * kk], S[2 * kk + 1]);
                const uint4 wd = __builtin_bit_cast(uint4, Sb[kk]);
                *reinterpret_cast<uint2*>(stc + (cb + jl) * PQ + 32 * kk + 4 * g) = make_uint2(wd.x, wd.y);
                *reinterpret_cast<uint2*>(stc + (cb + jl) * PQ + 32 * kk + 16 + 4 * g) = make_uint2(wd.z, wd.w);
            }
            // KS = K S, rows 16 tb + 4 g + e; the next row block's A fragments are read
            // while the current one's products issue
            f32x4_t ks[4];
            bf16x8_t ka[2][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) ka[0][kk] = frag_row_pk(kc, PQ, jl, kk, lane);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                if (tb < 3) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        ka[(tb + 1) & 1][kk] = frag_row_pk(kc, PQ, 16 * (tb + 1) + jl, kk, lane);
                }
                ks[tb] = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) ks[tb] = mfma16(ka[tb & 1][kk], Sb[kk], ks[tb]);
            }
            // T fragments and the value tile (independent of the state)
            bf16x8_t tf[6];
            const int pc[6] = {0, 2, 4, 5, 6, 7};   // piece 2 tb + kk of T
#pragma unroll
            for (int x = 0; x < 6; ++x)
                tf[x] = *reinterpret_cast<const bf16x8_t*>(tc + (pc[x] * 64 + lane) * 8);
            float vv[4][4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[tb][e] = __uint_as_float(VS[j].v[tb][e] << 16);
            wave_lds_sync();   // this wave's gate factors are in LDS
            // X = beta (V - gamma KS)
            f32x4_t X[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float4 g4 = *reinterpret_cast<const float4*>(&gw[0][16 * tb + 4 * g]);
                const float4 b4 = *reinterpret_cast<const float4*>(&gw[2][16 * tb + 4 * g]);
                X[tb][0] = b4.x * (vv[tb][0] - g4.x * ks[tb][0]);
                X[tb][1] = b4.y * (vv[tb][1] - g4.y * ks[tb][1]);
                X[tb][2] = b4.z * (vv[tb][2] - g4.z * ks[tb][2]);
                X[tb][3] = b4.w * (vv[tb][3] - g4.w * ks[tb][3]);
            }
            const bf16x8_t Xb0 = pack_pk(X[0], X[1]), Xb1 = pack_pk(X[2], X[3]);
            // U = T X (T lower triangular: row blocks 0, 1 need tokens 0..31 only)
            f32x4_t u[4];
            u[0] = mfma16(tf[0], Xb0, zero4());
            u[1] = mfma16(tf[1], Xb0, zero4());
            u[2] = mfma16(tf[2], Xb0, zero4());
            u[2] = mfma16(tf[3], Xb1, u[2]);
            u[3] = mfma16(tf[4], Xb0, zero4());
            u[3] = mfma16(tf[5], Xb1, u[3]);
            // U^T for the output waves
            uint16_t* utc = uts_(J);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                *reinterpret_cast<uint2*>(utc + (cb + jl) * PC + 16 * tb + 4 * g) = pack4(u[tb]);
            // S <- gamma_last S + K^T (d U)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float4 d4 = *reinterpret_cast<const float4*>(&gw[1][16 * tb + 4 * g]);
                u[tb][0] *= d4.x; u[tb][1] *= d4.y; u[tb][2] *= d4.z; u[tb][3] *= d4.w;
            }
            const bf16x8_t Ub0 = pack_pk(u[0], u[1]), Ub1 = pack_pk(u[2], u[3]);
            const float glast = fast_exp(clast);
            bf16x8_t kt[2][2];
            kt[0][0] = frag_tr_pk(kc, PQ, 0, 0, lane);
            kt[0][1] = frag_tr_pk(kc, PQ, 1, 0, lane);
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) {
                if (ib < 7) {
                    kt[(ib + 1) & 1][0] = frag_tr_pk(kc, PQ, 0, 16 * (ib + 1), lane);
                    kt[(ib + 1) & 1][1] = frag_tr_pk(kc, PQ, 1, 16 * (ib + 1), lane);
                }
                f32x4_t s_ = S[ib] * glast;
                s_ = mfma16(kt[ib & 1][0], Ub0, s_);
                s_ = mfma16(kt[ib & 1][1], Ub1, s_);
                S[ib] = s_;
            }
            // the next chunk's K and T (copies issued an iteration ago) have landed
            wait_vmcnt<Sh::VM_CHAIN>();
            lds_barrier();
        };

        dma_k(sl0.k, 0);
        dma_t(sl0.t, 0);
        dma_k(sl1.k, 1);
        dma_t(sl1.t, 1);
        load_v(VS[0], 0);
        load_v(VS[1], 1);
        load_g(G[0], 0);
        load_g(G[1], 1);
        wait_vmcnt<0>();
        lds_barrier();
        for (int ch = 0; ch < niter; ch += 4) {
            step(Ic<0>{}, ch);
            step(Ic<1>{}, ch + 1);
            step(Ic<2>{}, ch + 2);
            step(Ic<3>{}, ch + 3);
        }
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g + e;
                a.S[seq * DK * DV + size_t(i) * DV + c0 + cb + jl] = S[ib][e];
            }
    } else {
        // =========================== output wave ===========================
        struct QSet {
            uint4 q[2][4];    // rows 16 rb + j of q (the wave's two row blocks), keys 32 kk + 8 g ..
            uint32_t ga;
        };
        auto run = [&](auto pc) {
            constexpr int P = decltype(pc)::value;
            constexpr int RB[2] = {P == 0 ? 0 : 1, P == 0 ? 3 : 2};
            // per-lane offsets of the wave's q rows within a chunk and of its output rows
            uint32_t qoff[2], ooff[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                qoff[h] = ((16 * RB[h] + jl) * DK + 8 * g) * 2u;
                ooff[h] = ((16 * RB[h] + jl) * uint32_t(DV) + c0 + 4 * g) * 2u;
            }
            auto load_q = [&](QSet& Q, int ch) {
                Q.ga = buf_ld_gate_off<GB>(gate_rsrc(a.alpha, ch), goff);
                const rsrc_t r = make_rsrc(a.q + (tok0 + size_t(ch) * C) * DK, rows_left(ch) * DK * 2u);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) Q.q[h][kk] = buf_ld16_off(r, qoff[h], 64 * kk);
            };
            // rows of row block RB[h] of chunk cp: scores, then outputs
            auto rows = [&](const QSet& Qp, auto hc, const rsrc_t& orc, const uint16_t* kc,
                            const uint16_t* stc, const uint16_t* utc) {
                constexpr int h = decltype(hc)::value;
                constexpr int rb = RB[h];
                const int r = 16 * rb + jl;
                const float crr = gw[0][r];
                f32x4_t pt[4] = {zero4(), zero4(), zero4(), zero4()};
                bf16x8_t kf[2][4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kf[0][kk] = frag_kc(kc, PQ, 0, 32 * kk, lane);
#pragma unroll
                for (int sb = 0; sb <= rb; ++sb) {
                    if (sb < rb) {
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            kf[(sb + 1) & 1][kk] = frag_kc(kc, PQ, 16 * (sb + 1), 32 * kk, lane);
                    }
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        pt[sb] = mfma16(kf[sb & 1][kk], __builtin_bit_cast(bf16x8_t, Qp.q[h][kk]), pt[sb]);
                }
                bf16x8_t sf[NCW][4];
#pragma unroll
                for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) sf[ct][kk] = frag_kc(stc, PQ, 16 * ct, 32 * kk, lane);
                bf16x8_t uf[NCW][2];
#pragma unroll
                for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
                    for (int kk = 0; kk < (rb >= 2 ? 2 : 1); ++kk)
                        uf[ct][kk] = frag_row_pk(utc, PC, 16 * ct + jl, kk, lane);
#pragma unroll
                for (int sb = 0; sb <= rb; ++sb) {
                    const float4 cs = *reinterpret_cast<const float4*>(&gw[0][16 * sb + 4 * g]);
                    const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * sb + 4 * g + e;
                        const float x = fast_exp(crr - csv[e]) * pt[sb][e];
                        pt[sb][e] = (sb < rb || s <= r) ? x : 0.f;
                    }
                }
                const bf16x8_t pf0 = pack_pk(pt[0], pt[1]), pf1 = pack_pk(pt[2], pt[3]);
                const float gr = fast_exp(crr);
                // O^T = gamma (S^T Q^T) + U^T P^T: columns 16 ct + 4 g .. of token r
#pragma unroll
                for (int ct = 0; ct < NCW; ++ct) {
                    f32x4_t oq = zero4();
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        oq = mfma16(sf[ct][kk], __builtin_bit_cast(bf16x8_t, Qp.q[h][kk]), oq);
                    f32x4_t o_ = oq * gr;
                    o_ = mfma16(uf[ct][0], pf0, o_);
                    if constexpr (rb >= 2) o_ = mfma16(uf[ct][1], pf1, o_);
                    buf_st8_off(orc, ooff[h], 32 * ct, pack4(o_));
                }
            };
            QSet Q[4];   // chunk x's q in set x mod 4, loaded two iterations ahead
            auto step = [&](auto J, int ch) {
                constexpr int j = decltype(J)::value;
                dma_k(ks_(Ic<j + 2>{}), ch + 2);
                dma_t(ts_(Ic<j + 2>{}), ch + 2);
                load_q(Q[(j + 2) & 3], ch + 2);
                __builtin_amdgcn_sched_barrier(0);
                const int cp = ch - 1;
                if (cp >= 0) {
                    const QSet& Qp = Q[(j + 3) & 3];
                    const int n = min(C, sp.len - cp * C);
                    const float lg = lane < n ? fast_log(gate_val<GB>(Qp.ga)) : 0.f;
                    gw[0][lane] = wave_inclusive_scan(lg);
                    wave_lds_sync();
                    const uint16_t* kc = ks_(Ic<j + 3>{});
                    const uint16_t* stc = sts_(Ic<j + 1>{});
                    const uint16_t* utc = uts_(Ic<j + 1>{});
                    const rsrc_t orc = make_rsrc(a.o + (tok0 + size_t(cp) * C) * DV,
                                                 rows_left(cp) * uint32_t(DV) * 2u);
                    rows(Qp, Ic<0>{}, orc, kc, stc, utc);
                    rows(Qp, Ic<1>{}, orc, kc, stc, utc);
                }
                wait_vmcnt<Sh::VM_OUT>();
                lds_barrier();
            };
            dma_k(sl0.k, 0);
            dma_t(sl0.t, 0);
            dma_k(sl1.k, 1);
            dma_t(sl1.t, 1);
            load_q(Q[0], 0);
            load_q(Q[1], 1);
            wait_vmcnt<0>();
            lds_barrier();
            for (int ch = 0; ch < niter; ch += 4) {
                step(Ic<0>{}, ch);
                step(Ic<1>{}, ch + 1);
                step(Ic<2>{}, ch + 2);
                step(Ic<3>{}, ch + 3);
            }
        };
        if (w == NCW) run(Ic<0>{});
        else run(Ic<1>{});
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

template <int NCW, bool GB>
hipError_t launch_cfg(const Problem& p) {
    constexpr int VT = 16 * NCW;
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
    gdn_fwd_kernel<NCW, GB>
        <<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(64 * (NCW + 2)), 0, p.stream>>>(a);
    return hipGetLastError();
}

template <bool GB>
hipError_t launch_gb(const Problem& p) {
    return p.dv >= 32 ? launch_cfg<2, GB>(p) : launch_cfg<1, GB>(p);
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
    if (p.gate_bf16) return launch_gb<true>(p);
    return launch_gb<false>(p);
}

}  // namespace la
