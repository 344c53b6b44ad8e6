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
//            every chunk, written to the workspace as T diag(beta) in bf16 and in MFMA
//            fragment order (T depends only on the chunk's k, alpha, beta, never on the
//            state; with beta folded in, U = (T diag(beta)) (V - gamma K S));
//   forward  one workgroup per (sequence, value tile of 16 or 32 columns): chain waves
//            that each carry 16 columns of the fp32 state through the chunks in
//            registers (columns of S never mix, so a chain needs no other wave's
//            results), and output waves one chunk behind that form the causal score
//            tiles P_rs = exp(c_r - c_s) q_r.k_s (s <= r) and the outputs
//            O = gamma (S^T q) + P U from the copies of S and U the chains leave in LDS.
//            One barrier per chunk; the tiles of one sequence share an XCD so their
//            q / k / T reads hit the same L2.
//
#include <type_traits>

#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int DK = 128;
constexpr int C = kMfmaChunk;  // 64
constexpr int NT = 256;
constexpr int PQ = DK + 16;    // pitch (elements) of [*][128] bf16 tiles (72 dwords: 16-byte
                               // reads of 16 rows at one column are free of bank conflicts)
constexpr int PC = C + 8;      // pitch of [*][64] bf16 tiles
constexpr int PD = 16 + 4;     // pitch of the fp32 16 x 16 diagonal L blocks
constexpr int PY = 32 + 8;     // pitch of the bf16 32-row scratch tiles
// T in fragment order is eight 1 KiB pieces 2 rb + kk; pieces 1 and 3 (row blocks 0 and 1,
// tokens 32..63) are zero since T is lower triangular, so the workspace holds the other
// six: stored piece i is fragment piece t_piece(i).
constexpr int TPC = 6;
constexpr int TCH = TPC * 512;  // bf16 elements of T per chunk in the workspace
__host__ __device__ constexpr int t_piece(int i) { return i < 2 ? 2 * i : i + 2; }

// 40 KiB, so that four workgroups share a compute unit: the level scratch tiles reuse
// the K tile, which no wave reads after the L products.
struct __align__(16) PrepSmem {
    union {
        __align__(16) uint16_t k[C * PQ];
        struct {
            __align__(16) uint16_t ya[2][32 * PY];  // level-a scratch: Y = L_ij T_jj (rows 0..15
                                                    // written; the products mask the rest)
            __align__(16) uint16_t yb[32 * PY];     // level-b scratch: Y = L[32:64, 0:32] A^{-1}
        };
    };
    __align__(16) uint16_t t[C * PC];             // T [r][s]
    __align__(16) uint16_t lo[(C - 16) * PC];     // off-diagonal blocks of L, rows 16..63 [r - 16][s]
    __align__(16) float ld[4][16 * PD];           // diagonal blocks of L, fp32
    float cum[C], beta[C];
};
static_assert(sizeof(PrepSmem) <= 40960, "four prep workgroups per compute unit");

struct GdnArgs {
    const uint16_t *q, *k, *v;
    const void *alpha, *beta;
    const float* S0;
    uint16_t* o;
    float* S;
    uint16_t* T;   // workspace: [nseq][nchunks][TCH] bf16, T diag(beta) per chunk (six pieces)
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
// Persistent: a grid of a few workgroups per compute unit walks the (sequence, chunk)
// units; each iteration issues the next unit's loads (K rows and the gates, through
// per-chunk buffer resources that read zeros past the sequence's end) before it works on
// the current one, so the load latency is hidden behind the previous chunk's work.
template <bool GB>
__global__ __launch_bounds__(NT) void gdn_prep_kernel(GdnArgs a, int nunits) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int g = lane >> 4, jl = lane & 15;
    constexpr uint32_t GS = GB ? 2u : 4u;
    // a unit's loads, and its sequence span (found once, when its loads are issued: with a
    // packed batch that reads the sequence bounds, and a wait for them must not fall
    // after the next unit's loads)
    struct In { uint4 kv[4]; uint32_t graw; size_t base; int len; };
    // waves 0 and 1 load the gates alpha and beta, the others alpha again (unused), so
    // that every thread issues the same loads
    auto load = [&](int u, In& in) {
        const int seq = u / a.nchunks, ch = u % a.nchunks;
        const SeqSpan sp = seq_span(seq, a.H, a.N, a.L, a.cu);
        in.base = sp.base;
        in.len = sp.len;
        const int t0 = ch * C;
        const uint32_t rows_left = uint32_t(max(0, sp.len - t0));
        const rsrc_t rk = make_rsrc(a.k + (sp.base + t0) * DK, rows_left * DK * 2u);
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const int x = tid + NT * x4, r = x >> 4, col = (x & 15) * 8;
            in.kv[x4] = buf_ld16_off(rk, uint32_t(r * DK + col) * 2u, 0);
        }
        const void* gp = w == 1 ? a.beta : a.alpha;
        const rsrc_t rg = make_rsrc(static_cast<const char*>(gp) + (sp.base + t0) * GS, rows_left * GS);
        in.graw = buf_ld_gate_off<GB>(rg, uint32_t(lane) * GS);
    };
    auto chunk = [&](int u, const In& in) {
    const size_t seq = size_t(u / a.nchunks);
    const int ch = u % a.nchunks;
    const SeqSpan sp{in.base, in.len};
    const int t0 = ch * C, n = min(C, sp.len - t0);
    if (n <= 0) return;   // past this sequence's end: the forward reads zeros instead
    const uint4* kv = in.kv;
    const uint32_t graw = in.graw;
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
        // zero the six upper blocks of T
        const int r = lane >> 2, cc = (lane & 3) * 4;
        const int ub[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};
        for (int x = w - 2; x < 6; x += 2)
            *reinterpret_cast<uint2*>(sm.t + (16 * ub[x][0] + r) * PC + 16 * ub[x][1] + cc) =
                make_uint2(0, 0);
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
            store_dT(sm.lo, PC, 16 * sb, 16 * (rb - 1), d, lane);
        }
    }
    lds_barrier();
    // level a: T_10 = -T_11 L_10 T_00 (wave 1), T_32 = -T_33 L_32 T_22 (wave 2)
    if (w == 1 || w == 2) {
        const int i = w == 1 ? 1 : 3, j = i - 1;
        uint16_t* y = sm.ya[w - 1];
        // Y^T = T_jj^T L_ij^T -> y[r][jj] (rows 0..15)
        f32x4_t d = mfma16(k16(frag_kr(sm.t, PC, 16 * j, 16 * j, lane), lane),
                           k16(frag_kc(sm.lo, PC, 16 * (i - 1), 16 * j, lane), lane), zero4());
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
                                 frag_kc(sm.lo, PC, 16 + 16 * rb, 0, lane), zero4());
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
    // T diag(beta) (so that the forward forms U = (T diag(beta)) (V - gamma K S) without
    // scaling by beta itself), its six nonzero pieces in fragment order with the column slots of a pair of
    // matrix-core result tiles: 16-byte piece (rb, kk, lane = 16 g + j) holds row 16 rb + j,
    // columns 32 kk + 4 g .. + 3 then 32 kk + 16 + 4 g .. + 3, so that a forward wave reads
    // its A fragment as one contiguous kilobyte and multiplies it with a B fragment packed
    // straight from two of its own result tiles
    uint16_t* Tg = a.T + (seq * a.nchunks + ch) * size_t(TCH);
#pragma unroll
    for (int x2 = 0; x2 < 2; ++x2) {
        const int x = tid + NT * x2;
        if (x >= TPC * 64) break;
        const int pi = t_piece(x >> 6), rb = pi >> 1, kk = pi & 1, l = x & 63;
        const int c = 32 * kk + 4 * (l >> 4);
        const int off = (16 * rb + (l & 15)) * PC + c;
        uint32_t wv[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint2 t2 = *reinterpret_cast<const uint2*>(sm.t + off + 16 * hh);
            const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + c + 16 * hh);
            wv[2 * hh] = pack_bf16x2(__uint_as_float(t2.x << 16) * b4.x,
                                     __uint_as_float(t2.x & 0xffff0000u) * b4.y);
            wv[2 * hh + 1] = pack_bf16x2(__uint_as_float(t2.y << 16) * b4.z,
                                         __uint_as_float(t2.y & 0xffff0000u) * b4.w);
        }
        *reinterpret_cast<uint4*>(Tg + 8 * x) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    };

    // two input sets, swapped by unrolling rather than copied (a copy would wait for the
    // loads in flight): each step issues the next unit's loads into the other set, then
    // works on its own
    auto step = [&](int& u, const In& cur, In& nxt) -> bool {
        const int un = u + int(gridDim.x);
        if (un < nunits) load(un, nxt);
        chunk(u, cur);
        lds_barrier();   // every wave is done with this unit's LDS before the next writes it
        u = un;
        return un < nunits;
    };
    int u = blockIdx.x;
    if (u >= nunits) return;
    In ia, ib;
    load(u, ia);
    while (step(u, ia, ib) && step(u, ib, ia)) {
    }
}

// ---------------------------------------------------------------------------
// forward kernel
// ---------------------------------------------------------------------------
// One workgroup per (sequence, VT = 16 NCB value columns, NCB = 1 or 2): NCB chain waves
// (waves 0 and 1) and four output waves (waves 2 .. 5), one workgroup barrier per chunk.
// Waves w and w + 4 share a SIMD. A wave does not issue vector ALU work while its own
// matrix-core product runs, but another wave on the same SIMD does, so each chain wave is
// paired with one of the two lightest output waves, whose work fills the chain's stalls.
//
// Chain wave c owns 16 value columns (16 c .. + 15 of the tile) of the state for all 128
// key rows, as eight fp32 16 x 16 result tiles in registers. Its walk over the chunks
// needs nothing from the other waves but the chunk's staged operands. For chunk c:
//   S^T (bf16, the state entering the chunk) -> LDS, for the output waves
//   KS = K S                       (A: rows of K)
//   X = V - gamma KS               (V read in the result-tile layout)
//   U = T diag(beta) X             (A: T diag(beta) as the prep stored it)
//   U^T (bf16) -> LDS, for the output waves
//   S <- gamma_last S + K^T (d U),  d_r = exp(c_last - c_r)   (A: K^T by transpose reads)
// The state's key rows are kept in a permuted order: row 4 g + e of tiles 2 kk and 2 kk + 1
// (lane 16 g + j) hold keys 32 kk + 8 g + e and 32 kk + 8 g + 4 + e. A sum over keys does
// not depend on their order, and with this one the B fragment packed from two result tiles
// carries keys 32 kk + 8 g .. + 7 in natural order, so K's rows are read 16 bytes at a time
// and S^T is written 16 bytes at a time. The token slots of the products over the chunk
// come in the order the matrix cores return them (rows 4 g .. + 3 of the lower tile, then
// of the upper one), and each matching A fragment is read in that order. S^T and U^T go
// to LDS in the order the chain wave holds them, 16 contiguous bytes per lane (strided
// LDS writes cost several times more than contiguous ones).
//
// The four output waves run one chunk behind: output wave p (wave 2 + p) takes row block
// 3 - p (28, 24, 18 and 14 products). In the iteration of chunk c it forms the score tiles
// P^T_{c-1} = (K Q^T) o D of its rows (D_sr = exp(c_r - c_s), s <= r) and writes
// O_{c-1}^T = gamma (S^T Q^T) + U^T P^T from the copies the chain waves left in LDS.
//
// The chunk operands (K, T, the value tile) go from global memory straight into LDS
// (buffer loads with an LDS destination, 16 bytes per lane), two chunks ahead, into a ring
// of four slots; the output waves issue all of these copies, every fourth 1 KiB block each,
// and wait for their own copies of the next chunk before the barrier that ends the current
// one. Output wave 0 also lays out each chunk's gate factors one chunk ahead. Every slot is
// an LDS object of its own and the chunk loop is unrolled by four, so the compiler sees
// which slot each access touches and never waits on a copy in flight to another slot.
// Per-sequence buffer resources make every load past the end of the sequence read zero and
// drop every store past it, so ragged tails need no branches.

typedef __attribute__((address_space(3))) void lds_void_t;
// 16 bytes per lane from a buffer straight into LDS at lds + 16 lane (lds wave-uniform).
__device__ __forceinline__ void dma16(rsrc_t r, const uint16_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, voff, 0, 0, 0);
}
// A fragment of K^T for the state update: M = the 16 state rows of tile 2 kk + h in the
// permuted key order (keys 32 kk + 4 h + 8 q + e, q, e < 4), K = tokens 32 tkk .. + 31 in
// the pair-of-tiles slot order. LDS transpose reads: lane L of a 16-lane group addresses
// token row L / 4 of a 4-row block and four keys that land in lanes 4 (L & 3) .. + 3.
__device__ __forceinline__ bf16x8_t frag_kt(const uint16_t* t, int tkk, int kk, int h, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const uint16_t* p = t + (32 * tkk + 4 * g + (L >> 2)) * PQ + 32 * kk + 4 * h + 8 * (L & 3);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 16 * PQ));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
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

template <int NCB>
struct FwdShape {
    static constexpr int VT = 16 * NCB;
    static constexpr int NW = 6;                       // waves per workgroup
    static constexpr int NO = 4;                       // output waves
    // Copies into LDS are issued by the output waves, output wave p taking the 1 KiB
    // blocks p, p + 4, ...: the padded K tile (64 rows of PQ / 8 16-byte pieces), T (8
    // blocks) and the value tile (64 rows of VT / 8 pieces).
    static constexpr int KBLK = C * (PQ / 8) / 64;
    static constexpr int TBLK = TPC;   // the stored pieces of T
    static constexpr int VBLK = C * (VT / 8) / 64;
    static constexpr int share(int nb, int p) { return (nb - p + NO - 1) / NO; }
    // vector-memory loads output wave p issues per iteration: copies, q rows, and the
    // gates for wave 0 (its stores come after them, so waiting for all but this many is
    // at least as strict as needed)
    static constexpr int vm_out(int p) {
        return share(KBLK, p) + share(TBLK, p) + share(VBLK, p) + 4 + (p == 0 ? 1 : 0);
    }
    // two iterations of loads in flight stay within the 6-bit vector-memory counter
    static_assert(2 * vm_out(0) <= 63, "vmcnt range");
};
static_assert(PQ % 8 == 0 && C * (PQ / 8) % 64 == 0, "padded K rows in whole 1 KiB blocks");

template <int J>
using Ic = std::integral_constant<int, J>;

// Value column of state column j (0..15) of chain wave cb within the tile. With two chain
// waves the columns interleave in fours (wave cb holds 8 q + 4 cb + r, j = 4 q + r), so
// the output rows the result tiles of both waves give one lane are eight contiguous
// columns: one 16-byte store per lane and row block. Sums over value columns do not exist
// in this kernel, so the order is free.
template <int NCB>
__device__ __forceinline__ int tile_col(int cb, int j) {
    return NCB == 2 ? 8 * (j >> 2) + 4 * cb + (j & 3) : 16 * cb + j;
}

// One chunk's operands as the waves read them, copied straight from global memory: K
// [s][i] (padded rows), T in fragment order, the value tile [s][col].
template <int VT>
struct __align__(16) ChunkSmem {
    __align__(16) uint16_t k[C * PQ];
    __align__(16) uint16_t t[C * C];
    __align__(16) uint16_t v[C * VT];
};

template <int NCB, bool GB>
__global__ __launch_bounds__(384) void gdn_fwd_kernel(GdnArgs a) {
    using Sh = FwdShape<NCB>;
    constexpr int VT = Sh::VT;
    // a ring of four chunks (slot = chunk mod 4), each slot one LDS object
    __shared__ ChunkSmem<VT> sl0, sl1, sl2, sl3;
    // S^T and U^T as the output waves' A fragments, in the order the chain wave holds them
    // (fragment-major, 16 bytes per lane: every write and read covers 1 KiB contiguously)
    __shared__ __align__(16) uint16_t st0[NCB * 4 * 512], st1[NCB * 4 * 512];
    __shared__ __align__(16) uint16_t ut0[NCB * 2 * 512], ut1[NCB * 2 * 512];
    // per-chunk gate factors (slot = chunk mod 4): cumulative log gate c_r, gamma_r =
    // exp(c_r), d_r = exp(c_last - c_r)
    __shared__ __align__(16) float gsl[4][3][C];
    auto slot_ = [&](auto I) -> ChunkSmem<VT>& {
        constexpr int s = decltype(I)::value & 3;
        if constexpr (s == 0) return sl0; else if constexpr (s == 1) return sl1;
        else if constexpr (s == 2) return sl2; else return sl3;
    };
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

    if (w < 2) {
        // =========================== chain wave ===========================
        // Reads only LDS: the chunk's K, T and value tile and its gate factors are in
        // place when the iteration starts. S[2 kk + h][e] is key 32 kk + 8 g + 4 h + e of
        // column c0 + tile_col(cb, j).
        const int cb = w;
        f32x4_t S[8];
        auto key = [&](int ib, int e) { return 32 * (ib >> 1) + 8 * g + 4 * (ib & 1) + e; };
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[ib][e] = (a.S0 && cb < NCB) ? a.S0[seq * DK * DV + size_t(key(ib, e)) * DV + c0 + tile_col<NCB>(cb, jl)]
                                              : 0.f;

        auto step = [&](auto J) {
            constexpr int j = decltype(J)::value;
            if (cb >= NCB) {   // no columns for this wave: keep the barriers only
                lds_barrier();
                return;
            }
            const uint16_t* kc = slot_(J).k;
            const uint16_t* tc = slot_(J).t;
            const uint16_t* vc = slot_(J).v;
            const float (*gc)[C] = gsl[j & 3];
            // The chunk's value tile (transpose reads: lane j receives column tile_col(cb, j)
            // of rows 16 tb + 4 g .. + 3, the result-tile layout) and its gate factors, read
            // before any LDS write of this step: the compiler keeps LDS reads behind earlier
            // LDS writes it cannot tell apart, so read later each would be a round trip of
            // its own on the chain's dependent path.
            i16x4_t vx[4];
            float4 g4[4], d4[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint16_t* p = vc + (16 * tb + 4 * g + (jl >> 2)) * VT + tile_col<NCB>(cb, 4 * (jl & 3));
                vx[tb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
                g4[tb] = *reinterpret_cast<const float4*>(&gc[1][16 * tb + 4 * g]);
                d4[tb] = *reinterpret_cast<const float4*>(&gc[2][16 * tb + 4 * g]);
            }
            const float glast = gc[1][C - 1];
            // S as B fragments (keys 32 kk + 8 g .. + 7), and S^T entering the chunk for
            // the output waves from the same words (row 16 cb + j, keys 32 kk + 8 g ..: the
            // output waves' A fragment (cb, kk) of lane 16 g + j)
            bf16x8_t Sb[4];
            uint16_t* stc = sts_(J);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Sb[kk] = pack_pk(S[2 * kk], S[2 * kk + 1]);
                *reinterpret_cast<bf16x8_t*>(stc + ((4 * cb + kk) * 64 + lane) * 8) = Sb[kk];
            }
            // KS = K S, rows 16 tb + 4 g + e; the next row block's A fragments are read
            // while the current one's products issue
            f32x4_t ks[4];
            bf16x8_t ka[2][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) ka[0][kk] = frag_kc(kc, PQ, 0, 32 * kk, lane);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                if (tb < 3) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        ka[(tb + 1) & 1][kk] = frag_kc(kc, PQ, 16 * (tb + 1), 32 * kk, lane);
                }
                ks[tb] = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) ks[tb] = mfma16(ka[tb & 1][kk], Sb[kk], ks[tb]);
            }
            // T fragments
            bf16x8_t tf[6];
            const int pc[6] = {0, 2, 4, 5, 6, 7};   // piece 2 tb + kk of T
#pragma unroll
            for (int x = 0; x < 6; ++x)
                tf[x] = *reinterpret_cast<const bf16x8_t*>(tc + (pc[x] * 64 + lane) * 8);
            // X = V - gamma KS (beta is folded into T)
            f32x4_t X[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float gv[4] = {g4[tb].x, g4[tb].y, g4[tb].z, g4[tb].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = __uint_as_float(uint32_t(uint16_t(vx[tb][e])) << 16);
                    X[tb][e] = v - gv[e] * ks[tb][e];
                }
            }
            const bf16x8_t Xb0 = pack_pk(X[0], X[1]), Xb1 = pack_pk(X[2], X[3]);
            // U = T X (T lower triangular: row blocks 0, 1 need tokens 0..31 only); U^T for
            // the output waves (row 16 cb + j, tokens of tiles 2 kk and 2 kk + 1 in the pair-
            // of-tiles slot order: their A fragment (cb, kk)); then d U as B fragments
            f32x4_t u[4];
            u[0] = mfma16(tf[0], Xb0, zero4());
            u[1] = mfma16(tf[1], Xb0, zero4());
            u[2] = mfma16(tf[2], Xb0, zero4());
            u[3] = mfma16(tf[4], Xb0, zero4());
            u[2] = mfma16(tf[3], Xb1, u[2]);
            u[3] = mfma16(tf[5], Xb1, u[3]);
            uint16_t* utc = uts_(J);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                *reinterpret_cast<bf16x8_t*>(utc + ((2 * cb + kk) * 64 + lane) * 8) =
                    pack_pk(u[2 * kk], u[2 * kk + 1]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                u[tb][0] *= d4[tb].x; u[tb][1] *= d4[tb].y; u[tb][2] *= d4[tb].z; u[tb][3] *= d4[tb].w;
            }
            const bf16x8_t Ub0 = pack_pk(u[0], u[1]), Ub1 = pack_pk(u[2], u[3]);
            // S <- gamma_last S + K^T (d U)
            bf16x8_t kt[2][2];
            kt[0][0] = frag_kt(kc, 0, 0, 0, lane);
            kt[0][1] = frag_kt(kc, 1, 0, 0, lane);
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) {
                if (ib < 7) {
                    kt[(ib + 1) & 1][0] = frag_kt(kc, 0, (ib + 1) >> 1, (ib + 1) & 1, lane);
                    kt[(ib + 1) & 1][1] = frag_kt(kc, 1, (ib + 1) >> 1, (ib + 1) & 1, lane);
                }
                f32x4_t s_ = S[ib] * glast;
                s_ = mfma16(kt[ib & 1][0], Ub0, s_);
                s_ = mfma16(kt[ib & 1][1], Ub1, s_);
                S[ib] = s_;
            }
            lds_barrier();
        };

        lds_barrier();
        for (int ch = 0; ch < niter; ch += 4) {
            step(Ic<0>{});
            step(Ic<1>{});
            step(Ic<2>{});
            step(Ic<3>{});
        }
        if (cb < NCB) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.S[seq * DK * DV + size_t(key(ib, e)) * DV + c0 + tile_col<NCB>(cb, jl)] = S[ib][e];
        }
    } else {
        // =========================== output wave ===========================
        // Output wave p (waves 2 .. 5) copies every fourth 1 KiB block of the chunk operands
        // two chunks ahead, output wave 0 also loads the gates three chunks ahead and lays
        // out the next chunk's gate factors; each then writes the outputs of its row block of
        // the chunk before the chain's.
        constexpr uint32_t GS = GB ? 2u : 4u;
        auto rows_left = [&](int ch) { return uint32_t(max(0, sp.len - ch * C)); };
        auto gate_rsrc = [&](const void* base, int ch) {
            return make_rsrc(static_cast<const char*>(base) + (tok0 + size_t(ch) * C) * GS,
                             rows_left(ch) * GS);
        };
        const uint32_t goff = uint32_t(lane) * GS;   // lane = token
        struct Gate { uint32_t ga; };
        auto run = [&](auto pc) {
            constexpr int P = decltype(pc)::value;
            constexpr int NRB = 1;
            constexpr int RL = 3 - P, RF = RL;   // the wave's row block
            constexpr int NK = Sh::share(Sh::KBLK, P), NT_ = Sh::share(Sh::TBLK, P),
                          NV = Sh::share(Sh::VBLK, P);
            // Each copy's per-lane offset is fixed for the whole walk (registers never
            // rewritten while a copy that names them may still be in flight); the chunk is
            // selected by the buffer resource, built per chunk from scalars with the bytes
            // left in the sequence (none past its end, so those copies fill zeros).
            // K: piece 64 b + lane of the padded tile is row / column piece (pieces past the
            // 16 of a row are padding, filled with piece 0)
            uint32_t koff[NK], toff[NT_], voff[NV > 0 ? NV : 1];
#pragma unroll
            for (int x = 0; x < NK; ++x) {
                const int pz = 64 * (Sh::NO * x + P) + lane;
                const int row = pz / (PQ / 8), ck = pz % (PQ / 8);
                koff[x] = uint32_t(row * DK + (ck < DK / 8 ? ck : 0) * 8) * 2u;
            }
#pragma unroll
            for (int x = 0; x < NT_; ++x) toff[x] = uint32_t(Sh::NO * x + P) * 1024u + lane * 16u;   // stored piece
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                const int pz = 64 * (Sh::NO * x + P) + lane;
                const int row = pz / (VT / 8), ck = pz % (VT / 8);
                voff[x] = uint32_t(row * DV + c0 + 8 * ck) * 2u;
            }
            auto copies = [&](ChunkSmem<VT>& dst, int ch) {
                const rsrc_t rk = make_rsrc(a.k + (tok0 + size_t(ch) * C) * DK, rows_left(ch) * DK * 2u);
#pragma unroll
                for (int x = 0; x < NK; ++x) dma16(rk, dst.k + (Sh::NO * x + P) * 512, koff[x]);
                const rsrc_t rt = make_rsrc(a.T + (seq * size_t(a.nchunks) + size_t(ch)) * TCH,
                                            ch < nchunks ? TCH * 2u : 0u);
#pragma unroll
                for (int x = 0; x < NT_; ++x) dma16(rt, dst.t + t_piece(Sh::NO * x + P) * 512, toff[x]);
                const rsrc_t rv = make_rsrc(a.v + (tok0 + size_t(ch) * C) * DV,
                                            rows_left(ch) * uint32_t(DV) * 2u);
#pragma unroll
                for (int x = 0; x < NV; ++x) dma16(rv, dst.v + (Sh::NO * x + P) * 512, voff[x]);
            };
            // per-lane offsets of the wave's q rows within a chunk and of its output rows
            uint32_t qoff[NRB], ooff[NRB];
#pragma unroll
            for (int h = 0; h < NRB; ++h) {
                const int rb = h == NRB - 1 ? RL : RF;
                qoff[h] = ((16 * rb + jl) * DK + 8 * g) * 2u;
                ooff[h] = ((16 * rb + jl) * uint32_t(DV) + c0 + (NCB == 2 ? 8 : 4) * g) * 2u;
            }
            struct QSet {
                uint4 q[NRB][4];   // rows 16 rb + j of q (the wave's row blocks), keys 32 kk + 8 g ..
            };
            auto load_q = [&](QSet& Q, int ch) {
                const rsrc_t r = make_rsrc(a.q + (tok0 + size_t(ch) * C) * DK, rows_left(ch) * DK * 2u);
#pragma unroll
                for (int h = 0; h < NRB; ++h)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) Q.q[h][kk] = buf_ld16_off(r, qoff[h], 64 * kk);
            };
            auto load_g = [&](Gate& G, int ch) { G.ga = buf_ld_gate_off<GB>(gate_rsrc(a.alpha, ch), goff); };
            // gate factors of chunk ch (lane = token; padding rows are identity steps)
            auto gates = [&](const Gate& G, int ch, float (*dst)[C]) {
                const int n = min(C, sp.len - ch * C);
                const float lg = lane < n ? fast_log(gate_val<GB>(G.ga)) : 0.f;
                const float cum = wave_inclusive_scan(lg);
                const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 63));
                dst[0][lane] = cum;
                dst[1][lane] = fast_exp(cum);
                dst[2][lane] = fast_exp(clast - cum);
            };
            // the wave's row blocks of chunk cp: scores, then outputs
            auto rows = [&](const QSet& Qp, const rsrc_t& orc, const uint16_t* kc,
                            const uint16_t* stc, const uint16_t* utc, const float* cum) {
                // score tiles P^T[s][r] of the row blocks (h = NRB - 1: RL, h = 0: RF), each K
                // block read once
                f32x4_t pt[NRB][4];
#pragma unroll
                for (int h = 0; h < NRB; ++h)
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) pt[h][sb] = zero4();
                bf16x8_t kf[2][4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kf[0][kk] = frag_kc(kc, PQ, 0, 32 * kk, lane);
#pragma unroll
                for (int sb = 0; sb <= RL; ++sb) {
                    if (sb < RL) {
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            kf[(sb + 1) & 1][kk] = frag_kc(kc, PQ, 16 * (sb + 1), 32 * kk, lane);
                    }
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        pt[NRB - 1][sb] = mfma16(kf[sb & 1][kk], __builtin_bit_cast(bf16x8_t, Qp.q[NRB - 1][kk]),
                                                 pt[NRB - 1][sb]);
                        if (NRB == 2 && sb <= RF)
                            pt[0][sb] = mfma16(kf[sb & 1][kk], __builtin_bit_cast(bf16x8_t, Qp.q[0][kk]), pt[0][sb]);
                    }
                }
                // S^T and U^T fragments, read once for all the row blocks
                bf16x8_t sf[NCB][4];
#pragma unroll
                for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        sf[ct][kk] = *reinterpret_cast<const bf16x8_t*>(stc + ((4 * ct + kk) * 64 + lane) * 8);
                bf16x8_t uf[NCB][2];
#pragma unroll
                for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                    for (int kk = 0; kk < (RL >= 2 ? 2 : 1); ++kk)
                        uf[ct][kk] = *reinterpret_cast<const bf16x8_t*>(utc + ((2 * ct + kk) * 64 + lane) * 8);
#pragma unroll
                for (int h = 0; h < NRB; ++h) {
                    const int rb = h == NRB - 1 ? RL : RF;
                    const int r = 16 * rb + jl;
                    const float crr = cum[r];
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) {
                        if (sb > rb) continue;
                        const float4 cs = *reinterpret_cast<const float4*>(&cum[16 * sb + 4 * g]);
                        const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = 16 * sb + 4 * g + e;
                            const float x = fast_exp(crr - csv[e]) * pt[h][sb][e];
                            pt[h][sb][e] = (sb < rb || s <= r) ? x : 0.f;
                        }
                    }
                    const bf16x8_t pf0 = pack_pk(pt[h][0], pt[h][1]), pf1 = pack_pk(pt[h][2], pt[h][3]);
                    const float gr = fast_exp(crr);
                    // O^T = gamma (S^T Q^T) + U^T P^T: value columns tile_col(ct, 4 g ..) of
                    // token r, both chain waves' four columns stored together
                    uint2 ow[NCB];
#pragma unroll
                    for (int ct = 0; ct < NCB; ++ct) {
                        f32x4_t oq = zero4();
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            oq = mfma16(sf[ct][kk], __builtin_bit_cast(bf16x8_t, Qp.q[h][kk]), oq);
                        f32x4_t o_ = oq * gr;
                        o_ = mfma16(uf[ct][0], pf0, o_);
                        if (rb >= 2) o_ = mfma16(uf[ct][1], pf1, o_);
                        ow[ct] = pack4(o_);
                    }
                    if constexpr (NCB == 2) buf_st16_out(orc, ooff[h], make_uint4(ow[0].x, ow[0].y, ow[1].x, ow[1].y));
                    else buf_st8_off(orc, ooff[h], 0, ow[0]);
                }
            };
            QSet Q[4];   // chunk x's q in set x mod 4, loaded two iterations ahead
            Gate G[4];   // chunk x's gates in set x mod 4, loaded three iterations ahead
            auto step = [&](auto J, int ch) {
                constexpr int j = decltype(J)::value;
                copies(slot_(Ic<j + 2>{}), ch + 2);
                load_q(Q[(j + 2) & 3], ch + 2);
                if constexpr (P == 0) load_g(G[(j + 3) & 3], ch + 3);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (P == 0) gates(G[(j + 1) & 3], ch + 1, gsl[(j + 1) & 3]);
                const int cp = ch - 1;
                if (cp >= 0) {
                    const rsrc_t orc = make_rsrc(a.o + (tok0 + size_t(cp) * C) * DV,
                                                 rows_left(cp) * uint32_t(DV) * 2u);
                    rows(Q[(j + 3) & 3], orc, slot_(Ic<j + 3>{}).k, sts_(Ic<j + 1>{}),
                         uts_(Ic<j + 1>{}), gsl[(j + 3) & 3][0]);
                }
                wait_vmcnt<Sh::vm_out(P)>();
                lds_barrier();
            };
            copies(sl0, 0);
            copies(sl1, 1);
            load_q(Q[0], 0);
            load_q(Q[1], 1);
            if constexpr (P == 0) {
                load_g(G[0], 0);
                load_g(G[1], 1);
                load_g(G[2], 2);
            }
            wait_vmcnt<0>();
            if constexpr (P == 0) gates(G[0], 0, gsl[0]);
            lds_barrier();
            for (int ch = 0; ch < niter; ch += 4) {
                step(Ic<0>{}, ch);
                step(Ic<1>{}, ch + 1);
                step(Ic<2>{}, ch + 2);
                step(Ic<3>{}, ch + 3);
            }
        };
        if (w == 2) run(Ic<0>{});
        else if (w == 3) run(Ic<1>{});
        else if (w == 4) run(Ic<2>{});
        else run(Ic<3>{});
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

template <int NCB, bool GB>
hipError_t launch_cfg(const Problem& p) {
    constexpr int VT = 16 * NCB;
    GdnArgs a = make_args(p);
    a.ntiles = p.dv / VT;
    hipError_t e;
    {
        const size_t smem = sizeof(PrepSmem);
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_prep_kernel<GB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        const size_t units = size_t(a.nseq) * size_t(a.nchunks);
        if (units > 0x7fffffffull) return hipErrorInvalidValue;
        // four workgroups fit a compute unit's LDS
        const size_t grid = std::min(units, size_t(device_cus()) * 4);
        gdn_prep_kernel<GB><<<dim3(unsigned(grid)), dim3(NT), smem, p.stream>>>(a, int(units));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    gdn_fwd_kernel<NCB, GB>
        <<<dim3(xcd_grid(a.ntiles, a.nseq)), dim3(64 * FwdShape<NCB>::NW), 0, p.stream>>>(a);
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
    return size_t(p.B) * size_t(p.H) * nchunks * TCH * sizeof(uint16_t);
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
