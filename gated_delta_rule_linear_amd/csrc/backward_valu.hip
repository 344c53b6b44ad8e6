// Backward of the chunked prefill for the diagonal transitions (GLA: one gate per key
// dim, "Linear / RNN 路线" section 2.2; SSD: one decay per token, sections 3.6 and 4.1),
// in fp32 on the vector ALUs with chunk C = 16 and per-element decays (cumulative gates
// in base-2 logarithms, decay factors by the hardware base-2 exponential).
//
// For a loss with dL/do = dO and dL/dS_final, with B_r the cumulative log gate inside a
// chunk (per key dim), S_in the state entering it and dS_out the gradient of the state
// leaving it (everything after the chunk), the reverse-mode derivative of the chunked
// forward is, for rows r, s of the chunk (s <= r, mask M; written with exp, computed
// as exp2 of base-2 logarithms):
//   A    = (dO V^T) o M                       (only this workgroup's value columns)
//   P_rs = sum_i q_ri k_si exp(B_ri - B_si)    (s <= r)
//   dV_s = sum_{r>=s} P_rs dO_r + K^_s dS_out,  K^_si = k_si exp(B_last,i - B_si)
//   dQ_ri = exp(B_ri) (dO_r . S_in[i,:]) + sum_{s<=r} A_rs k_si exp(B_ri - B_si)
//   dK_si = sum_{r>=s} A_rs q_ri exp(B_ri - B_si) + exp(B_last,i - B_si) (dS_out[i,:] . v_s)
//   dS_in = diag(exp(B_last)) dS_out + sum_r diag(exp(B_r)) q_r dO_r^T
// The gate gradient is taken directly, dL/dg_s,i = sum_c dS_s[i,c] S_{s-1}[i,c] (summed
// over i as well for SSD's one decay), with every element's token states S_{s-1} rebuilt
// forward from S_in and its gradients dS_s backward from dS_out inside the chunk. (The
// equivalent closed form g_s dL/dg_s = sum_{t>=s} (q_t dq_t - k_t dk_t) + the final-state
// term is a reverse cumulative sum whose terms cancel down to O(g_s); dividing by g_s
// amplifies fp32 rounding by 1/g_s, so it is not used.)
//
// Only the chunk-to-chunk carries are sequential, and they are elementwise: with the
// chunk's state contribution dS_c = sum_s diag(exp(B_last - B_s)) k_s v_s^T, its output-
// gradient contribution G_c = sum_r diag(exp(B_r)) q_r dO_r^T and its decay a_c =
// exp(B_last),
//   S_in[c+1] = a_c o S_in[c] + dS_c,    dS_out[c-1] = a_c o dS_out[c] + G_c.
// So the work runs in three kernels: sums (every chunk in parallel: dS_c, G_c, a_c), scans
// (one thread per state element walks the chunks forward for S_in and backward for
// dS_out, in place), and grads (every chunk in parallel, looping over the value tiles: dV,
// and dQ, dK and dg summed over the tiles).
//
// KATH (normalised ELU+1 attention, "Linear / RNN 路线" section 2.1) is the same machinery
// with gate 1, phi(q) and phi(k) in place of q and k, and one more value column. With
// num_t = S_t^T phi(q_t) and den_t = phi(q_t).z_t + eps, o_t = num_t / den_t gives dL/dnum_t
// = do_t / den_t and dL/dden_t = -(do_t . o_t) / den_t; the normaliser z is a state column
// whose value is 1 and whose output gradient is dL/dden, so the augmented state [S, z]
// follows S_t = S_{t-1} + phi(k_t) [v_t, 1]^T and the GLA formulas with dO = [dnum, dden]
// give dphi(q), dphi(k), dv, dS0 and dz0 at once. dnum and dden need the forward's num_t
// and den_t, so the sums and scans run in two halves: the state half first (S_in and z_in of
// every chunk), then a kernel that forms num_t and den_t of every chunk in parallel from them
// and writes dnum and dden, then the gradient half. The chain rule through phi is phi'(x) =
// min(phi(x), 1).
#include "common.hpp"
#include "la_internal.h"

namespace la {
namespace {

constexpr int C = kValuChunk;  // 16
constexpr int VT = 16;         // value columns per workgroup
constexpr int NT = 256;

struct BwdArgs {
    const void *q, *k, *v, *g, *dO;
    const float *S0, *dSf;
    void *dq, *dk, *dv, *dg;
    float* dS0;
    float *dnum, *dden;         // KATH: dL/dnum [tokens][DV] and dL/dden [tokens] (fp32)
    const float *z0, *dzf;      // KATH: initial normaliser and its final gradient, or null
    float* dz0;                 // KATH
    float eps;                  // KATH
    int mode;                   // sums and scans: bit 0 the state half, bit 1 the gradient half
    float* Sst;      // [nseq][nchunks][DK][DV]: dS_c, then S_in (in place)
    float* dSt;      // [nseq][nchunks][DK][DV]: G_c, then dS_out (in place)
    float* ac;       // [nseq][nchunks][DK] (GLA) or [nseq][nchunks] (SSD): chunk decay
    int N, nseq, ntiles, nchunks;
    int io_bf16, gate_bf16;
};

template <int VAR>
constexpr bool scalar_gate() { return VAR == LA_SSD || VAR == LA_KATH; }

constexpr bool scalar_gate_rt(int variant) { return variant == LA_SSD || variant == LA_KATH; }

// Columns of the carried state: d_v, plus one tile whose first column is KATH's normaliser.
template <int VAR, int DV>
constexpr int state_width() { return DV + (VAR == LA_KATH ? VT : 0); }

// One chunk's operands in LDS: q, k, the gates and their cumulative base-2 logarithms,
// and the value tile of v and dO. Rows past the end are zero with gate 1.
template <int DK, bool SG>
struct ChunkSmem {
    static constexpr int DKP = DK + 1;
    float q[C][DKP], k[C][DKP];
    float lg[SG ? 1 : C][SG ? 1 : DKP];   // cumulative log2 gate (per key dim)
    float gt[SG ? 1 : C][SG ? 1 : DKP];   // the gates themselves
    float sc[C], sgt[C];                  // the same for one gate per token
    // decay factors, all <= 1: eq = exp(B_r), ek = exp(B_last - B_s) per (row, key dim), or
    // per row with one gate per token, and the pair factors exp(B_r - B_s) (s <= r) of the
    // one-gate case
    float eq[SG ? 1 : C][SG ? 1 : DKP], ek[SG ? 1 : C][SG ? 1 : DKP];
    float seq[C], sek[C], pd[SG ? C : 1][SG ? C + 1 : 1];
    float v[C][VT], dO[C][VT];
};

// The loaders below fix the storage type once per call and read rows past the end of the
// sequence as its last row (zeroed afterwards), so their loads form one straight run that
// the compiler can issue together instead of one branch per element.

// The value tile (columns c0 .. c0 + VT - 1) of v and dO for one chunk, one element of each
// per thread: fetched into registers (so the next tile can be in flight while this one
// works), then stashed in LDS. KATH's extra tile holds the normaliser column (v = 1, output
// gradient dden).
template <int VAR, int DV>
__device__ __forceinline__ float2 fetch_tile(const BwdArgs& a, size_t tok0, int t0, int n, int c0) {
    constexpr bool KA = VAR == LA_KATH;
    const int tid = threadIdx.x;
    const bool iob = a.io_bf16 != 0;
    const int r = tid / VT, c = tid % VT;
    const size_t tk = tok0 + t0 + min(r, n - 1), e = tk * DV + c0 + c;   // n >= 1
    float vv = 0.f, dd = 0.f;
    if (!KA) {
        if (iob) {
            vv = ld<uint16_t>(a.v, e);
            dd = ld<uint16_t>(a.dO, e);
        } else {
            vv = ld<float>(a.v, e);
            dd = ld<float>(a.dO, e);
        }
    } else if (c0 < DV) {
        vv = iob ? ld<uint16_t>(a.v, e) : ld<float>(a.v, e);
        dd = a.dnum[e];
    } else if (c == 0) {   // the normaliser column
        vv = 1.f;
        dd = a.dden[tk];
    }
    return make_float2(vv, dd);
}

template <int DK, bool SG>
__device__ __forceinline__ void stash_tile(ChunkSmem<DK, SG>& sm, float2 x, int n) {
    const int r = int(threadIdx.x) / VT, c = int(threadIdx.x) % VT;
    sm.v[r][c] = r < n ? x.x : 0.f;
    sm.dO[r][c] = r < n ? x.y : 0.f;
}

template <int VAR, int DK, int DV, bool SG>
__device__ __forceinline__ void load_tile(ChunkSmem<DK, SG>& sm, const BwdArgs& a, size_t tok0,
                                          int t0, int n, int c0) {
    stash_tile(sm, fetch_tile<VAR, DV>(a, tok0, t0, n, c0), n);
}

template <int VAR, int DK, int DV, bool SG>
__device__ __forceinline__ void load_chunk(ChunkSmem<DK, SG>& sm, const BwdArgs& a, size_t tok0,
                                           int t0, int n, int c0) {
    constexpr bool KA = VAR == LA_KATH;
    const int tid = threadIdx.x;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    constexpr int NL = C * DK / NT;   // elements per thread (n >= 1)
    static_assert(NL * NT == C * DK, "row tiling");
    auto qk = [&](auto tag) {
        using T = decltype(tag);
        float qv[NL], kv[NL];
#pragma unroll
        for (int m = 0; m < NL; ++m) {
            const int idx = tid + NT * m, r = idx / DK, i = idx % DK;
            const size_t e = (tok0 + t0 + min(r, n - 1)) * DK + i;
            qv[m] = ld<T>(a.q, e);
            kv[m] = ld<T>(a.k, e);
        }
#pragma unroll
        for (int m = 0; m < NL; ++m) {
            const int idx = tid + NT * m, r = idx / DK, i = idx % DK;
            sm.q[r][i] = r < n ? (KA ? elu_plus_one(qv[m]) : qv[m]) : 0.f;
            sm.k[r][i] = r < n ? (KA ? elu_plus_one(kv[m]) : kv[m]) : 0.f;
        }
    };
    auto gates = [&](auto tag) {
        using T = decltype(tag);
        float gv[NL];
#pragma unroll
        for (int m = 0; m < NL; ++m) {
            const int idx = tid + NT * m, r = idx / DK, i = idx % DK;
            gv[m] = ld<T>(a.g, (tok0 + t0 + min(r, n - 1)) * DK + i);
        }
#pragma unroll
        for (int m = 0; m < NL; ++m) {
            const int idx = tid + NT * m, r = idx / DK, i = idx % DK;
            const float g_ = r < n ? gv[m] : 1.f;
            sm.gt[r][i] = g_;
            sm.lg[r][i] = __builtin_amdgcn_logf(g_);
        }
    };
    if (iob)
        qk(uint16_t{});
    else
        qk(float{});
    if (!SG) {
        if (gb)
            gates(uint16_t{});
        else
            gates(float{});
    }
    if (SG && tid < C) {
        const float gv = (tid < n && !KA) ? load_elem(a.g, tok0 + t0 + tid, gb) : 1.f;
        sm.sgt[tid] = gv;
        sm.sc[tid] = __builtin_amdgcn_logf(gv);
    }
    load_tile<VAR, DK, DV, SG>(sm, a, tok0, t0, n, c0);
    __syncthreads();
    if (!SG) {
        for (int i = tid; i < DK; i += NT) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) { acc += sm.lg[r][i]; sm.lg[r][i] = acc; }
        }
    } else if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) { acc += sm.sc[r]; sm.sc[r] = acc; }
    }
    __syncthreads();
    if (!SG) {
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            sm.eq[r][i] = __builtin_amdgcn_exp2f(sm.lg[r][i]);
            sm.ek[r][i] = __builtin_amdgcn_exp2f(sm.lg[C - 1][i] - sm.lg[r][i]);
        }
    } else {
        const int r = tid / C, s = tid % C;   // C * C = NT
        sm.pd[r][s] = s <= r ? __builtin_amdgcn_exp2f(sm.sc[r] - sm.sc[s]) : 0.f;
        if (tid < C) {
            sm.seq[tid] = __builtin_amdgcn_exp2f(sm.sc[tid]);
            sm.sek[tid] = __builtin_amdgcn_exp2f(sm.sc[C - 1] - sm.sc[tid]);
        }
    }
    __syncthreads();
}

// workgroup -> (sequence, chunk)
struct ChunkUnit {
    size_t seq;
    int ch;
};

// ---------------------------------------------------------------------------- sums
// one workgroup per (sequence, chunk): the chunk's rows and decay tables once, then every
// value tile in turn
template <int VAR, int DK, int DV>
__global__ __launch_bounds__(NT, VAR == LA_GLA ? 2 : 6) void bwd_sums_kernel(BwdArgs a) {
    constexpr bool SG = scalar_gate<VAR>();
    constexpr int SW = state_width<VAR, DV>();
    __shared__ ChunkSmem<DK, SG> sm;
    ChunkUnit u;
    u.ch = int(blockIdx.x % unsigned(a.nchunks));
    u.seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = u.ch * C, n = min(C, a.N - t0);
    const size_t tok0 = u.seq * size_t(a.N);
    load_chunk<VAR, DK, DV, SG>(sm, a, tok0, t0, n, 0);   // rows and tile 0
    auto EQ = [&](int r, int i) { return SG ? sm.seq[r] : sm.eq[r][i]; };
    auto EK = [&](int r, int i) { return SG ? sm.sek[r] : sm.ek[r][i]; };
    const size_t sbase = (u.seq * a.nchunks + u.ch) * size_t(DK) * SW;
    // thread -> key dim i and CPT consecutive columns of every tile; its decayed key and
    // query columns stay in registers across the tiles, so a multiply-add reads LDS once
    // (a value row element shared by the lanes of one column run)
    constexpr int CPT = DK * VT / NT;
    static_assert(CPT >= 1 && CPT * NT == DK * VT, "columns per thread");
    const int i = int(threadIdx.x) % DK, cb = (int(threadIdx.x) / DK) * CPT;
    float wk[C], wq[C];
#pragma unroll
    for (int s_ = 0; s_ < C; ++s_) {
        wk[s_] = EK(s_, i) * sm.k[s_][i];
        wq[s_] = EQ(s_, i) * sm.q[s_][i];
    }
    auto put = [&](float* dst, const float (&x)[CPT]) {
        if constexpr (CPT % 4 == 0) {
#pragma unroll
            for (int u2 = 0; u2 < CPT; u2 += 4)
                *reinterpret_cast<float4*>(dst + u2) = make_float4(x[u2], x[u2 + 1], x[u2 + 2], x[u2 + 3]);
        } else {
#pragma unroll
            for (int u2 = 0; u2 < CPT; ++u2) dst[u2] = x[u2];
        }
    };
    float2 nx = make_float2(0.f, 0.f);   // the next tile's v and dO element
    if (a.ntiles > 1) nx = fetch_tile<VAR, DV>(a, tok0, t0, n, VT);
    for (int tile = 0; tile < a.ntiles; ++tile) {
        const int c0 = tile * VT;
        if (tile > 0) {
            __syncthreads();   // the previous tile's readers are done
            stash_tile(sm, nx, n);
            if (tile + 1 < a.ntiles) nx = fetch_tile<VAR, DV>(a, tok0, t0, n, c0 + VT);
            __syncthreads();
        }
        const size_t o = sbase + size_t(i) * SW + c0 + cb;
        if (a.mode & 1) {   // dS_c = sum_s diag(e^{B_last - B_s}) k_s v_s^T
            float ds[CPT] = {};
#pragma unroll
            for (int s_ = 0; s_ < C; ++s_)
#pragma unroll
                for (int u2 = 0; u2 < CPT; ++u2) ds[u2] += wk[s_] * sm.v[s_][cb + u2];
            put(a.Sst + o, ds);
        }
        if (a.mode & 2) {   // G_c = sum_r diag(e^{B_r}) q_r dO_r^T
            float gq[CPT] = {};
#pragma unroll
            for (int s_ = 0; s_ < C; ++s_)
#pragma unroll
                for (int u2 = 0; u2 < CPT; ++u2) gq[u2] += wq[s_] * sm.dO[s_][cb + u2];
            put(a.dSt + o, gq);
        }
    }
    {
        float* ac = a.ac + (u.seq * a.nchunks + u.ch) * (SG ? 1 : DK);
        if (SG) {
            if (threadIdx.x == 0) ac[0] = __builtin_amdgcn_exp2f(sm.sc[C - 1]);
        } else {
            for (int i = threadIdx.x; i < DK; i += NT) ac[i] = __builtin_amdgcn_exp2f(sm.lg[C - 1][i]);
        }
    }
}

// ---------------------------------------------------------------------------- scans
// One thread per state element (sequence, i, j): S_in forward, dS_out backward, in place.
template <int VAR, int DK, int DV>
__global__ __launch_bounds__(NT) void bwd_scans_kernel(BwdArgs a) {
    constexpr bool SG = scalar_gate<VAR>();
    constexpr int SW = state_width<VAR, DV>();
    const size_t e = size_t(blockIdx.x) * NT + threadIdx.x;
    if (e >= size_t(a.nseq) * DK * SW) return;
    const size_t seq = e / (size_t(DK) * SW), ij = e % (size_t(DK) * SW);
    const int i = int(ij / SW), col = int(ij % SW);
    const size_t stride = size_t(DK) * SW;
    const size_t es = (seq * DK + i) * DV + col;   // the [B,H,dk,dv] element (col < DV)
    const size_t ez = seq * DK + i;                // the [B,H,dk] element (col == DV)
    float* Ss = a.Sst + seq * a.nchunks * stride + ij;
    float* dSs = a.dSt + seq * a.nchunks * stride + ij;
    const float* ac = a.ac + seq * a.nchunks * (SG ? 1 : DK) + (SG ? 0 : i);
    float S = 0.f, dS = 0.f;
    if (col < DV) {
        if (a.S0) S = a.S0[es];
        if (a.dSf) dS = a.dSf[es];
    } else if (col == DV) {
        if (a.z0) S = a.z0[ez];
        if (a.dzf) dS = a.dzf[ez];
    }
    // Chunks go in batches of SB: the batch's sums and decays are loaded before any of
    // its stores, so the loads are in flight together instead of each waiting behind the
    // previous chunk's store to the same array. Wider batches pay off where the per-key-dim
    // decays add a third load per chunk; the scalar-gate scans run near the HBM rate at 8.
    constexpr int SB = SG ? 8 : 32;
    const int astr = SG ? 1 : DK;
    for (int c0 = 0; (a.mode & 1) && c0 < a.nchunks; c0 += SB) {
        float d[SB], g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int ch = c0 + b;
            d[b] = ch < a.nchunks ? Ss[ch * stride] : 0.f;
            g[b] = ch < a.nchunks ? ac[ch * astr] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int ch = c0 + b;
            if (ch < a.nchunks) Ss[ch * stride] = S;
            S = g[b] * S + d[b];
        }
    }
    if (!(a.mode & 2)) return;
    for (int c1 = a.nchunks - 1; c1 >= 0; c1 -= SB) {
        float d[SB], g[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int ch = c1 - b;
            d[b] = ch >= 0 ? dSs[ch * stride] : 0.f;
            g[b] = ch >= 0 ? ac[ch * astr] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int ch = c1 - b;
            if (ch >= 0) dSs[ch * stride] = dS;
            dS = g[b] * dS + d[b];
        }
    }
    if (col < DV) a.dS0[es] = dS;
    else if (col == DV) a.dz0[ez] = dS;
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1, 0xf, 0xf>(v);
    v += dpp_f<0x4E, 0xf, 0xf>(v);
    v += dpp_f<0x141, 0xf, 0xf>(v);
    v += dpp_f<0x140, 0xf, 0xf>(v);
    return v;
}

// KATH, one workgroup per (sequence, chunk): the forward's numerator num_t = phi(q_t)^T S_t
// and denominator den_t (state and normaliser entering the chunk, from the state half of
// the scans, plus the causal in-chunk part; fp32) give dnum = dO / den and dden = -(dO .
// num) / den^2, the output gradients of the state and normaliser recurrences. Every global
// load of the chunk is issued at once and staged in LDS, so a chunk waits on memory about
// once; DV / 16 wavefronts (at most 4), each over its own slice of
// the value columns, and each thread owns RPG rows x 4 columns of num.
constexpr int kath_out_threads(int dv) { return 64 * (dv / 16 < 4 ? dv / 16 : 4); }
template <int DK, int DV>
__global__ __launch_bounds__(kath_out_threads(DV)) void kath_out_kernel(BwdArgs a) {
    constexpr int SW = DV + VT, L = kath_out_threads(DV), NW = L / 64;
    constexpr int CG = DV / 4 / NW, RG = 64 / CG, RPG = C / RG;   // per wave: column groups,
    static_assert(RG * RPG == C && RG * CG == 64, "thread tiling"); // row groups
    constexpr int EP = 256 / L, LP = C / EP;   // P entries per thread, threads per row of P
    static_assert(EP * L == C * C, "P tiling");
    constexpr int TP = C + 4;                  // transposed row pitch, float4 aligned
    constexpr int NQ = C * DK / L, NS = DK * DV / 4 / L, NV = C * DV / L;   // loads per thread
    static_assert(NQ * L == C * DK && NS * 4 * L == DK * DV && NV * L == C * DV, "loads");
    __shared__ __align__(16) float sqT[DK][TP];     // phi(q): [key dim][row]
    __shared__ __align__(16) float skT[DK][TP];     // phi(k): [key dim][row]
    __shared__ __align__(16) float sS[DK][DV];      // state entering the chunk
    __shared__ __align__(16) float sv[C][DV];
    __shared__ float sP[C][C + 1], sz[DK], sden[C], sw[NW][C];
    const int lane = threadIdx.x;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0), nl = n - 1;   // n >= 1
    const size_t tok = seq * size_t(a.N) + t0;
    const bool iob = a.io_bf16 != 0;
    const size_t sbase = (seq * a.nchunks + ch) * size_t(DK) * SW;
    const int wv = lane / 64, cg = lane % CG, r0 = (lane % 64 / CG) * RPG;
    const int x0 = 4 * (wv * CG + cg);

    // all loads first (rows past the end clamped to the last row and zeroed below), with
    // the storage type fixed once so that the loads are not split by per-element branches
    float qr[NQ], kr[NQ], vr[NV], dr[RPG][4];
    auto load_all = [&](auto tag) {
        using T = decltype(tag);
        const T* q = static_cast<const T*>(a.q);
        const T* k = static_cast<const T*>(a.k);
        const T* v = static_cast<const T*>(a.v);
        const T* dO = static_cast<const T*>(a.dO);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int idx = lane + L * m, r = idx / DK, i = idx % DK;
            const size_t e = (tok + min(r, nl)) * DK + i;
            qr[m] = to_f32(q[e]);
            kr[m] = to_f32(k[e]);
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int idx = lane + L * m, r = idx / DV, c = idx % DV;
            vr[m] = to_f32(v[(tok + min(r, nl)) * DV + c]);
        }
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                dr[rr][u] = to_f32(dO[(tok + min(r0 + rr, nl)) * DV + x0 + u]);
    };
    if (iob)
        load_all(uint16_t{});
    else
        load_all(float{});
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int idx = lane + L * m, i = idx / (DV / 4), c4 = idx % (DV / 4);
        *reinterpret_cast<float4*>(&sS[i][4 * c4]) =
            *reinterpret_cast<const float4*>(a.Sst + sbase + size_t(i) * SW + 4 * c4);
    }
    for (int i = lane; i < DK; i += L) sz[i] = a.Sst[sbase + size_t(i) * SW + DV];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
        const int idx = lane + L * m, r = idx / DK, i = idx % DK;
        sqT[i][r] = r < n ? elu_plus_one(qr[m]) : 0.f;
        skT[i][r] = r < n ? elu_plus_one(kr[m]) : 0.f;
    }
#pragma unroll
    for (int m = 0; m < NV; ++m) {
        const int idx = lane + L * m, r = idx / DV, c = idx % DV;
        sv[r][c] = r < n ? vr[m] : 0.f;
    }
    __syncthreads();
    {
        // P_ts = phi(q_t) . phi(k_s) (s <= t), thread -> row t, columns s0 .. s0 + EP - 1;
        // den_t = phi(q_t) . z_in + sum_s P_ts + eps, the z part split over the LP threads
        // (consecutive lanes) of row t
        const int t = lane / LP, s0 = (lane % LP) * EP;
        float p[EP] = {}, zq = 0.f;
#pragma unroll 4
        for (int i = 0; i < DK; ++i) {
            const float qi = sqT[i][t];
#pragma unroll
            for (int u = 0; u < EP; ++u) p[u] += qi * skT[i][s0 + u];
        }
        for (int i = lane % LP; i < DK; i += LP) zq += sqT[i][t] * sz[i];
#pragma unroll
        for (int u = 0; u < EP; ++u) {
            const float pu = s0 + u <= t ? p[u] : 0.f;
            sP[t][s0 + u] = pu;
            zq += pu;
        }
#pragma unroll
        for (int m = 1; m < LP; m <<= 1) zq += __shfl_xor(zq, m);
        if (lane % LP == 0) sden[t] = zq + a.eps;
    }
    __syncthreads();
    float num[RPG][4] = {};
#pragma unroll 8
    for (int i = 0; i < DK; ++i) {
        const float4 s4 = *reinterpret_cast<const float4*>(&sS[i][x0]);
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr) {
            const float qv = sqT[i][r0 + rr];
            num[rr][0] += qv * s4.x;
            num[rr][1] += qv * s4.y;
            num[rr][2] += qv * s4.z;
            num[rr][3] += qv * s4.w;
        }
    }
#pragma unroll 4
    for (int s2 = 0; s2 < C; ++s2) {   // sP is zero above the diagonal, sv past the end
        const float4 v4 = *reinterpret_cast<const float4*>(&sv[s2][x0]);
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr) {
            const float pv = sP[r0 + rr][s2];
            num[rr][0] += pv * v4.x;
            num[rr][1] += pv * v4.y;
            num[rr][2] += pv * v4.z;
            num[rr][3] += pv * v4.w;
        }
    }
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
        const int t = r0 + rr;
        const float den = sden[t];
        float w = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) w += dr[rr][u] * num[rr][u];
        if (t < n)
            *reinterpret_cast<float4*>(a.dnum + (tok + t) * DV + x0) =
                make_float4(dr[rr][0] / den, dr[rr][1] / den, dr[rr][2] / den, dr[rr][3] / den);
        // w_t: over the row group's CG consecutive lanes, then over the waves
#pragma unroll
        for (int m = 1; m < CG; m <<= 1) w += __shfl_xor(w, m);
        if (cg == 0) sw[wv][t] = w;
    }
    __syncthreads();
    if (lane < n) {
        float w = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) w += sw[v][lane];
        const float den = sden[lane];
        a.dden[tok + lane] = -w / (den * den);
    }
}

// ---------------------------------------------------------------------------- grads
// One workgroup per (sequence, chunk): P once over all key dims, then every value tile in
// turn (A = (dO V^T) o M, dV, and the tile's shares of dQ, dK and the gate gradient, summed
// over the tiles in registers and LDS), then the final dq, dk (through phi' for KATH) and
// dg. Four waves per SIMD where the LDS allows it (GLA's per-key-dim gate tables allow two).
template <int VAR, int DK, int DV>
__global__ __launch_bounds__(NT, VAR == LA_KATH ? 3 : 2) void bwd_grads_kernel(BwdArgs a) {
    constexpr bool SG = scalar_gate<VAR>();
    constexpr bool KA = VAR == LA_KATH;
    constexpr int SW = state_width<VAR, DV>();
    // dQ / dK: work item (row pair rp, key block ib) = rows 2 rp, 2 rp + 1 and key dims
    // 4 ib .. 4 ib + 3; 8 row pairs x DK / 4 key blocks, at most one item per thread
    constexpr int NB = DK / 4, NI = (C / 2) * NB;
    static_assert(NI <= NT && C == 16, "one dQ / dK item per thread");
    constexpr int MQ = 8;   // outputs per item
    __shared__ ChunkSmem<DK, SG> sm;
    // rows padded to VT + 1 floats: the dQ / dK step reads a column down consecutive rows
    __shared__ float sdS[DK][VT + 1];    // gradient of the state leaving the chunk
    __shared__ float sSin[DK][VT + 1];   // state entering it
    __shared__ float sP[C][C + 1], sA[C][C + 1];
    __shared__ float sdg[KA ? 1 : C][KA ? 1 : DK];   // gate gradient, summed over the tiles
    const int tid = threadIdx.x;
    const int ch = int(blockIdx.x % unsigned(a.nchunks));
    const size_t seq = blockIdx.x / unsigned(a.nchunks);
    const int t0 = ch * C, n = min(C, a.N - t0);
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    const size_t tok0 = seq * size_t(a.N);
    const size_t sbase = (seq * a.nchunks + ch) * size_t(DK) * SW;
    auto load_states = [&](int c0) {
        for (int idx = tid; idx < DK * VT; idx += NT) {
            const int i = idx / VT, c = idx % VT;
            sSin[i][c] = a.Sst[sbase + size_t(i) * SW + c0 + c];
            sdS[i][c] = a.dSt[sbase + size_t(i) * SW + c0 + c];
        }
    };
    load_states(0);
    load_chunk<VAR, DK, DV, SG>(sm, a, tok0, t0, n, 0);   // rows and tile 0; ends with a barrier
    auto EQ = [&](int r, int i) { return SG ? sm.seq[r] : sm.eq[r][i]; };
    auto EK = [&](int r, int i) { return SG ? sm.sek[r] : sm.ek[r][i]; };
    // exp(B_r - B_s) for s <= r
    auto PF = [&](int r, int s, int i) {
        return SG ? sm.pd[r][s] : __builtin_amdgcn_exp2f(sm.lg[r][i] - sm.lg[s][i]);
    };
    auto gate = [&](int r, int i) { return SG ? sm.sgt[r] : sm.gt[r][i]; };

    {   // P over all key dims, lower triangle
        const int r = tid / C, s = tid % C;
        float p = 0.f;
        if (s <= r) {
            if (SG) {
                for (int i = 0; i < DK; ++i) p += sm.q[r][i] * sm.k[s][i];
                p *= sm.pd[r][s];
            } else {
                for (int i = 0; i < DK; ++i)
                    p += sm.q[r][i] * sm.k[s][i] * __builtin_amdgcn_exp2f(sm.lg[r][i] - sm.lg[s][i]);
            }
        }
        sP[r][s] = p;
    }
    if constexpr (!KA)
        for (int idx = tid; idx < C * DK; idx += NT) sdg[idx / DK][idx % DK] = 0.f;
    float dq[MQ], dk[MQ];
#pragma unroll
    for (int m = 0; m < MQ; ++m) dq[m] = dk[m] = 0.f;

    // the next tile's state columns, v and dO are fetched into registers while this one works
    constexpr int MSG = DK * VT / NT;
    static_assert(MSG * NT == DK * VT, "state tile per thread");
    float ps[MSG], pds[MSG];
    float2 nx = make_float2(0.f, 0.f);
    auto fetch_next = [&](int c0) {
#pragma unroll
        for (int m = 0; m < MSG; ++m) {
            const int idx = tid + NT * m, i = idx / VT, c = idx % VT;
            ps[m] = a.Sst[sbase + size_t(i) * SW + c0 + c];
            pds[m] = a.dSt[sbase + size_t(i) * SW + c0 + c];
        }
        nx = fetch_tile<VAR, DV>(a, tok0, t0, n, c0);
    };
    if (a.ntiles > 1) fetch_next(VT);
    for (int tile = 0; tile < a.ntiles; ++tile) {
        const int c0 = tile * VT;
        if (tile > 0) {
            __syncthreads();   // the previous tile's readers are done
#pragma unroll
            for (int m = 0; m < MSG; ++m) {
                const int idx = tid + NT * m, i = idx / VT, c = idx % VT;
                sSin[i][c] = ps[m];
                sdS[i][c] = pds[m];
            }
            stash_tile(sm, nx, n);
            if (tile + 1 < a.ntiles) fetch_next(c0 + VT);
        }
        __syncthreads();
        {   // A = (dO V^T) o M over this tile's value columns
            const int r = tid / C, s = tid % C;
            float av = 0.f;
            if (s <= r)
                for (int c = 0; c < VT; ++c) av += sm.dO[r][c] * sm.v[s][c];
            sA[r][s] = av;
        }
        __syncthreads();
        {   // dV (final for this tile's columns)
            const int s = tid / VT, c = tid % VT;
            float acc = 0.f;
            for (int r = s; r < C; ++r) acc += sP[r][s] * sm.dO[r][c];
            for (int i = 0; i < DK; ++i) acc += sm.k[s][i] * EK(s, i) * sdS[i][c];
            if (s < n && c0 < DV) store_elem(a.dv, (tok0 + t0 + s) * DV + c0 + c, acc, iob);
        }
        // this tile's share of dQ and dK, 2 rows x 4 key dims per thread:
        //   dq_ri += e^{B_ri} (dO_r . S_in[i, :]) + sum_{s<=r} A_rs e^{B_ri - B_si} k_si
        //   dk_ri += e^{B_last,i - B_ri} (v_r . dS_out[i, :]) + sum_{t>=r} A_tr e^{B_ti - B_ri} q_ti
        // (A and the pair factors are zero above the diagonal)
        if (tid < NI) {
            const int r0 = 2 * (tid / NB), i0 = 4 * (tid % NB);
            float sd[2][4] = {}, kv[2][4] = {};
            for (int c = 0; c < VT; ++c) {
                const float o0 = sm.dO[r0][c], o1 = sm.dO[r0 + 1][c];
                const float v0 = sm.v[r0][c], v1 = sm.v[r0 + 1][c];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float si = sSin[i0 + u][c], di = sdS[i0 + u][c];
                    sd[0][u] += o0 * si;
                    sd[1][u] += o1 * si;
                    kv[0][u] += v0 * di;
                    kv[1][u] += v1 * di;
                }
            }
            float qa[2][4], ka[2][4];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    qa[rr][u] = EQ(r0 + rr, i0 + u) * sd[rr][u];
                    ka[rr][u] = EK(r0 + rr, i0 + u) * kv[rr][u];
                }
#pragma unroll 2
            for (int s2 = 0; s2 < C; ++s2) {
                const float a0 = sA[r0][s2], a1 = sA[r0 + 1][s2];      // q side: rows >= s2
                const float b0 = sA[s2][r0], b1 = sA[s2][r0 + 1];      // k side: rows <= s2
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + u;
                    const float kk = sm.k[s2][i], qq = sm.q[s2][i];
                    if (SG) {
                        qa[0][u] += a0 * sm.pd[r0][s2] * kk;
                        qa[1][u] += a1 * sm.pd[r0 + 1][s2] * kk;
                        ka[0][u] += b0 * sm.pd[s2][r0] * qq;
                        ka[1][u] += b1 * sm.pd[s2][r0 + 1] * qq;
                    } else {
                        const float ls = sm.lg[s2][i];
                        const float l0 = sm.lg[r0][i], l1 = sm.lg[r0 + 1][i];
                        if (s2 <= r0) qa[0][u] += a0 * kk * __builtin_amdgcn_exp2f(l0 - ls);
                        if (s2 <= r0 + 1) qa[1][u] += a1 * kk * __builtin_amdgcn_exp2f(l1 - ls);
                        if (s2 >= r0) ka[0][u] += b0 * qq * __builtin_amdgcn_exp2f(ls - l0);
                        if (s2 >= r0 + 1) ka[1][u] += b1 * qq * __builtin_amdgcn_exp2f(ls - l1);
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    dq[rr * 4 + u] += qa[rr][u];
                    dk[rr * 4 + u] += ka[rr][u];
                }
        }
        // this tile's share of dg: thread (row group rg, column c) owns elements (rg + 16 m,
        // c); for each it rebuilds S_{s-1} forward and dS_s backward over the chunk, and the
        // products are summed over the 16 column lanes (consecutive lanes) with DPP
        if constexpr (!KA) {
            const int c = tid % VT, rg = tid / VT;
#pragma unroll 1
            for (int m = 0; m < DK / 16; ++m) {
                const int i = rg + 16 * m;
                float sp[C];   // S_{s-1}[i][c]
                float st = sSin[i][c];
#pragma unroll
                for (int s_ = 0; s_ < C; ++s_) {
                    sp[s_] = st;
                    st = gate(s_, i) * st + sm.k[s_][i] * sm.v[s_][c];
                }
                float dsv = sdS[i][c];   // dS_s[i][c], from the chunk's end backward
                float pr[C];
#pragma unroll
                for (int s_ = C - 1; s_ >= 0; --s_) {
                    if (s_ < C - 1) dsv *= gate(s_ + 1, i);
                    dsv += sm.q[s_][i] * sm.dO[s_][c];
                    pr[s_] = dsv * sp[s_];
                }
#pragma unroll
                for (int s_ = 0; s_ < C; ++s_) {
                    float v_ = pr[s_];
                    v_ += dpp_f<0xB1, 0xf, 0xf>(v_);
                    v_ += dpp_f<0x4E, 0xf, 0xf>(v_);
                    v_ += dpp_f<0x141, 0xf, 0xf>(v_);
                    v_ += dpp_f<0x140, 0xf, 0xf>(v_);
                    pr[s_] = v_;
                }
                if (c == 0) {   // one thread per (s, i): no other writer
#pragma unroll
                    for (int s_ = 0; s_ < C; ++s_) sdg[s_][i] += pr[s_];
                }
            }
        }
    }
    // final dq, dk (KATH: through phi'(x) = min(phi(x), 1), phi of the inputs in LDS)
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
        const int r = 2 * (tid / NB) + m / 4, i = 4 * (tid % NB) + m % 4;
        if (tid >= NI || r >= n) continue;
        float q_ = dq[m], k_ = dk[m];
        if (KA) {
            q_ *= fminf(sm.q[r][i], 1.f);
            k_ *= fminf(sm.k[r][i], 1.f);
        }
        const size_t e = (tok0 + t0 + r) * DK + i;
        store_elem(a.dq, e, q_, iob);
        store_elem(a.dk, e, k_, iob);
    }
    if constexpr (!KA) {
        __syncthreads();   // sdg complete
        if constexpr (!SG) {
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, i = idx % DK;
                if (r < n) store_elem(a.dg, (tok0 + t0 + r) * DK + i, sdg[r][i], gb);
            }
        } else {   // one decay per token: the sum over the key dims, thread (row, part)
            const int r = tid / 16, pt = tid % 16;
            float acc = 0.f;
            for (int i = pt; i < DK; i += 16) acc += sdg[r][i];
            acc = row16_sum(acc);
            if (pt == 0 && r < n) store_elem(a.dg, tok0 + t0 + r, acc, gb);
        }
    }
}

struct BwdLayout {
    size_t Sst, dSt, ac;
    size_t dnum, dden;   // KATH only
    size_t total;
};
BwdLayout bwd_layout(const Problem& p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const bool ka = p.variant == LA_KATH;
    const size_t sw = size_t(p.dv) + (ka ? VT : 0);
    const size_t nseq = size_t(p.B) * p.H;
    const size_t nchunks = size_t((p.N + C - 1) / C), ntok = nseq * size_t(p.N);
    BwdLayout L{};
    size_t off = 0;
    L.Sst = off; off += al(nseq * nchunks * p.dk * sw * 4);
    L.dSt = off; off += al(nseq * nchunks * p.dk * sw * 4);
    L.ac = off; off += al(nseq * nchunks * (scalar_gate_rt(p.variant) ? 1 : p.dk) * 4);
    if (ka) {
        L.dnum = off; off += al(ntok * p.dv * 4);
        L.dden = off; off += al(ntok * 4);
    }
    L.total = off;
    return L;
}

template <int VAR, int DK, int DV>
hipError_t launch_dims(const Problem& p, BwdArgs a) {
    constexpr int SW = state_width<VAR, DV>();
    hipError_t e;
    const unsigned chunks = unsigned(size_t(a.nseq) * a.nchunks);   // sums: one per chunk
    const size_t nel = size_t(a.nseq) * DK * SW;
    const dim3 scan_grid(unsigned((nel + NT - 1) / NT));
    if constexpr (VAR == LA_KATH) {
        // the state half, then dnum and dden from the forward's num and den, then the rest
        a.mode = 1;
        bwd_sums_kernel<VAR, DK, DV><<<dim3(chunks), dim3(NT), 0, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        bwd_scans_kernel<VAR, DK, DV><<<scan_grid, dim3(NT), 0, p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        kath_out_kernel<DK, DV><<<dim3(unsigned(size_t(a.nseq) * a.nchunks)),
                                  dim3(kath_out_threads(DV)), 0,
                                  p.stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        a.mode = 2;
    } else {
        a.mode = 3;
    }
    bwd_sums_kernel<VAR, DK, DV><<<dim3(chunks), dim3(NT), 0, p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_scans_kernel<VAR, DK, DV><<<scan_grid, dim3(NT), 0, p.stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_grads_kernel<VAR, DK, DV><<<dim3(chunks), dim3(NT), 0, p.stream>>>(a);
    return hipGetLastError();
}

template <int VAR, int DK>
hipError_t dispatch_dv(const Problem& p, const BwdArgs& a) {
    switch (p.dv) {
        case 16: return launch_dims<VAR, DK, 16>(p, a);
        case 32: return launch_dims<VAR, DK, 32>(p, a);
        case 64: return launch_dims<VAR, DK, 64>(p, a);
        case 128: return launch_dims<VAR, DK, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

template <int VAR>
hipError_t dispatch_dk(const Problem& p, const BwdArgs& a) {
    switch (p.dk) {
        case 16: return dispatch_dv<VAR, 16>(p, a);
        case 32: return dispatch_dv<VAR, 32>(p, a);
        case 64: return dispatch_dv<VAR, 64>(p, a);
        case 128: return dispatch_dv<VAR, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

// N = 0: the gradients of the initial state (and normaliser) are the final ones
__global__ void bwd_copy_kernel(const float* dSf, float* dS0, size_t n, const float* dzf,
                                float* dz0, size_t nz) {
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dS0[i] = dSf ? dSf[i] : 0.f;
    if (dz0 && i < nz) dz0[i] = dzf ? dzf[i] : 0.f;
}

}  // namespace

bool backward_supported(int variant) {
    return variant == LA_GLA || variant == LA_SSD || variant == LA_GDN || variant == LA_KDA ||
           variant == LA_KATH;
}

size_t backward_workspace_bytes(const Problem& p) {
    if (p.N == 0 || p.B == 0 || p.H == 0) return 0;
    if (p.variant == LA_GDN || p.variant == LA_KDA) return gdn_backward_workspace_bytes(p);
    return bwd_layout(p).total;
}

hipError_t launch_backward(const BwdProblem& bp) {
    const Problem& p = bp.p;
    if (p.N == 0) {
        const size_t n = size_t(p.B) * p.H * p.dk * p.dv;
        const size_t nz = p.variant == LA_KATH ? size_t(p.B) * p.H * p.dk : 0;
        const size_t blocks = (n + 255) / 256;
        if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
        bwd_copy_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, p.stream>>>(
            bp.dS_final, bp.dS0, n, bp.dz_final, p.variant == LA_KATH ? bp.dz0 : nullptr, nz);
        return hipGetLastError();
    }
    if (p.variant == LA_GDN || p.variant == LA_KDA) return launch_backward_gdn(bp);
    const bool ka = p.variant == LA_KATH;
    const size_t nseq = size_t(p.B) * p.H;
    const size_t nchunks = size_t((p.N + C - 1) / C);
    const size_t sw = size_t(p.dv) + (ka ? VT : 0);
    if (nseq * nchunks * (sw / VT) > 0x7fffffffull || nseq * size_t(p.dk) * sw / NT > 0x7fffffffull ||
        nseq * size_t(p.N) * p.dk / NT > 0x7fffffffull)
        return hipErrorInvalidValue;
    const BwdLayout L = bwd_layout(p);
    unsigned char* ws = static_cast<unsigned char*>(p.ws);
    BwdArgs a{};
    a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.dO = bp.dO;
    a.S0 = p.S0; a.dSf = bp.dS_final;
    a.dq = bp.dq; a.dk = bp.dk; a.dv = bp.dv; a.dg = bp.dg; a.dS0 = bp.dS0;
    a.Sst = reinterpret_cast<float*>(ws + L.Sst);
    a.dSt = reinterpret_cast<float*>(ws + L.dSt);
    a.ac = reinterpret_cast<float*>(ws + L.ac);
    if (ka) {
        a.dnum = reinterpret_cast<float*>(ws + L.dnum);
        a.dden = reinterpret_cast<float*>(ws + L.dden);
        a.z0 = p.z0;
        a.dzf = bp.dz_final;
        a.dz0 = bp.dz0;
        a.eps = p.eps;
    }
    a.N = p.N;
    a.nseq = int(nseq);
    a.ntiles = int(sw / VT);
    a.nchunks = (p.N + C - 1) / C;
    a.io_bf16 = p.io_bf16;
    a.gate_bf16 = p.gate_bf16;
    switch (p.variant) {
        case LA_GLA: return dispatch_dk<LA_GLA>(p, a);
        case LA_SSD: return dispatch_dk<LA_SSD>(p, a);
        case LA_KATH: return dispatch_dk<LA_KATH>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
