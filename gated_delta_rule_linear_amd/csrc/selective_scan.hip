// Selective scan (Mamba-1 / S6): "Linear / RNN 路线" section 3.5 (the boxed
// discretisation Abar_t = exp(Delta_t A), Bbar_t = Delta_t B_t, with Delta, B, C taken
// from the input) and the forward of the simplified block in section 3.6;
// "状态空间与线性注意力", sections Selective SSM and 卷积与递推的等价 (the D x skip).
// For every batch row and channel d, a state h_d in R^n:
//   Delta_t = softplus(dt_t + bias_d)           (or dt_t + bias_d)
//   h_{d,i} <- exp(Delta_t A_{d,i}) h_{d,i} + Delta_t B_{t,i} x_{t,d}
//   y_{t,d}  = sum_i C_{t,i} h_{d,i} + D_d x_{t,d}
//
// Every (channel, state entry) pair has its own decay, so nothing here is a dense
// contraction: each state entry costs one exponential and four fp32 operations per token,
// and the kernel is bound by the vector ALUs (the exponential above all), not by HBM
// (per token and channel it moves a few bytes against n exponentials).
//
// Layout of the work: LPC = n / NS lanes own one channel, lane j its NS consecutive
// state entries; a workgroup of 4 waves holds 256 / LPC channels of one batch row. Per
// chunk of 32 tokens the workgroup stages B and C (shared by all channels) in LDS as
// fp32, and Delta (computed once per token and channel), Delta x and x; the lanes then
// run the recurrence over the chunk from LDS and sum C . h over groups of 16 (or 8)
// lanes with DPP steps; a channel spread over two groups leaves two partial sums, added
// when the chunk's outputs are written back together. The next chunk's loads are in
// flight while a chunk is processed. Padding tokens past the end are identity steps
// (Delta = 0). Channel blocks that share HBM lines go to one XCD.
#include "common.hpp"
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int NT = 256;     // threads per workgroup
constexpr int TC = 32;      // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

struct ScanArgs {
    const void *dt, *Bm, *Cm, *x;
    const float *A, *Dskip, *bias, *h0;
    void* y;
    float* hT;
    int Bt, T, D, nblk, softplus;
};

template <int N, int CH, int RPC>
struct __align__(16) ScanSmem {
    __align__(16) float b[2][TC * N];       // B_t (fp32)
    __align__(16) float c[2][TC * N];       // C_t
    __align__(16) float2 dd[2][TC * CH];    // (Delta, Delta x) per token and channel
    __align__(16) float xs[2][TC * CH];     // x, for the skip
    __align__(16) float ys[RPC][TC * CH];   // partial C . h per token and channel
};

// softplus(u) = max(u, 0) + log(1 + exp(-|u|)), with the hardware base-2 exponential
// and logarithm; the argument of the logarithm lies in (1, 2]
__device__ __forceinline__ float softplus_f(float u) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(u) * 1.4426950408889634f);
    return fmaxf(u, 0.f) + __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f;
}

// workgroup id -> unit (row * nblk + channel block); four consecutive channel blocks
// (64 channels: one 128-byte line of a bf16 row) share an XCD, so the lines of x, dt
// and y are fetched and written once per XCD
__device__ __forceinline__ int scan_unit(int bid) {
    const int xcd = bid & 7, slot = bid >> 3;
    return ((slot >> 2) * 8 + xcd) * 4 + (slot & 3);
}

template <int N, int NS, bool IOB>
__global__ __launch_bounds__(NT) void selective_scan_kernel(ScanArgs a) {
    constexpr int LPC = N / NS;                      // lanes per channel
    constexpr int G = LPC < 16 ? LPC : 16;           // lanes per reduction group
    constexpr int RPC = LPC / G;                     // partial sums per channel
    constexpr int CH = NT / LPC;                     // channels per workgroup
    static_assert((G == 8 || G == 16) && RPC * G == LPC && CH * LPC == NT, "scan tiling");
    static_assert((TC * CH) % NT == 0 && TC % G == 0, "every thread stages whole tokens");
    constexpr int ISZ = IOB ? 2 : 4;
    constexpr int EPP = 16 / ISZ;                    // elements per 16-byte piece
    constexpr int BPIECES = TC * N / EPP;            // pieces of B (or C) per chunk
    constexpr int BPT = (BPIECES + NT - 1) / NT;     // per thread
    constexpr int EPT = TC * CH / NT;                // dt / x elements per thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScanSmem<N, CH, RPC>& sm = *reinterpret_cast<ScanSmem<N, CH, RPC>*>(smem_raw);

    const int unit = scan_unit(blockIdx.x);
    if (unit >= a.Bt * a.nblk) return;
    const int row = unit / a.nblk, d0 = (unit % a.nblk) * CH;
    const int tid = threadIdx.x;
    const int cl = tid / LPC, j = tid % LPC;   // channel in the block, state slice
    const int r = j / G, jj = j % G;           // partial sum, lane in the group
    const int d = d0 + cl;
    const bool live = d < a.D;
    const int T = a.T;

    const size_t rowtok = size_t(row) * size_t(T);
    const rsrc_t rdt = make_rsrc(static_cast<const char*>(a.dt) + rowtok * a.D * ISZ,
                                 uint32_t(size_t(T) * a.D * ISZ));
    const rsrc_t rx = make_rsrc(static_cast<const char*>(a.x) + rowtok * a.D * ISZ,
                                uint32_t(size_t(T) * a.D * ISZ));
    const rsrc_t rB = make_rsrc(static_cast<const char*>(a.Bm) + rowtok * N * ISZ,
                                uint32_t(size_t(T) * N * ISZ));
    const rsrc_t rC = make_rsrc(static_cast<const char*>(a.Cm) + rowtok * N * ISZ,
                                uint32_t(size_t(T) * N * ISZ));

    // this lane's state entries and decay rates (A log2 e, so exp(Delta A) = exp2(Delta A2))
    float h[NS], A2[NS];
    {
        const size_t sb = (size_t(row) * a.D + d) * N + size_t(j) * NS;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            h[s] = (live && a.h0) ? a.h0[sb + s] : 0.f;
            A2[s] = live ? a.A[size_t(d) * N + size_t(j) * NS + s] * kLog2e : 0.f;
        }
    }
    // the staging and output phases handle channel d0 + tid % CH of each token (the
    // element index tid + 256 u keeps its residue): its bias and skip, loaded once
    const int cst = tid % CH;
    const bool live_st = d0 + cst < a.D;
    const float bias_st = (live_st && a.bias) ? a.bias[d0 + cst] : 0.f;
    const float skip_st = (live_st && a.Dskip) ? a.Dskip[d0 + cst] : 0.f;
    // consume these loads here: a first use inside the chunk loop would make every chunk
    // wait for all loads in flight, the next chunk's prefetch included
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(h[s]), "+v"(A2[s]));
    {
        float b_ = bias_st, s_ = skip_st;
        asm volatile("" : "+v"(b_), "+v"(s_));
    }

    // staging registers of one chunk
    struct Stage {
        uint4 b[BPT], c[BPT];
        uint32_t dt[EPT], x[EPT];
    };
    auto load_chunk = [&](Stage& st, int ch) {
        const uint32_t t0 = uint32_t(ch) * TC;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int p = tid + NT * u;
            // pieces past the chunk (small n) read beyond the resource: zeros, unused
            const uint32_t off = p < BPIECES ? (t0 * N + uint32_t(p) * EPP) * ISZ : 0xffffff00u;
            st.b[u] = buf_ld16(rB, off);
            st.c[u] = buf_ld16(rC, off);
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / CH, c = e % CH;
            const uint32_t off = d0 + c < a.D ? ((t0 + t) * uint32_t(a.D) + d0 + c) * ISZ
                                              : 0xffffff00u;
            st.dt[u] = IOB ? buf_ld2(rdt, off) : buf_ld4(rdt, off);
            st.x[u] = IOB ? buf_ld2(rx, off) : buf_ld4(rx, off);
        }
    };
    auto to_f = [](uint32_t raw) { return IOB ? __uint_as_float(raw << 16) : __uint_as_float(raw); };
    auto store_chunk = [&](const Stage& st, int ch, int buf) {
        const int t0 = ch * TC;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int p = tid + NT * u;
            if (p >= BPIECES) continue;
            float fb[EPP], fc[EPP];
            if constexpr (IOB) {
                const uint32_t wb[4] = {st.b[u].x, st.b[u].y, st.b[u].z, st.b[u].w};
                const uint32_t wc[4] = {st.c[u].x, st.c[u].y, st.c[u].z, st.c[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    fb[2 * q] = __uint_as_float(wb[q] << 16);
                    fb[2 * q + 1] = __uint_as_float(wb[q] & 0xffff0000u);
                    fc[2 * q] = __uint_as_float(wc[q] << 16);
                    fc[2 * q + 1] = __uint_as_float(wc[q] & 0xffff0000u);
                }
            } else {
                fb[0] = __uint_as_float(st.b[u].x); fb[1] = __uint_as_float(st.b[u].y);
                fb[2] = __uint_as_float(st.b[u].z); fb[3] = __uint_as_float(st.b[u].w);
                fc[0] = __uint_as_float(st.c[u].x); fc[1] = __uint_as_float(st.c[u].y);
                fc[2] = __uint_as_float(st.c[u].z); fc[3] = __uint_as_float(st.c[u].w);
            }
#pragma unroll
            for (int q = 0; q < EPP; q += 4) {
                *reinterpret_cast<float4*>(&sm.b[buf][p * EPP + q]) =
                    make_float4(fb[q], fb[q + 1], fb[q + 2], fb[q + 3]);
                *reinterpret_cast<float4*>(&sm.c[buf][p * EPP + q]) =
                    make_float4(fc[q], fc[q + 1], fc[q + 2], fc[q + 3]);
            }
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / CH, c = e % CH;
            float delta = 0.f, xv = 0.f;
            if (t0 + t < T && live_st) {   // padding tokens: Delta = 0, an identity step
                xv = to_f(st.x[u]);
                delta = to_f(st.dt[u]) + bias_st;
                if (a.softplus) delta = softplus_f(delta);
            }
            sm.dd[buf][e] = make_float2(delta, delta * xv);
            sm.xs[buf][e] = xv;
        }
    };

    const int nch = (T + TC - 1) / TC;
    const rsrc_t ry = make_rsrc(static_cast<char*>(a.y) + rowtok * a.D * ISZ,
                                uint32_t(size_t(T) * a.D * ISZ));
    // one chunk from LDS buffer buf: the recurrence, then its outputs y = C . h + D x
    auto process = [&](int ch, int buf) {
        const float* bb = sm.b[buf] + j * NS;
        const float* cc = sm.c[buf] + j * NS;
        // one token's operands from LDS: (Delta, Delta x) and this lane's B and C entries
        struct Ops {
            float2 dd;
            float b[NS], c[NS];
        };
        auto read_ops = [&](Ops& o, int t) {
            o.dd = sm.dd[buf][t * CH + cl];
            if constexpr (NS >= 4) {
#pragma unroll
                for (int s = 0; s < NS; s += 4) {
                    const float4 b4 = *reinterpret_cast<const float4*>(bb + t * N + s);
                    const float4 c4 = *reinterpret_cast<const float4*>(cc + t * N + s);
                    o.b[s] = b4.x; o.b[s + 1] = b4.y; o.b[s + 2] = b4.z; o.b[s + 3] = b4.w;
                    o.c[s] = c4.x; o.c[s + 1] = c4.y; o.c[s + 2] = c4.z; o.c[s + 3] = c4.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    o.b[s] = bb[t * N + s];
                    o.c[s] = cc[t * N + s];
                }
            }
        };
        // the token step: this lane's state entries, and its part of C . h
        auto step = [&](const Ops& o) {
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float ab = __builtin_amdgcn_exp2f(o.dd.x * A2[s]);
                h[s] = fmaf(ab, h[s], o.dd.y * o.b[s]);
                if (s & 1) acc1 = fmaf(o.c[s], h[s], acc1);
                else acc0 = fmaf(o.c[s], h[s], acc0);
            }
            return acc0 + acc1;
        };
        // Tokens go in blocks of TB: the next block's operands are read while this block's
        // group sums (independent DPP chains, interleaved) complete.
        constexpr int TB = NS == 1 ? 16 : NS == 2 ? 8 : 4;   // tokens per block (fewer registers per token at small NS)
        static_assert(TC % TB == 0 && G % TB == 0, "whole token blocks per group");
        float yk = 0.f;   // lane jj keeps the sum of token G m + jj
        Ops o[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) read_ops(o[b], b);
#pragma unroll 2
        for (int t = 0; t < TC; t += TB) {
            float v[TB];
#pragma unroll
            for (int b = 0; b < TB; ++b) v[b] = step(o[b]);
            if (t + TB < TC) {
#pragma unroll
                for (int b = 0; b < TB; ++b) read_ops(o[b], t + TB + b);
            }
#pragma unroll
            for (int b = 0; b < TB; ++b) v[b] += dpp_f<0xB1, 0xf, 0xf>(v[b]);   // quad_perm [1,0,3,2]
#pragma unroll
            for (int b = 0; b < TB; ++b) v[b] += dpp_f<0x4E, 0xf, 0xf>(v[b]);   // quad_perm [2,3,0,1]
#pragma unroll
            for (int b = 0; b < TB; ++b) v[b] += dpp_f<0x141, 0xf, 0xf>(v[b]);  // row_half_mirror
            if constexpr (G == 16) {
#pragma unroll
                for (int b = 0; b < TB; ++b) v[b] += dpp_f<0x140, 0xf, 0xf>(v[b]);   // row_mirror
            }
#pragma unroll
            for (int b = 0; b < TB; ++b) yk = ((t + b) % G) == jj ? v[b] : yk;
            if ((t + TB - 1) % G == G - 1) sm.ys[r][(t + TB - G + jj) * CH + cl] = yk;
        }
        lds_barrier();   // ys complete
        const int t0 = ch * TC;
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / CH, c = e % CH;
            const bool ok = t0 + t < T && live_st;
            float yv = skip_st * sm.xs[buf][e];
#pragma unroll
            for (int q = 0; q < RPC; ++q) yv += sm.ys[q][e];
            const uint32_t off = ok ? (uint32_t(t0 + t) * uint32_t(a.D) + d0 + c) * ISZ : 0xffffff00u;
            if constexpr (IOB)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(yv), ry, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, off, 0, 0);
        }
    };

    // two register sets alternate: chunk ch + 1 is staged into LDS while chunk ch + 2 loads
    Stage SA, SB;
    if (nch > 0) {
        load_chunk(SA, 0);
        store_chunk(SA, 0, 0);
        if (nch > 1) load_chunk(SB, 1);
    }
    lds_barrier();
    for (int ch = 0; ch < nch; ch += 2) {
        process(ch, 0);
        if (ch + 1 < nch) {
            store_chunk(SB, ch + 1, 1);
            if (ch + 2 < nch) load_chunk(SA, ch + 2);
        }
        lds_barrier();   // buffer 1 staged; every read of ys and buffer 0 done
        if (ch + 1 >= nch) break;
        process(ch + 1, 1);
        if (ch + 2 < nch) {
            store_chunk(SA, ch + 2, 0);
            if (ch + 3 < nch) load_chunk(SB, ch + 3);
        }
        lds_barrier();
    }
    if (live) {
        const size_t sb = (size_t(row) * a.D + d) * N + size_t(j) * NS;
#pragma unroll
        for (int s = 0; s < NS; ++s) a.hT[sb + s] = h[s];
    }
}

// State entries per lane for each state size: NS = n / 16 puts one channel on 16 lanes;
// a smaller NS spreads a channel over more lanes (more waves, less work per lane).
constexpr int scan_ns(int n) { return n == 128 ? 4 : n == 64 ? 4 : n == 32 ? 2 : 1; }

template <int N>
hipError_t launch_n(const ScanProblem& p, ScanArgs a) {
    constexpr int NS = scan_ns(N), LPC = N / NS, G = LPC < 16 ? LPC : 16;
    constexpr int CH = NT / LPC;
    const size_t smem = sizeof(ScanSmem<N, CH, LPC / G>);
    a.nblk = (p.D + CH - 1) / CH;
    const size_t units = size_t(a.Bt) * size_t(a.nblk);
    const size_t grid = (units + 31) / 32 * 32;
    if (grid > 0x7fffffffull) return hipErrorInvalidValue;
    hipError_t e;
    if (p.io_bf16) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&selective_scan_kernel<N, NS, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        selective_scan_kernel<N, NS, true><<<dim3(unsigned(grid)), dim3(NT), smem, p.stream>>>(a);
    } else {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&selective_scan_kernel<N, NS, false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
        selective_scan_kernel<N, NS, false><<<dim3(unsigned(grid)), dim3(NT), smem, p.stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

bool selective_scan_supported(int n) { return n == 16 || n == 32 || n == 64 || n == 128; }

hipError_t launch_selective_scan(const ScanProblem& p) {
    // 32-bit buffer offsets: one batch row of dt / x / y and of B / C
    const size_t isz = p.io_bf16 ? 2 : 4;
    if (size_t(p.T) * size_t(p.D) * isz >= (size_t(1) << 31) - 256 ||
        size_t(p.T + TC) * size_t(p.n) * isz >= (size_t(1) << 31) - 256)
        return hipErrorInvalidValue;
    ScanArgs a{p.dt, p.Bm, p.Cm, p.x, p.A, p.Dskip, p.dt_bias, p.h0, p.y, p.hT,
               p.Bt, p.T, p.D, 0, p.dt_softplus};
    switch (p.n) {
        case 16: return launch_n<16>(p, a);
        case 32: return launch_n<32>(p, a);
        case 64: return launch_n<64>(p, a);
        case 128: return launch_n<128>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
