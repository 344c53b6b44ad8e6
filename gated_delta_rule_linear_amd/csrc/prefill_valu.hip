// Chunked prefill in fp32 on the vector ALUs (chunk C = 16, 16-column value tiles).
//
// This is the precise path (fp32 inputs, any supported d_k / d_v) and the
// fallback for shapes the matrix-core kernels do not take. It uses the same
// chunkwise method as the MFMA kernels but keeps every intermediate in fp32 and
// evaluates the in-chunk decay exactly, per element, in the log domain, so it is
// safe for any gate values.
//
// One workgroup owns one (b, h, value tile): columns of S never mix in any of the
// three recurrences, so value tiles are independent chains. The state tile lives
// in LDS for the whole sequence. Per chunk of tokens t0 .. t0+C-1 (local r, s):
//
//  KATH  P_rs = phi(q_r).phi(k_s) (s <= r)
//        o_r  = (phi(q_r)^T S + sum_s P_rs v_s) / (phi(q_r).z + sum_s P_rs + eps)
//        S   += sum_s phi(k_s) v_s^T,  z += sum_s phi(k_s)
//  GLA   B_r  = sum_{s<=r} log g_s (per key dim, from the chunk start)
//        P_rs = sum_i q_ri k_si exp(B_ri - B_si) (s <= r)
//        o_r  = (q_r * exp(B_r))^T S + sum_s P_rs v_s
//        S    = diag(exp(B_last)) S + sum_s diag(exp(B_last - B_s)) k_s v_s^T
//  GDN   c_r  = sum_{s<=r} log alpha_s, gamma_r = exp(c_r)
//        L_rs = beta_r exp(c_r - c_s) k_r.k_s (s < r)
//        (I + L) U = X,  X_r = beta_r (v_r - gamma_r S^T k_r)     [forward substitution]
//        o_r  = gamma_r S^T q_r + sum_{s<=r} exp(c_r - c_s) (q_r.k_s) u_s
//        S    = gamma_last S + sum_s exp(c_last - c_s) k_s u_s^T
//  KDA   B_r  = sum_{s<=r} log alpha_s (per key dim), the delta rule of GDN with the
//        decay inside the products:
//        L_rs = beta_r sum_i k_ri k_si exp(B_ri - B_si) (s < r)
//        (I + L) U = X,  X_r = beta_r (v_r - S^T (k_r * exp(B_r)))
//        o_r  = S^T (q_r * exp(B_r)) + sum_{s<=r} P_rs u_s,  P as for GLA
//        S    = diag(exp(B_last)) S + sum_s diag(exp(B_last - B_s)) k_s u_s^T
//  SSD   c_r  = sum_{s<=r} log a_s (one decay per token), GLA with that decay on every
//        key dim: P_rs = exp(c_r - c_s) q_r.k_s, o_r = exp(c_r) S^T q_r + sum_s P_rs v_s,
//        S    = exp(c_last) S + sum_s exp(c_last - c_s) k_s v_s^T
// These are exact rewrites of the token recurrences (the state after token r of
// the chunk, unrolled back to the chunk start). Padding tokens past N are
// identity steps: zero key and value, gate 1, beta 0.
#include "common.hpp"
#include "la_internal.h"
#include "mfma.hpp"

namespace la {
namespace {

constexpr int C = kValuChunk;  // 16
constexpr int VT = 16;         // value columns per workgroup
constexpr int NT = 256;        // threads per workgroup (= C * VT)

struct ValuArgs {
    const void *q, *k, *v, *g, *beta;
    const float *S0, *z0;
    void* o;
    float *S, *z;
    int N, ntiles;
    float eps;
    int io_bf16, gate_bf16;
    const int32_t* cu;   // packed variable-length batch, or null
    int H, L;
};

template <int VAR, int DK, int DV>
__global__ __launch_bounds__(NT) void prefill_valu_kernel(ValuArgs a) {
    constexpr int DKP = DK + 1;  // padded row pitch
    constexpr bool CHG = VAR == LA_GLA || VAR == LA_KDA;   // gate per key dim
    constexpr bool DLT = VAR == LA_GDN || VAR == LA_KDA;   // delta rule
    constexpr bool SCL = VAR == LA_GDN || VAR == LA_SSD;   // one gate per token
    __shared__ float sS[DK][VT];
    __shared__ float sz[DK];
    __shared__ float sQ[C][DKP], sK[C][DKP];
    __shared__ float sLg[CHG ? C : 1][CHG ? DKP : 1];
    __shared__ float sV[C][VT];
    __shared__ float sP[C][C + 1], sL[C][C + 1];
    __shared__ float sX[C][VT], sU[C][VT];
    __shared__ float sc[C], sbeta[C], sden[C];

    const int tid = threadIdx.x;
    const size_t seq = blockIdx.x / a.ntiles;
    const int tile = blockIdx.x % a.ntiles;
    const int c0 = tile * VT;
    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    const SeqSpan sp = seq_span(int(seq), a.H, a.N, a.L, a.cu);
    const size_t tok0 = sp.base;
    const int len = sp.len;

    // initial state tile
    for (int idx = tid; idx < DK * VT; idx += NT) {
        const int i = idx / VT, c = idx % VT;
        sS[i][c] = a.S0 ? a.S0[seq * DK * DV + size_t(i) * DV + c0 + c] : 0.f;
    }
    if (VAR == LA_KATH)
        for (int i = tid; i < DK; i += NT) sz[i] = a.z0 ? a.z0[seq * DK + i] : 0.f;

    const int r_me = tid / VT, c_me = tid % VT;  // (row, column) of this thread's output
    const int nchunks = (len + C - 1) / C;

    // A chunk's inputs are fetched as raw words one chunk ahead, while the chunk before it
    // is processed, so that their latency is not paid once per chunk. The loads are
    // unconditional (per-chunk buffer resources read zeros past the sequence's end) and
    // of the storage width, chosen once for all of them.
    constexpr int NQ = C * DK / NT;   // q / k elements per thread per chunk
    static_assert(C * DK % NT == 0, "whole elements per thread");
    struct Raw {
        uint32_t q[NQ], k[NQ], g[CHG ? NQ : 1], v, gs, bs;
    };
    const uint32_t es = iob ? 2u : 4u, gsz = gb ? 2u : 4u;
    auto fetch = [&](Raw& R, int ch) {
        const int t0 = ch * C;
        const uint32_t rows = uint32_t(max(0, min(C, len - t0)));
        const size_t tk = tok0 + size_t(t0);
        const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + tk * DK * es, rows * DK * es);
        const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + tk * DK * es, rows * DK * es);
        const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + tk * DV * es, rows * DV * es);
        const rsrc_t rg = make_rsrc(a.g ? static_cast<const char*>(a.g) + tk * (CHG ? DK : 1) * gsz : nullptr,
                                    a.g ? rows * (CHG ? DK : 1) * gsz : 0u);
        const rsrc_t rb = make_rsrc(a.beta ? static_cast<const char*>(a.beta) + tk * gsz : nullptr,
                                    a.beta ? rows * gsz : 0u);
        const uint32_t ov = uint32_t(r_me * DV + c0 + c_me);
        const uint32_t ot = uint32_t(tid < C ? tid : 0);
        if (iob) {
#pragma unroll
            for (int x = 0; x < NQ; ++x) {
                const uint32_t idx = uint32_t(tid + NT * x);
                R.q[x] = buf_ld2(rq, idx * 2u);
                R.k[x] = buf_ld2(rk, idx * 2u);
            }
            R.v = buf_ld2(rv, ov * 2u);
        } else {
#pragma unroll
            for (int x = 0; x < NQ; ++x) {
                const uint32_t idx = uint32_t(tid + NT * x);
                R.q[x] = buf_ld4(rq, idx * 4u);
                R.k[x] = buf_ld4(rk, idx * 4u);
            }
            R.v = buf_ld4(rv, ov * 4u);
        }
        if (gb) {
            if (CHG) {
#pragma unroll
                for (int x = 0; x < NQ; ++x) R.g[x] = buf_ld2(rg, uint32_t(tid + NT * x) * 2u);
            }
            if (SCL) R.gs = buf_ld2(rg, ot * 2u);
            if (DLT) R.bs = buf_ld2(rb, ot * 2u);
        } else {
            if (CHG) {
#pragma unroll
                for (int x = 0; x < NQ; ++x) R.g[x] = buf_ld4(rg, uint32_t(tid + NT * x) * 4u);
            }
            if (SCL) R.gs = buf_ld4(rg, ot * 4u);
            if (DLT) R.bs = buf_ld4(rb, ot * 4u);
        }
    };
    auto word = [](uint32_t w, bool bf) { return bf ? __uint_as_float(w << 16) : __uint_as_float(w); };

    auto body = [&](const Raw& R, Raw& Rn, int ch) {
        const int t0 = ch * C;
        const int n = min(C, len - t0);
        __syncthreads();  // previous chunk's readers of sQ/sK/sV/sS are done
#pragma unroll
        for (int x = 0; x < NQ; ++x) {
            const int idx = tid + NT * x;
            const int r = idx / DK, i = idx % DK;
            float qv = 0.f, kv = 0.f, lg = 0.f;
            if (r < n) {
                qv = word(R.q[x], iob);
                kv = word(R.k[x], iob);
                if (VAR == LA_KATH) {
                    qv = elu_plus_one(qv);
                    kv = elu_plus_one(kv);
                }
                if (CHG) lg = logf(word(R.g[x], gb));
            }
            sQ[r][i] = qv;
            sK[r][i] = kv;
            if (CHG) sLg[r][i] = lg;
        }
        sV[r_me][c_me] = r_me < n ? word(R.v, iob) : 0.f;
        if ((DLT || SCL) && tid < C) {
            const int r = tid;
            if (SCL) sc[r] = r < n ? logf(word(R.gs, gb)) : 0.f;
            if (DLT) sbeta[r] = r < n ? word(R.bs, gb) : 0.f;
        }
        if (ch + 1 < nchunks) fetch(Rn, ch + 1);
        __syncthreads();
        // in-chunk cumulative log gates
        if (CHG) {
            for (int i = tid; i < DK; i += NT) {
                float acc = 0.f;
                for (int r = 0; r < C; ++r) {
                    acc += sLg[r][i];
                    sLg[r][i] = acc;
                }
            }
        }
        if (SCL && tid == 0) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += sc[r];
                sc[r] = acc;
            }
        }
        __syncthreads();
        // scores: thread -> (r, s)
        {
            const int r = tid / C, s = tid % C;
            float p = 0.f, l = 0.f;
            if (s <= r) {
                if (CHG) {
                    for (int i = 0; i < DK; ++i) p += sQ[r][i] * sK[s][i] * expf(sLg[r][i] - sLg[s][i]);
                } else {
                    for (int i = 0; i < DK; ++i) p += sQ[r][i] * sK[s][i];
                }
                if (VAR == LA_KDA && s < r) {
                    for (int i = 0; i < DK; ++i) l += sK[r][i] * sK[s][i] * expf(sLg[r][i] - sLg[s][i]);
                    l *= sbeta[r];
                }
                if (SCL) {
                    const float d = expf(sc[r] - sc[s]);
                    p *= d;
                    if (DLT && s < r) {
                        for (int i = 0; i < DK; ++i) l += sK[r][i] * sK[s][i];
                        l *= sbeta[r] * d;
                    }
                }
            }
            sP[r][s] = p;
            if (DLT) sL[r][s] = l;
        }
        if (VAR == LA_KATH && tid < C) {
            float d = 0.f;
            for (int i = 0; i < DK; ++i) d += sQ[tid][i] * sz[i];
            sden[tid] = d;
        }
        if (VAR == LA_GDN) {
            const int r = r_me, c = c_me;
            float ks = 0.f;
            for (int i = 0; i < DK; ++i) ks += sK[r][i] * sS[i][c];
            sX[r][c] = sbeta[r] * (sV[r][c] - expf(sc[r]) * ks);
        }
        if (VAR == LA_KDA) {
            const int r = r_me, c = c_me;
            float ks = 0.f;
            for (int i = 0; i < DK; ++i) ks += sK[r][i] * expf(sLg[r][i]) * sS[i][c];
            sX[r][c] = sbeta[r] * (sV[r][c] - ks);
        }
        __syncthreads();
        if (DLT) {
            // forward substitution (I + L) U = X, one thread per column
            if (tid < VT) {
                const int c = tid;
                for (int r = 0; r < C; ++r) {
                    float u = sX[r][c];
                    for (int s = 0; s < r; ++s) u -= sL[r][s] * sU[s][c];
                    sU[r][c] = u;
                }
            }
            __syncthreads();
        }
        // outputs: thread -> (r, c)
        {
            const int r = r_me, c = c_me;
            float acc = 0.f;
            if (CHG) {
                for (int i = 0; i < DK; ++i) acc += sQ[r][i] * expf(sLg[r][i]) * sS[i][c];
            } else {
                for (int i = 0; i < DK; ++i) acc += sQ[r][i] * sS[i][c];
            }
            if (SCL) acc *= expf(sc[r]);
            float intra = 0.f, psum = 0.f;
            for (int s = 0; s <= r; ++s) {
                const float p = sP[r][s];
                intra += p * (DLT ? sU[s][c] : sV[s][c]);
                psum += p;
            }
            float out = acc + intra;
            if (VAR == LA_KATH) out = out / (sden[r] + psum + a.eps);
            if (r < n) store_elem(a.o, (tok0 + t0 + r) * DV + c0 + c, out, iob);
        }
        __syncthreads();  // all reads of the old state are done
        // state update
        for (int idx = tid; idx < DK * VT; idx += NT) {
            const int i = idx / VT, c = idx % VT;
            float acc = 0.f;
            if (VAR == LA_GLA) {
                const float bl = sLg[C - 1][i];
                for (int s = 0; s < C; ++s) acc += sK[s][i] * expf(bl - sLg[s][i]) * sV[s][c];
                sS[i][c] = expf(bl) * sS[i][c] + acc;
            } else if (VAR == LA_KDA) {
                const float bl = sLg[C - 1][i];
                for (int s = 0; s < C; ++s) acc += sK[s][i] * expf(bl - sLg[s][i]) * sU[s][c];
                sS[i][c] = expf(bl) * sS[i][c] + acc;
            } else if (SCL) {
                const float cl = sc[C - 1];
                for (int s = 0; s < C; ++s)
                    acc += sK[s][i] * expf(cl - sc[s]) * (DLT ? sU[s][c] : sV[s][c]);
                sS[i][c] = expf(cl) * sS[i][c] + acc;
            } else {
                for (int s = 0; s < C; ++s) acc += sK[s][i] * sV[s][c];
                sS[i][c] += acc;
            }
        }
        if (VAR == LA_KATH) {
            for (int i = tid; i < DK; i += NT) {
                float acc = 0.f;
                for (int s = 0; s < C; ++s) acc += sK[s][i];
                sz[i] += acc;
            }
        }
    };
    // two sets of raw words, swapped by unrolling
    Raw RA, RB;
    if (nchunks > 0) fetch(RA, 0);
    for (int ch = 0; ch < nchunks; ch += 2) {
        body(RA, RB, ch);
        if (ch + 1 >= nchunks) break;
        body(RB, RA, ch + 1);
    }
    __syncthreads();
    for (int idx = tid; idx < DK * VT; idx += NT) {
        const int i = idx / VT, c = idx % VT;
        a.S[seq * DK * DV + size_t(i) * DV + c0 + c] = sS[i][c];
    }
    if (VAR == LA_KATH && tile == 0)
        for (int i = tid; i < DK; i += NT) a.z[seq * DK + i] = sz[i];
}

template <int VAR, int DK, int DV>
hipError_t launch_one(const Problem& p, ValuArgs a) {
    a.ntiles = DV / VT;
    const size_t nblocks = size_t(p.B) * size_t(p.H) * size_t(a.ntiles);
    if (nblocks > 0x7fffffffull) return hipErrorInvalidValue;
    prefill_valu_kernel<VAR, DK, DV><<<dim3(unsigned(nblocks)), dim3(NT), 0, p.stream>>>(a);
    return hipGetLastError();
}

template <int VAR, int DK>
hipError_t dispatch_dv(const Problem& p, const ValuArgs& a) {
    switch (p.dv) {
        case 16: return launch_one<VAR, DK, 16>(p, a);
        case 32: return launch_one<VAR, DK, 32>(p, a);
        case 64: return launch_one<VAR, DK, 64>(p, a);
        case 128: return launch_one<VAR, DK, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

template <int VAR>
hipError_t dispatch_dk(const Problem& p, const ValuArgs& a) {
    switch (p.dk) {
        case 16: return dispatch_dv<VAR, 16>(p, a);
        case 32: return dispatch_dv<VAR, 32>(p, a);
        case 64: return dispatch_dv<VAR, 64>(p, a);
        case 128: return dispatch_dv<VAR, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

// N = 0: the final state is the initial state.
__global__ void state_init_kernel(const float* S0, const float* z0, float* S, float* z,
                                  size_t nS, size_t nz) {
    const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nS && S != S0) S[i] = S0 ? S0[i] : 0.f;
    if (z && i < nz && z != z0) z[i] = z0 ? z0[i] : 0.f;
}

}  // namespace

hipError_t launch_prefill_valu(const Problem& p) {
    ValuArgs a{p.q, p.k, p.v, p.g, p.beta, p.S0, p.z0, p.o, p.S, p.z, p.N, 1, p.eps,
               p.io_bf16, p.gate_bf16, p.cu, p.H, p.L};
    switch (p.variant) {
        case LA_KATH: return dispatch_dk<LA_KATH>(p, a);
        case LA_GLA: return dispatch_dk<LA_GLA>(p, a);
        case LA_GDN: return dispatch_dk<LA_GDN>(p, a);
        case LA_KDA: return dispatch_dk<LA_KDA>(p, a);
        case LA_SSD: return dispatch_dk<LA_SSD>(p, a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_state_init(const Problem& p) {
    const size_t nS = size_t(p.B) * p.H * p.dk * p.dv;
    const size_t nz = p.variant == LA_KATH ? size_t(p.B) * p.H * p.dk : 0;
    const size_t blocks = (nS + 255) / 256;
    if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
    state_init_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, p.stream>>>(p.S0, p.z0, p.S, p.z,
                                                                          nS, nz);
    return hipGetLastError();
}

}  // namespace la
