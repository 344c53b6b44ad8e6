// Decode: one token per (b, h) sequence, state updated in place.
//
// The step is pure state read-modify-write: the fp32 state (d_k x d_v, 64 KiB at
// 128 x 128) is read once and written once, everything else is a few hundred
// bytes. So the kernel is laid out for HBM streaming: one workgroup per state,
// each thread owns RPT rows x 4 consecutive columns (16-byte accesses; a wave
// covers whole contiguous rows), keeps them in registers across the reductions,
// and writes them back once.
//
// Each variant needs a single reduction over the key dim of the OLD state,
// because the post-update read can be expanded (columns of S never mix):
//   GDN  p = S^T k, r = S^T q;  u = beta (v - alpha p);  S <- alpha S + k u^T;
//        o = S_new^T q = alpha r + (k . q) u
//   GLA  r = S^T (q * g);  S <- diag(g) S + k v^T;  o = r + (q . k) v
//   KATH r = S^T phi(q);  S <- S + phi(k) v^T;  z <- z + phi(k);
//        o = (r + (phi(q) . phi(k)) v) / (phi(q) . z_new + eps)
//   KDA  p = S^T (a * k), r = S^T (a * q) (the decayed state Diag(a) S read through
//        k and q); u = beta (v - p);  S <- Diag(a) S + k u^T;  o = r + (k . q) u
//   SSD  r = S^T q;  S <- a S + k v^T;  o = a r + (q . k) v
// ("Linear / RNN 路线", sections 2.1, 2.2, 3.6 and 4.1; "线性注意力与 SSM", section GDN;
// "状态空间与线性注意力", section KDA.)
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "la_internal.h"

namespace la {
namespace {

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float *S, *z;
    void* o;
    float eps;
    int io_bf16, gate_bf16;
};

// Threads per workgroup: a 64 KiB state tile streamed by 512 threads with nontemporal
// 16-byte accesses measured 6.2 TB/s for an in-place read-modify-write on MI355X, against
// 5.8 TB/s with 256 threads. GLA and SSD (the lighter kernels) measured faster still
// with 1024 threads on a 128 x 128 state; GDN, with twice the registers per thread,
// slower. A narrower state keeps 512 threads, so each thread still has 4 rows in flight.
template <int VAR, int DV>
constexpr int decode_nthreads() { return (VAR == LA_GLA || VAR == LA_SSD) && DV >= 128 ? 1024 : 512; }
template <int VAR>
constexpr bool has_delta() { return VAR == LA_GDN || VAR == LA_KDA; }
template <int VAR>
constexpr bool has_channel_gate() { return VAR == LA_GLA || VAR == LA_KDA; }

template <int DK, int DV, int NTH>
struct DecodeShape {
    static constexpr int NCG = DV / 4;                         // 4-column groups
    static constexpr int RG_ALL = NTH / NCG;
    static constexpr int RG = RG_ALL < DK ? RG_ALL : DK;       // row groups
    static constexpr int RPT = DK / RG;                        // rows per thread
    static constexpr int NT = NCG * RG;                        // threads per workgroup
    static_assert(NT > 0 && NT <= NTH && RPT * RG == DK, "decode tiling");
};

constexpr int decode_threads(int dk, int dv, int nth) {
    return (dv / 4) * ((nth / (dv / 4)) < dk ? (nth / (dv / 4)) : dk);
}

template <int VAR, int DK, int DV>
__global__ __launch_bounds__(decode_threads(DK, DV, decode_nthreads<VAR, DV>())) void decode_kernel(
    DecodeArgs a) {
    using Sh = DecodeShape<DK, DV, decode_nthreads<VAR, DV>()>;
    constexpr int NCG = Sh::NCG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
    const int tid = threadIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    const size_t seq = blockIdx.x;
    float* S = a.S + seq * (size_t(DK) * DV);

    __shared__ float sq[DK], sk[DK], sw[DK];  // sw: the gate per key dim (GLA, KDA)
    __shared__ float sv[DV];
    __shared__ float4 red[2][RG][NCG];
    __shared__ float scal[4];

    // Issue the state loads first: they are the whole cost of the step.
    float4 s[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + RG * r;
        s[r] = load_nt4(S + size_t(i) * DV + cg * 4);
    }

    const bool iob = a.io_bf16 != 0, gb = a.gate_bf16 != 0;
    for (int i = tid; i < DK; i += NT) {
        float qi = load_elem(a.q, seq * DK + i, iob);
        float ki = load_elem(a.k, seq * DK + i, iob);
        if (VAR == LA_KATH) {
            qi = elu_plus_one(qi);
            ki = elu_plus_one(ki);
        }
        sq[i] = qi;
        sk[i] = ki;
        if (has_channel_gate<VAR>()) sw[i] = load_elem(a.g, seq * DK + i, gb);
    }
    for (int j = tid; j < DV; j += NT) sv[j] = load_elem(a.v, seq * DV + j, iob);
    __syncthreads();

    // wave 0: the scalar dot products
    if (tid < kWave) {
        float qk = 0.f, qz = 0.f;
        for (int i = tid; i < DK; i += kWave) {
            qk += sq[i] * sk[i];
            if (VAR == LA_KATH) qz += sq[i] * (a.z[seq * DK + i] + sk[i]);
        }
        qk = wave_sum(qk);
        if (VAR == LA_KATH) qz = wave_sum(qz);
        if (tid == 0) {
            scal[0] = qk;
            scal[1] = qz + a.eps;
            if (VAR == LA_GDN || VAR == LA_SSD) scal[2] = load_elem(a.g, seq, gb);
            if (has_delta<VAR>()) scal[3] = load_elem(a.beta, seq, gb);
        }
    }

    // partial reductions of the old state over this thread's rows
    float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), rr = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + RG * r;
        float wq = sq[i];
        if (has_channel_gate<VAR>()) wq *= sw[i];
        rr.x += s[r].x * wq; rr.y += s[r].y * wq; rr.z += s[r].z * wq; rr.w += s[r].w * wq;
        if (has_delta<VAR>()) {
            const float ki = VAR == LA_KDA ? sk[i] * sw[i] : sk[i];
            pr.x += s[r].x * ki; pr.y += s[r].y * ki; pr.z += s[r].z * ki; pr.w += s[r].w * ki;
        }
    }
    red[0][rg][cg] = rr;
    if (has_delta<VAR>()) red[1][rg][cg] = pr;
    __syncthreads();
    float4 R = make_float4(0.f, 0.f, 0.f, 0.f), P = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int x = 0; x < RG; ++x) {
        const float4 t = red[0][x][cg];
        R.x += t.x; R.y += t.y; R.z += t.z; R.w += t.w;
        if (has_delta<VAR>()) {
            const float4 t2 = red[1][x][cg];
            P.x += t2.x; P.y += t2.y; P.z += t2.z; P.w += t2.w;
        }
    }
    const float qk = scal[0];
    const float4 v4 = make_float4(sv[cg * 4], sv[cg * 4 + 1], sv[cg * 4 + 2], sv[cg * 4 + 3]);
    float4 o4;
    if (VAR == LA_KDA) {
        const float be = scal[3];
        float4 u;
        u.x = be * (v4.x - P.x); u.y = be * (v4.y - P.y);
        u.z = be * (v4.z - P.z); u.w = be * (v4.w - P.w);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            const float ki = sk[i], ai = sw[i];
            float4 n;
            n.x = ai * s[r].x + ki * u.x; n.y = ai * s[r].y + ki * u.y;
            n.z = ai * s[r].z + ki * u.z; n.w = ai * s[r].w + ki * u.w;
            store_nt4(S + size_t(i) * DV + cg * 4, n);
        }
        o4.x = R.x + qk * u.x; o4.y = R.y + qk * u.y;
        o4.z = R.z + qk * u.z; o4.w = R.w + qk * u.w;
    } else if (VAR == LA_GDN) {
        const float al = scal[2], be = scal[3];
        float4 u;
        u.x = be * (v4.x - al * P.x); u.y = be * (v4.y - al * P.y);
        u.z = be * (v4.z - al * P.z); u.w = be * (v4.w - al * P.w);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            const float ki = sk[i];
            float4 n;
            n.x = al * s[r].x + ki * u.x; n.y = al * s[r].y + ki * u.y;
            n.z = al * s[r].z + ki * u.z; n.w = al * s[r].w + ki * u.w;
            store_nt4(S + size_t(i) * DV + cg * 4, n);
        }
        o4.x = al * R.x + qk * u.x; o4.y = al * R.y + qk * u.y;
        o4.z = al * R.z + qk * u.z; o4.w = al * R.w + qk * u.w;
    } else {
        const float as = VAR == LA_SSD ? scal[2] : 1.f;   // SSD: the token's decay
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            const float ki = sk[i];
            const float gi = VAR == LA_GLA ? sw[i] : as;
            float4 n;
            n.x = gi * s[r].x + ki * v4.x; n.y = gi * s[r].y + ki * v4.y;
            n.z = gi * s[r].z + ki * v4.z; n.w = gi * s[r].w + ki * v4.w;
            store_nt4(S + size_t(i) * DV + cg * 4, n);
        }
        o4.x = as * R.x + qk * v4.x; o4.y = as * R.y + qk * v4.y;
        o4.z = as * R.z + qk * v4.z; o4.w = as * R.w + qk * v4.w;
        if (VAR == LA_KATH) {
            const float inv = 1.f / scal[1];
            o4.x *= inv; o4.y *= inv; o4.z *= inv; o4.w *= inv;
        }
    }
    if (VAR == LA_KATH) {
        // z is read by wave 0 above; every thread is past the reduction barrier,
        // so the old values have been consumed before any write below.
        for (int i = tid; i < DK; i += NT) a.z[seq * DK + i] += sk[i];
    }
    if (rg == 0) store4(a.o, seq * DV + size_t(cg) * 4, o4, iob);
}

// Persistent form: a grid of a few workgroups per compute unit walks the states
// (blockIdx.x, + gridDim.x, ...). Each iteration first issues the loads of the next state
// it will take (into a second register set) and of that state's q, k, v and gates, then
// reduces, updates and stores the current one, so the HBM reads of one state overlap the
// reductions, barriers and writes of the previous. LDS is double-buffered by iteration
// parity; the two barriers of an iteration separate every write of a buffer from the
// reads of the iteration that last used it.
template <int VAR, int DK, int DV, int NTH, bool IOB, bool GB, int MAXIT>
__global__ __launch_bounds__(decode_threads(DK, DV, NTH)) void decode_persist_kernel(DecodeArgs a, int nseq) {
    using Sh = DecodeShape<DK, DV, NTH>;
    constexpr int NCG = Sh::NCG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
    static_assert(DK <= NT && DV <= NT, "one small element per thread");
    const int tid = threadIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    // storage types are template arguments: a run-time choice would put branches between
    // the loads, and the waits after them could no longer count the loads in flight
    constexpr bool iob = IOB, gb = GB;

    __shared__ float sq[2][DK], sk[2][DK], sw[2][DK];   // sw: the gate per key dim (GLA, KDA)
    __shared__ float sv[2][DV];
    __shared__ float4 red[2][2][RG][NCG];
    __shared__ float scal[2][4];

    // The small per-token inputs are loaded as raw bits and converted only where they are
    // used, so that no wait for them (and hence for the state loads issued before them)
    // lands in the middle of the iteration.
    struct Small { uint32_t q, k, w, v, ga, be; };
    auto raw = [](const void* p, size_t i, bool bf16) -> uint32_t {
        if (bf16) return uint32_t(static_cast<const uint16_t*>(p)[i]);
        return static_cast<const uint32_t*>(p)[i];
    };
    auto val = [](uint32_t r, bool bf16) { return __uint_as_float(bf16 ? r << 16 : r); };
    // every thread issues the same loads (indices wrapped), so the number of loads in
    // flight is the same on every path and the waits stay exact
    auto load_small = [&](size_t seq, Small& m) {
        m.q = raw(a.q, seq * DK + tid % DK, iob);
        m.k = raw(a.k, seq * DK + tid % DK, iob);
        if (has_channel_gate<VAR>()) m.w = raw(a.g, seq * DK + tid % DK, gb);
        m.v = raw(a.v, seq * DV + tid % DV, iob);
        if (VAR == LA_GDN || VAR == LA_SSD) m.ga = raw(a.g, seq, gb);
        if (has_delta<VAR>()) m.be = raw(a.beta, seq, gb);
    };
    auto load_state = [&](size_t seq, float4 (&s)[RPT]) {
        const float* S = a.S + seq * (size_t(DK) * DV);
#pragma unroll
        for (int r = 0; r < RPT; ++r) s[r] = load_nt4(S + size_t(rg + RG * r) * DV + cg * 4);
    };

    // One state: t, with its state in cur and inputs in mc; the next state's loads go to
    // nxt and mn. Returns false after the last state of this workgroup.
    auto step = [&](int& t, float4 (&cur)[RPT], float4 (&nxt)[RPT], const Small& mc, Small& mn,
                    int par) -> bool {
        const size_t seq = size_t(t);
        const int tn = t + int(gridDim.x);
        if (tn < nseq) {
            load_state(size_t(tn), nxt);
            load_small(size_t(tn), mn);
        }
        // stage this state's vectors
        if (tid < DK) {
            float qi = val(mc.q, iob), ki = val(mc.k, iob);
            if (VAR == LA_KATH) {
                qi = elu_plus_one(qi);
                ki = elu_plus_one(ki);
            }
            sq[par][tid] = qi;
            sk[par][tid] = ki;
            if (has_channel_gate<VAR>()) sw[par][tid] = val(mc.w, gb);
        }
        if (tid < DV) sv[par][tid] = val(mc.v, iob);
        __syncthreads();
        // wave 0: the scalar dot products
        if (tid < kWave) {
            float qk = 0.f, qz = 0.f;
            for (int i = tid; i < DK; i += kWave) {
                qk += sq[par][i] * sk[par][i];
                if (VAR == LA_KATH) qz += sq[par][i] * (a.z[seq * DK + i] + sk[par][i]);
            }
            qk = wave_sum(qk);
            if (VAR == LA_KATH) qz = wave_sum(qz);
            if (tid == 0) {
                scal[par][0] = qk;
                scal[par][1] = qz + a.eps;
                if (VAR == LA_GDN || VAR == LA_SSD) scal[par][2] = val(mc.ga, gb);
                if (has_delta<VAR>()) scal[par][3] = val(mc.be, gb);
            }
        }
        // partial reductions of the old state over this thread's rows
        float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), rr = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            float wq = sq[par][i];
            if (has_channel_gate<VAR>()) wq *= sw[par][i];
            rr.x += cur[r].x * wq; rr.y += cur[r].y * wq; rr.z += cur[r].z * wq; rr.w += cur[r].w * wq;
            if (has_delta<VAR>()) {
                const float ki = VAR == LA_KDA ? sk[par][i] * sw[par][i] : sk[par][i];
                pr.x += cur[r].x * ki; pr.y += cur[r].y * ki; pr.z += cur[r].z * ki; pr.w += cur[r].w * ki;
            }
        }
        red[par][0][rg][cg] = rr;
        if (has_delta<VAR>()) red[par][1][rg][cg] = pr;
        __syncthreads();
        float4 R = make_float4(0.f, 0.f, 0.f, 0.f), P = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int x = 0; x < RG; ++x) {
            const float4 t1 = red[par][0][x][cg];
            R.x += t1.x; R.y += t1.y; R.z += t1.z; R.w += t1.w;
            if (has_delta<VAR>()) {
                const float4 t2 = red[par][1][x][cg];
                P.x += t2.x; P.y += t2.y; P.z += t2.z; P.w += t2.w;
            }
        }
        float* S = a.S + seq * (size_t(DK) * DV);
        const float qk = scal[par][0];
        const float4 v4 = make_float4(sv[par][cg * 4], sv[par][cg * 4 + 1], sv[par][cg * 4 + 2], sv[par][cg * 4 + 3]);
        float4 o4;
        if (has_delta<VAR>()) {
            // GDN: u = beta (v - alpha p), S <- alpha S + k u^T, o = alpha r + (k.q) u;
            // KDA: u = beta (v - p), S <- Diag(a) S + k u^T, o = r + (k.q) u
            const float al = VAR == LA_GDN ? scal[par][2] : 1.f, be = scal[par][3];
            float4 u;
            u.x = be * (v4.x - al * P.x); u.y = be * (v4.y - al * P.y);
            u.z = be * (v4.z - al * P.z); u.w = be * (v4.w - al * P.w);
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                const float ki = sk[par][i], ai = VAR == LA_KDA ? sw[par][i] : al;
                float4 n;
                n.x = ai * cur[r].x + ki * u.x; n.y = ai * cur[r].y + ki * u.y;
                n.z = ai * cur[r].z + ki * u.z; n.w = ai * cur[r].w + ki * u.w;
                store_nt4(S + size_t(i) * DV + cg * 4, n);
            }
            o4.x = al * R.x + qk * u.x; o4.y = al * R.y + qk * u.y;
            o4.z = al * R.z + qk * u.z; o4.w = al * R.w + qk * u.w;
        } else {
            const float as = VAR == LA_SSD ? scal[par][2] : 1.f;   // SSD: the token's decay
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                const float ki = sk[par][i];
                const float gi = VAR == LA_GLA ? sw[par][i] : as;
                float4 n;
                n.x = gi * cur[r].x + ki * v4.x; n.y = gi * cur[r].y + ki * v4.y;
                n.z = gi * cur[r].z + ki * v4.z; n.w = gi * cur[r].w + ki * v4.w;
                store_nt4(S + size_t(i) * DV + cg * 4, n);
            }
            o4.x = as * R.x + qk * v4.x; o4.y = as * R.y + qk * v4.y;
            o4.z = as * R.z + qk * v4.z; o4.w = as * R.w + qk * v4.w;
            if (VAR == LA_KATH) {
                const float inv = 1.f / scal[par][1];
                o4.x *= inv; o4.y *= inv; o4.z *= inv; o4.w *= inv;
            }
        }
        if (VAR == LA_KATH) {
            // z is read by wave 0 above; every thread is past the reduction barrier,
            // so the old values have been consumed before any write below.
            if (tid < DK) a.z[seq * DK + tid] += sk[par][tid];
        }
        if (rg == 0) store4(a.o, seq * DV + size_t(cg) * 4, o4, iob);
        t = tn;
        return tn < nseq;
    };

    int t = blockIdx.x;
    if (t >= nseq) return;
    float4 sa[RPT], sb[RPT];
    Small ma{}, mb{};
    load_state(size_t(t), sa);
    load_small(size_t(t), ma);
    // at most MAXIT states per workgroup, fully unrolled: two register sets swapped by
    // unrolling rather than copied (a copy would wait for the loads in flight), and
    // straight-line code, in which the waits count exactly which loads are in flight
#pragma unroll
    for (int it = 0; it < MAXIT; it += 2) {
        if (!step(t, sa, sb, ma, mb, 0)) break;
        if (it + 1 >= MAXIT || !step(t, sb, sa, mb, ma, 1)) break;
    }
}

// The persistent form for bf16 token inputs and gates with d_k = 128 (the large states):
// threads per workgroup and states per workgroup as measured best for an in-place step of
// 8,192 states on MI355X (GLA and SSD at d_v = 128: 1024 threads, up to 16 states; the
// others: 512 threads, up to 8), at least two workgroups per compute unit.
template <int VAR, int DV>
constexpr int persist_threads() { return (VAR == LA_GLA || VAR == LA_SSD) && DV >= 128 ? 1024 : 512; }
template <int VAR, int DV>
constexpr int persist_states() { return persist_threads<VAR, DV>() == 1024 ? 16 : 8; }

template <int VAR, int DK, int DV>
hipError_t launch_one(const Problem& p, const DecodeArgs& a) {
    const size_t nseq = size_t(p.B) * size_t(p.H);
    if constexpr (DK == 128 && DV >= 64) {
        if (p.io_bf16 && p.gate_bf16) {
            constexpr int NTH = persist_threads<VAR, DV>(), MAXIT = persist_states<VAR, DV>();
            const size_t need = (nseq + MAXIT - 1) / MAXIT;
            const size_t grid = std::min(nseq, std::max(size_t(device_cus()) * 2, need));
            decode_persist_kernel<VAR, DK, DV, NTH, true, true, MAXIT>
                <<<dim3(unsigned(grid)), dim3(DecodeShape<DK, DV, NTH>::NT), 0, p.stream>>>(a, int(nseq));
            return hipGetLastError();
        }
    }
    decode_kernel<VAR, DK, DV>
        <<<dim3(unsigned(nseq)), dim3(DecodeShape<DK, DV, decode_nthreads<VAR, DV>()>::NT), 0, p.stream>>>(a);
    return hipGetLastError();
}

template <int VAR, int DK>
hipError_t dispatch_dv(const Problem& p, const DecodeArgs& a) {
    switch (p.dv) {
        case 16: return launch_one<VAR, DK, 16>(p, a);
        case 32: return launch_one<VAR, DK, 32>(p, a);
        case 64: return launch_one<VAR, DK, 64>(p, a);
        case 128: return launch_one<VAR, DK, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

template <int VAR>
hipError_t dispatch_dk(const Problem& p, const DecodeArgs& a) {
    switch (p.dk) {
        case 16: return dispatch_dv<VAR, 16>(p, a);
        case 32: return dispatch_dv<VAR, 32>(p, a);
        case 64: return dispatch_dv<VAR, 64>(p, a);
        case 128: return dispatch_dv<VAR, 128>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// compute units of the current device (queried once per device; 256 if the query fails)
int device_cus() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_decode(const Problem& p) {
    if (size_t(p.B) * size_t(p.H) > 0x7fffffffull) return hipErrorInvalidValue;   // fits int
    DecodeArgs a{p.q, p.k, p.v, p.g, p.beta, p.S, p.z, p.o, p.eps, p.io_bf16, p.gate_bf16};
    switch (p.variant) {
        case LA_KATH: return dispatch_dk<LA_KATH>(p, a);
        case LA_GLA: return dispatch_dk<LA_GLA>(p, a);
        case LA_GDN: return dispatch_dk<LA_GDN>(p, a);
        case LA_KDA: return dispatch_dk<LA_KDA>(p, a);
        case LA_SSD: return dispatch_dk<LA_SSD>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
