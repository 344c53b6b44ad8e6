// C-ABI entry points: argument validation, planning (path, chunk, segments,
// workspace) and dispatch to the kernel launchers. All validation happens
// before the first HIP call, so an invalid call enqueues nothing and touches
// no output.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "la_internal.h"

namespace {

using la::Problem;

constexpr uint64_t kMaxElems = uint64_t(1) << 46;  // per buffer; keeps every size in 64 bits

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// a * b, or 0 on overflow past kMaxElems
uint64_t mul(uint64_t a, uint64_t b) {
    if (a == 0 || b == 0) return 0;
    if (a > kMaxElems / b) return UINT64_MAX;
    return a * b;
}

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range(const void* p, uint64_t bytes) {
    Range r;
    if (p && bytes && bytes != UINT64_MAX) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + bytes;
    }
    return r;
}

bool overlap(Range a, Range b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool check_alignment(const la_desc& d, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const void* S0, const void* z0,
                     const void* o, const void* S, const void* z) {
    const void* vec[] = {q, k, v, S0, z0, o, S, z};
    for (const void* ptr : vec)
        if (ptr && !aligned(ptr, 16)) return false;
    const uintptr_t gsz = d.gate_dtype == LA_BF16 ? 2 : 4;
    if ((d.variant == LA_GLA || d.variant == LA_KDA) && g && !aligned(g, 16)) return false;
    if (d.variant == LA_GDN && ((g && !aligned(g, gsz)) || (beta && !aligned(beta, gsz))))
        return false;
    if (d.variant == LA_SSD && g && !aligned(g, gsz)) return false;
    if (d.variant == LA_KDA && beta && !aligned(beta, gsz)) return false;
    return true;
}

struct Sizes {
    uint64_t q, k, v, o, g, beta, S, z;
};

// Byte sizes of every buffer for this descriptor (decode: N = 1).
Sizes sizes_of(const la_desc& d) {
    Sizes s{};
    const uint64_t isz = d.io_dtype == LA_BF16 ? 2 : 4, gsz = d.gate_dtype == LA_BF16 ? 2 : 4;
    const uint64_t tok = mul(mul(uint64_t(d.B), uint64_t(d.H)), uint64_t(d.N));
    const uint64_t seq = mul(uint64_t(d.B), uint64_t(d.H));
    s.q = s.k = mul(mul(tok, d.dk), isz);
    s.v = s.o = mul(mul(tok, d.dv), isz);
    s.g = (d.variant == LA_GLA || d.variant == LA_KDA) ? mul(mul(tok, d.dk), gsz)
          : (d.variant == LA_GDN || d.variant == LA_SSD) ? mul(tok, gsz)
                                                        : 0;
    s.beta = (d.variant == LA_GDN || d.variant == LA_KDA) ? mul(tok, gsz) : 0;
    s.S = mul(mul(mul(seq, d.dk), d.dv), 4);
    s.z = d.variant == LA_KATH ? mul(mul(seq, d.dk), 4) : 0;
    return s;
}

// Descriptor checks shared by prefill, decode and the workspace query.
int check_desc(const la_desc* d, bool decode) {
    if (!d) return LA_ERR_INVALID;
    if (d->variant < LA_KATH || d->variant > LA_SSD) return LA_ERR_INVALID;
    if (d->io_dtype != LA_F32 && d->io_dtype != LA_BF16) return LA_ERR_INVALID;
    if (d->variant != LA_KATH && d->gate_dtype != LA_F32 && d->gate_dtype != LA_BF16)
        return LA_ERR_INVALID;
    if (d->B < 0 || d->H < 0 || d->N < 0) return LA_ERR_INVALID;
    if (decode && d->N != 1) return LA_ERR_INVALID;
    if (d->variant == LA_KATH && !(std::isfinite(d->eps) && d->eps >= 0.f)) return LA_ERR_INVALID;
    if (d->path < LA_PATH_AUTO || d->path > LA_PATH_MFMA) return LA_ERR_INVALID;
    if (d->chunk < 0 || d->segments < 0) return LA_ERR_INVALID;
    if (!supported_dim(d->dk) || !supported_dim(d->dv)) return LA_ERR_UNSUPPORTED;
    const Sizes s = sizes_of(*d);
    if (s.q == UINT64_MAX || s.v == UINT64_MAX || s.g == UINT64_MAX || s.S == UINT64_MAX ||
        s.z == UINT64_MAX)
        return LA_ERR_INVALID;
    return LA_OK;
}

// Resolve path, chunk and segments for a prefill over nseq sequences per head whose
// longest has max_len tokens (a dense batch: nseq = B, max_len = N, cu = null).
int plan_prefill(const la_desc& d, Problem& p, int nseq, int max_len, const int32_t* cu,
                 bool packed) {
    p.B = nseq; p.H = d.H; p.N = d.N; p.dk = d.dk; p.dv = d.dv;
    p.L = max_len;
    p.cu = cu;
    p.packed = packed;
    p.variant = d.variant;
    p.io_bf16 = d.io_dtype == LA_BF16;
    p.gate_bf16 = d.gate_dtype == LA_BF16;
    p.eps = d.eps;
    const bool mfma_ok = d.variant == LA_GDN   ? la::gdn_mfma_supported(d.dk, d.dv, p.io_bf16)
                         : d.variant == LA_KDA ? la::kda_mfma_supported(d.dk, d.dv, p.io_bf16)
                         : (d.variant == LA_GLA || d.variant == LA_SSD)
                             ? la::gla_mfma_supported(d.dk, d.dv, p.io_bf16)
                                               : la::kath_mfma_supported(d.dk, d.dv, p.io_bf16);
    int path = d.path;
    if (path == LA_PATH_AUTO) path = mfma_ok ? LA_PATH_MFMA : LA_PATH_VALU;
    if (path == LA_PATH_MFMA && !mfma_ok) return LA_ERR_UNSUPPORTED;
    p.path = path;
    p.chunk = path == LA_PATH_MFMA ? la::kMfmaChunk : la::kValuChunk;
    if (d.chunk != 0 && d.chunk != p.chunk) return LA_ERR_UNSUPPORTED;
    p.segments = 1;
    const bool diag = d.variant == LA_GLA || d.variant == LA_SSD;   // diagonal transition
    if (path == LA_PATH_MFMA && (d.variant == LA_KATH || diag) && p.L > 0) {
        const int nchunks = (p.L + p.chunk - 1) / p.chunk;
        int segs = d.segments > 0 ? d.segments
                   : diag         ? la::gla_mfma_auto_segments(p)
                                  : la::kath_mfma_auto_segments(p);
        if (segs > nchunks) segs = nchunks;
        if (segs < 1) segs = 1;
        // equal segments of cps chunks; drop segments that would be empty
        const int cps = (nchunks + segs - 1) / segs;
        p.segments = (nchunks + cps - 1) / cps;
    }
    return LA_OK;
}

size_t workspace_for(const Problem& p) {
    if (p.N == 0 || p.L == 0 || p.B == 0 || p.H == 0) return 0;
    if (p.path == LA_PATH_MFMA)
        return p.variant == LA_GDN   ? la::gdn_mfma_workspace_bytes(p)
               : p.variant == LA_KDA ? la::kda_mfma_workspace_bytes(p)
               : p.variant == LA_GLA ? la::gla_mfma_workspace_bytes(p)
               : p.variant == LA_SSD ? la::ssd_mfma_workspace_bytes(p)
                                     : la::kath_mfma_workspace_bytes(p);
    return 0;
}

}  // namespace

extern "C" {

int la_abi_version(void) { return LA_ABI_VERSION; }

const char* la_status_str(int status) {
    switch (status) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported shape, dtype, path or chunk size";
        case LA_ERR_HIP: return "HIP kernel launch failed";
        case LA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}

int la_prefill_workspace_size(const la_desc* d, size_t* bytes) {
    int rc = check_desc(d, false);
    if (rc != LA_OK) return rc;
    if (!bytes) return LA_ERR_INVALID;
    Problem p;
    rc = plan_prefill(*d, p, d->B, d->N, nullptr, false);
    if (rc != LA_OK) return rc;
    *bytes = workspace_for(p);
    return LA_OK;
}

int la_prefill_varlen_workspace_size(const la_desc* d, int32_t nseq, int32_t max_seqlen,
                                     size_t* bytes) {
    int rc = check_desc(d, false);
    if (rc != LA_OK) return rc;
    if (!bytes || d->B != 1 || nseq < 0 || max_seqlen < 0 || max_seqlen > d->N) return LA_ERR_INVALID;
    Problem p;
    rc = plan_prefill(*d, p, nseq, max_seqlen, nullptr, true);
    if (rc != LA_OK) return rc;
    *bytes = workspace_for(p);
    return LA_OK;
}

}  // extern "C"

namespace {

// Shared by la_prefill (nseq = B, cu = null, max_len = N) and la_prefill_varlen.
int prefill_impl(const la_desc* d, int nseq, const int32_t* cu, int max_len, const void* q,
                 const void* k, const void* v, const void* g, const void* beta, const float* S0,
                 const float* z0, void* o, float* S_final, float* z_final, void* workspace,
                 size_t workspace_bytes, void* stream) {
    int rc = check_desc(d, false);
    if (rc != LA_OK) return rc;
    Problem p;
    rc = plan_prefill(*d, p, nseq, max_len, cu, cu != nullptr);
    if (rc != LA_OK) return rc;
    const bool kath = d->variant == LA_KATH, gla = d->variant == LA_GLA,
               gdn = d->variant == LA_GDN, kda = d->variant == LA_KDA, ssd = d->variant == LA_SSD;
    const bool varlen = cu != nullptr;
    const bool empty_seq = (uint64_t(nseq) * uint64_t(d->H)) == 0;
    const bool tokens = !empty_seq && d->N > 0 && (uint64_t(d->B) * uint64_t(d->H)) > 0;
    // presence rules
    if (kath && (g || beta)) return LA_ERR_INVALID;
    if ((gla || ssd) && beta) return LA_ERR_INVALID;
    if (!kath && (z0 || z_final)) return LA_ERR_INVALID;
    if (!empty_seq) {
        if (!S_final) return LA_ERR_INVALID;
        if (kath && !z_final) return LA_ERR_INVALID;
    }
    if (tokens) {
        if (!q || !k || !v || !o) return LA_ERR_INVALID;
        if ((gla || gdn || kda || ssd) && !g) return LA_ERR_INVALID;
        if ((gdn || kda) && !beta) return LA_ERR_INVALID;
    }
    // alignment: 16 bytes for the arrays read or written with 128-bit accesses; the
    // per-token scalar gates of GDN (alpha, beta) only need element alignment
    if (!check_alignment(*d, q, k, v, g, beta, S0, z0, o, S_final, z_final))
        return LA_ERR_INVALID;
    // aliasing: outputs overlap nothing, except S_final == S0 and z_final == z0 exactly
    Sizes s = sizes_of(*d);
    if (varlen) {   // states are per (sequence, head), not per (batch row, head)
        const uint64_t states = mul(uint64_t(nseq), uint64_t(d->H));
        s.S = mul(mul(mul(states, d->dk), d->dv), 4);
        s.z = d->variant == LA_KATH ? mul(mul(states, d->dk), 4) : 0;
        if (s.S == UINT64_MAX || s.z == UINT64_MAX) return LA_ERR_INVALID;
    }
    const Range rq = range(q, tokens ? s.q : 0), rk = range(k, tokens ? s.k : 0),
                rv = range(v, tokens ? s.v : 0), rg = range(g, tokens ? s.g : 0),
                rb = range(beta, tokens ? s.beta : 0), rS0 = range(S0, s.S), rz0 = range(z0, s.z),
                ro = range(o, tokens ? s.o : 0), rS = range(S_final, s.S),
                rz = range(z_final, s.z),
                rc_ = range(cu, varlen ? (uint64_t(nseq) + 1) * 4 : 0);
    const Range inputs[] = {rq, rk, rv, rg, rb, rS0, rz0, rc_};
    for (const Range& in : inputs) {
        if (overlap(ro, in)) return LA_ERR_INVALID;
    }
    if (overlap(ro, rS) || overlap(ro, rz) || overlap(rS, rz)) return LA_ERR_INVALID;
    const Range nonstate_inputs[] = {rq, rk, rv, rg, rb};
    for (const Range& in : nonstate_inputs) {
        if (overlap(rS, in) || overlap(rz, in)) return LA_ERR_INVALID;
    }
    if (overlap(rS, rS0) && S_final != S0) return LA_ERR_INVALID;
    if (overlap(rS, rz0) || overlap(rz, rS0)) return LA_ERR_INVALID;
    if (overlap(rS, rc_) || overlap(rz, rc_)) return LA_ERR_INVALID;
    if (overlap(rz, rz0) && z_final != z0) return LA_ERR_INVALID;
    // workspace
    const size_t need = workspace_for(p);
    if (need > 0) {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
            return LA_ERR_WORKSPACE;
        const Range rw = range(workspace, need);
        const Range every[] = {rq, rk, rv, rg, rb, rS0, rz0, ro, rS, rz, rc_};
        for (const Range& x : every)
            if (overlap(rw, x)) return LA_ERR_INVALID;
    }
    if (empty_seq) return LA_OK;

    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.S0 = S0; p.z0 = z0; p.o = o; p.S = S_final; p.z = z_final;
    p.ws = workspace; p.ws_bytes = workspace_bytes;
    p.stream = static_cast<hipStream_t>(stream);

    (void)hipGetLastError();  // clear a stale error so the check below sees this call's
    hipError_t err;
    if (p.N == 0 || p.L == 0)
        err = la::launch_state_init(p);
    else if (p.path == LA_PATH_MFMA)
        err = gdn                     ? la::launch_prefill_gdn_mfma(p)
              : kda                   ? la::launch_prefill_kda_mfma(p)
              : gla                   ? la::launch_prefill_gla_mfma(p)
              : ssd                   ? la::launch_prefill_ssd_mfma(p)
                                    : la::launch_prefill_kath_mfma(p);
    else
        err = la::launch_prefill_valu(p);
    if (err == hipSuccess) err = hipGetLastError();
    return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

extern "C" {

int la_prefill(const la_desc* d, const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* S0, const float* z0, void* o, float* S_final,
               float* z_final, void* workspace, size_t workspace_bytes, void* stream) {
    if (!d) return LA_ERR_INVALID;
    return prefill_impl(d, d->B, nullptr, d->N, q, k, v, g, beta, S0, z0, o, S_final, z_final,
                        workspace, workspace_bytes, stream);
}

int la_prefill_varlen(const la_desc* d, int32_t nseq, const int32_t* cu_seqlens,
                      int32_t max_seqlen, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S0, const float* z0, void* o,
                      float* S_final, float* z_final, void* workspace, size_t workspace_bytes,
                      void* stream) {
    if (!d) return LA_ERR_INVALID;
    if (d->B != 1 || nseq < 0 || max_seqlen < 0 || max_seqlen > d->N) return LA_ERR_INVALID;
    if (nseq > 0 && (!cu_seqlens || !aligned(cu_seqlens, 4))) return LA_ERR_INVALID;
    if (nseq == 0) cu_seqlens = nullptr;
    if (nseq > 0) {
        return prefill_impl(d, nseq, cu_seqlens, max_seqlen, q, k, v, g, beta, S0, z0, o,
                            S_final, z_final, workspace, workspace_bytes, stream);
    }
    // no sequences: only the descriptor and argument presence are checked
    return prefill_impl(d, 0, nullptr, 0, q, k, v, g, beta, S0, z0, o, S_final, z_final,
                        workspace, workspace_bytes, stream);
}

int la_decode_step(const la_desc* d, const void* q, const void* k, const void* v, const void* g,
                   const void* beta, float* S, float* z, void* o, void* stream) {
    int rc = check_desc(d, true);
    if (rc != LA_OK) return rc;
    const bool kath = d->variant == LA_KATH, gla = d->variant == LA_GLA,
               gdn = d->variant == LA_GDN, kda = d->variant == LA_KDA, ssd = d->variant == LA_SSD;
    if (kath && (g || beta)) return LA_ERR_INVALID;
    if ((gla || ssd) && beta) return LA_ERR_INVALID;
    if (!kath && z) return LA_ERR_INVALID;
    const bool empty_seq = (uint64_t(d->B) * uint64_t(d->H)) == 0;
    if (!empty_seq) {
        if (!q || !k || !v || !o || !S) return LA_ERR_INVALID;
        if ((gla || gdn || kda || ssd) && !g) return LA_ERR_INVALID;
        if ((gdn || kda) && !beta) return LA_ERR_INVALID;
        if (kath && !z) return LA_ERR_INVALID;
    }
    if (!check_alignment(*d, q, k, v, g, beta, nullptr, nullptr, o, S, z)) return LA_ERR_INVALID;
    const Sizes s = sizes_of(*d);
    const Range rq = range(q, s.q), rk = range(k, s.k), rv = range(v, s.v), rg = range(g, s.g),
                rb = range(beta, s.beta), rS = range(S, s.S), rz = range(z, s.z),
                ro = range(o, s.o);
    const Range others[] = {rq, rk, rv, rg, rb, rS, rz};
    for (const Range& x : others)
        if (overlap(ro, x)) return LA_ERR_INVALID;
    const Range tok_inputs[] = {rq, rk, rv, rg, rb};
    for (const Range& x : tok_inputs)
        if (overlap(rS, x) || overlap(rz, x)) return LA_ERR_INVALID;
    if (overlap(rS, rz)) return LA_ERR_INVALID;
    if (empty_seq) return LA_OK;

    Problem p;
    p.B = d->B; p.H = d->H; p.N = 1; p.dk = d->dk; p.dv = d->dv;
    p.variant = d->variant;
    p.io_bf16 = d->io_dtype == LA_BF16;
    p.gate_bf16 = d->gate_dtype == LA_BF16;
    p.eps = d->eps;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.S = S; p.z = z; p.o = o;
    p.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t err = la::launch_decode(p);
    if (err == hipSuccess) err = hipGetLastError();
    return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Backward: the forward's descriptor and a variant with a backward kernel. Path AUTO takes
// the matrix-core backward where the shape allows it (bf16 q, k, v; SSD with d_k = 128,
// d_v = 64; GDN with d_k = 128, d_v = 64 or 128), else the fp32 VALU backward.
static int check_backward_desc(const la_desc* d, la::Problem& p) {
    int rc = check_desc(d, false);
    if (rc != LA_OK) return rc;
    if (!la::backward_supported(d->variant)) return LA_ERR_UNSUPPORTED;
    p.B = d->B; p.H = d->H; p.N = d->N; p.dk = d->dk; p.dv = d->dv; p.L = d->N;
    p.variant = d->variant;
    p.io_bf16 = d->io_dtype == LA_BF16;
    p.gate_bf16 = d->gate_dtype == LA_BF16;
    p.eps = d->eps;
    const bool mfma_ok = la::ssd_backward_mfma_supported(p) || la::gdn_backward_mfma_supported(p);
    if (d->path == LA_PATH_MFMA && !mfma_ok) return LA_ERR_UNSUPPORTED;
    p.path = (d->path != LA_PATH_VALU && mfma_ok) ? LA_PATH_MFMA : LA_PATH_VALU;
    p.chunk = p.path == LA_PATH_MFMA ? la::kMfmaChunk : la::kValuChunk;
    if (d->chunk != 0 && d->chunk != p.chunk) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

static size_t backward_workspace(const la::Problem& p) {
    if (p.path != LA_PATH_MFMA) return la::backward_workspace_bytes(p);
    return p.variant == LA_GDN ? la::gdn_backward_mfma_workspace_bytes(p)
                               : la::ssd_backward_mfma_workspace_bytes(p);
}

int la_prefill_backward_workspace_size(const la_desc* d, size_t* bytes) {
    if (!bytes) return LA_ERR_INVALID;
    la::Problem p;
    const int rc = check_backward_desc(d, p);
    if (rc != LA_OK) return rc;
    *bytes = backward_workspace(p);
    return LA_OK;
}

int la_prefill_backward(const la_desc* d, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const float* S0, const float* z0,
                        const void* dO, const float* dS_final, const float* dz_final, void* dq,
                        void* dk, void* dv, void* dg, void* dbeta, float* dS0, float* dz0,
                        void* workspace, size_t workspace_bytes, void* stream) {
    la::Problem p;
    int rc = check_backward_desc(d, p);
    if (rc != LA_OK) return rc;
    // GDN and KDA (the delta rule) take beta; KATH has no gate and carries the normaliser z
    const bool delta = d->variant == LA_GDN || d->variant == LA_KDA, kath = d->variant == LA_KATH;
    if (!kath && (z0 || dz_final || dz0)) return LA_ERR_INVALID;
    if (kath && (g || dg)) return LA_ERR_INVALID;
    if (!delta && (beta || dbeta)) return LA_ERR_INVALID;
    const bool seqs = (uint64_t(d->B) * uint64_t(d->H)) > 0;
    const bool tokens = seqs && d->N > 0;
    if (seqs && (!dS0 || (kath && !dz0))) return LA_ERR_INVALID;
    if (tokens && (!q || !k || !v || !dO || !dq || !dk || !dv)) return LA_ERR_INVALID;
    if (tokens && !kath && (!g || !dg)) return LA_ERR_INVALID;
    if (tokens && delta && (!beta || !dbeta)) return LA_ERR_INVALID;
    // alignment: dq, dk as q; dv, dO as v; dg as g; dbeta as beta; the fp32 states 16 bytes
    if (!check_alignment(*d, q, k, v, g, beta, S0, z0, dv, dS0, dz0) ||
        !check_alignment(*d, dq, dk, dO, dg, dbeta, dS_final, dz_final, nullptr, nullptr, nullptr))
        return LA_ERR_INVALID;
    const Sizes s = sizes_of(*d);
    const uint64_t tk = tokens ? 1 : 0;
    const Range rq = range(q, s.q * tk), rk = range(k, s.k * tk), rv = range(v, s.v * tk),
                rg = range(g, s.g * tk), rS0 = range(S0, s.S), rdO = range(dO, s.o * tk),
                rdSf = range(dS_final, s.S), rdq = range(dq, s.q * tk), rdk = range(dk, s.k * tk),
                rdv = range(dv, s.v * tk), rdg = range(dg, s.g * tk),
                rdS0 = range(dS0, s.S), rb = range(beta, s.beta * tk),
                rdb = range(dbeta, s.beta * tk), rz0 = range(z0, s.z),
                rdzf = range(dz_final, s.z), rdz0 = range(dz0, s.z);
    // outputs overlap nothing: not the inputs, not each other
    const Range outs[] = {rdq, rdk, rdv, rdg, rdS0, rdb, rdz0};
    const Range all[] = {rq,  rk,  rv,  rg,  rS0,  rdO, rdSf, rb, rz0,
                         rdzf, rdq, rdk, rdv, rdg, rdS0, rdb, rdz0};
    for (int a = 0; a < 7; ++a)
        for (const Range& x : all)
            if (&x != &all[10 + a] && overlap(outs[a], x)) return LA_ERR_INVALID;
    const size_t need = backward_workspace(p);
    if (need > 0) {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return LA_ERR_WORKSPACE;
        const Range rw = range(workspace, need);
        for (const Range& x : all)
            if (overlap(rw, x)) return LA_ERR_INVALID;
    }
    if (!seqs) return LA_OK;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0; p.z0 = z0;
    p.ws = workspace; p.ws_bytes = workspace_bytes;
    p.stream = static_cast<hipStream_t>(stream);
    la::BwdProblem bp;
    bp.p = p;
    bp.dO = dO; bp.dS_final = dS_final;
    bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta; bp.dS0 = dS0;
    bp.dz_final = dz_final; bp.dz0 = dz0;
    (void)hipGetLastError();
    hipError_t err = hipSuccess;
    if (p.path == LA_PATH_MFMA && p.N > 0)
        err = p.variant == LA_GDN ? la::launch_backward_gdn_mfma(bp) : la::launch_backward_ssd_mfma(bp);
    else
        err = la::launch_backward(bp);
    if (err == hipSuccess) err = hipGetLastError();
    return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_selective_scan(const la_scan_desc* d, const void* dt, const float* A, const void* Bm,
                      const void* Cm, const void* x, const float* Dskip, const float* dt_bias,
                      const float* h0, void* y, float* h_final, void* stream) {
    if (!d) return LA_ERR_INVALID;
    if (d->io_dtype != LA_F32 && d->io_dtype != LA_BF16) return LA_ERR_INVALID;
    if (d->Bt < 0 || d->T < 0 || d->D < 0 || d->n < 0) return LA_ERR_INVALID;
    if (d->dt_softplus != 0 && d->dt_softplus != 1) return LA_ERR_INVALID;
    if (!la::selective_scan_supported(d->n)) return LA_ERR_UNSUPPORTED;
    const uint64_t isz = d->io_dtype == LA_BF16 ? 2 : 4;
    const uint64_t rows = uint64_t(d->Bt), T = uint64_t(d->T), D = uint64_t(d->D),
                   n = uint64_t(d->n);
    const uint64_t s_tok = mul(mul(mul(rows, T), D), isz);   // dt, x, y
    const uint64_t s_bc = mul(mul(mul(rows, T), n), isz);    // B, C
    const uint64_t s_A = mul(mul(D, n), 4), s_ch = mul(D, 4);
    const uint64_t s_h = mul(mul(mul(rows, D), n), 4);
    if (s_tok == UINT64_MAX || s_bc == UINT64_MAX || s_A == UINT64_MAX || s_h == UINT64_MAX)
        return LA_ERR_INVALID;
    // one batch row of dt / x / y, and of B / C (with a chunk of padding), must stay below
    // 2 GiB: the kernel addresses a row with 32-bit offsets
    if (mul(T, mul(D, isz)) >= (uint64_t(1) << 31) - 256 ||
        mul(T + 32, mul(n, isz)) >= (uint64_t(1) << 31) - 256)
        return LA_ERR_UNSUPPORTED;
    const bool states = rows * D > 0;
    const bool tokens = states && T > 0;
    if (states && (!A || !h_final)) return LA_ERR_INVALID;
    if (tokens && (!dt || !Bm || !Cm || !x || !y)) return LA_ERR_INVALID;
    // alignment: element alignment for the per-channel token arrays, 16 bytes for the rows
    // of B and C and for A and the states (read as 16-byte pieces)
    const void* a16[] = {Bm, Cm, A, h0, h_final};
    for (const void* ptr : a16)
        if (ptr && !aligned(ptr, 16)) return LA_ERR_INVALID;
    const void* ael[] = {dt, x, y};
    for (const void* ptr : ael)
        if (ptr && !aligned(ptr, isz)) return LA_ERR_INVALID;
    if ((Dskip && !aligned(Dskip, 4)) || (dt_bias && !aligned(dt_bias, 4))) return LA_ERR_INVALID;
    // aliasing: y overlaps nothing; h_final overlaps only h0, and only exactly
    const uint64_t tk = tokens ? 1 : 0;
    const Range rdt = range(dt, s_tok * tk), rx = range(x, s_tok * tk), ry = range(y, s_tok * tk),
                rB = range(Bm, s_bc * tk), rC = range(Cm, s_bc * tk), rA = range(A, s_A),
                rD = range(Dskip, s_ch), rb = range(dt_bias, s_ch), rh0 = range(h0, s_h),
                rh = range(h_final, s_h);
    const Range ins[] = {rdt, rx, rB, rC, rA, rD, rb, rh0, rh};
    for (const Range& r : ins)
        if (overlap(ry, r)) return LA_ERR_INVALID;
    const Range others[] = {rdt, rx, rB, rC, rA, rD, rb};
    for (const Range& r : others)
        if (overlap(rh, r)) return LA_ERR_INVALID;
    if (overlap(rh, rh0) && h_final != h0) return LA_ERR_INVALID;
    if (!states) return LA_OK;

    la::ScanProblem p;
    p.Bt = d->Bt; p.T = d->T; p.D = d->D; p.n = d->n;
    p.io_bf16 = d->io_dtype == LA_BF16;
    p.dt_softplus = d->dt_softplus;
    p.dt = dt; p.Bm = Bm; p.Cm = Cm; p.x = x;
    p.A = A; p.Dskip = Dskip; p.dt_bias = dt_bias; p.h0 = h0;
    p.y = y; p.hT = h_final;
    p.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t err = la::launch_selective_scan(p);
    if (err == hipSuccess) err = hipGetLastError();
    return err == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
