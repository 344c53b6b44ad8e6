/*
 * linattn.h -- C ABI of the causal linear-attention state recurrence on MI355X (gfx950).
 *
 * The library computes, for every (b, h) sequence independently, the recurrence
 * over a key-major matrix state S in R^{d_k x d_v} (row i belongs to key dim i):
 *
 *   LA_KATH  normalized Katharopoulos linear attention ("Linear / RNN 路线",
 *            section 2.1; "线性注意力与 SSM", section 02; "状态空间与线性注意力",
 *            section 线性注意力):
 *              phi(x) = ELU(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0), on q and k only
 *              S_t = S_{t-1} + phi(k_t) v_t^T,   z_t = z_{t-1} + phi(k_t)
 *              o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps)
 *   LA_GLA   gated linear attention with a per-key-dim forget gate ("Linear / RNN 路线",
 *            section 2.2): S_t = diag(g_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *   LA_GDN   gated delta rule ("线性注意力与 SSM", section GDN), stored key-major (the
 *            transpose of the page's value-major form, identical since I - b k k^T is
 *            symmetric): S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T, that is
 *              u_t = b_t (v_t - a_t S_{t-1}^T k_t),  S_t = a_t S_{t-1} + k_t u_t^T,
 *              o_t = S_t^T q_t
 *   LA_KDA   Kimi Delta Attention ("状态空间与线性注意力", section KDA): a retention
 *            per key channel decays the old state first, then the delta write reads
 *            the decayed state:  Sbar = Diag(a_t) S_{t-1},
 *              S_t = Sbar + b_t k_t (v_t - Sbar^T k_t)^T,   o_t = S_t^T q_t
 *   LA_SSD   Mamba-2's structured state space duality ("Linear / RNN 路线", sections 3.6
 *            and 4.1): the selective SSM h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t with
 *            one scalar decay per token and head is linear attention with k = B,
 *            v = x (already scaled by the step), q = C:
 *              S_t = a_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *            d_k is the state size and d_v the head dim; the caller passes a_t =
 *            exp(Delta_t A_h). (The per-channel Mamba-1 scan is la_selective_scan.)
 *
 * Every variant reads the state after the token's update. Prefill runs the
 * recurrence over N tokens with the chunkwise-parallel method (quadratic, causally
 * masked work inside a chunk, the state carried between chunks); decode applies one
 * token in place. Chunk size and tiling are internal and do not change the result
 * beyond rounding.
 *
 * Layouts (all dense, row-major, no strides; "io" = io_dtype, "gate" = gate_dtype):
 *   q, k     [B, H, N, d_k]  io        v, o  [B, H, N, d_v]  io
 *   g        LA_GLA: [B, H, N, d_k] gate, values in (0, 1]
 *            LA_GDN: alpha [B, H, N] gate, values in (0, 1]
 *            LA_KDA: alpha [B, H, N, d_k] gate (retention per key channel), in (0, 1]
 *            LA_SSD: a [B, H, N] decay, values in (0, 1]
 *   beta     LA_GDN, LA_KDA: [B, H, N] gate, values in [0, 1]
 *   S0, S    [B, H, d_k, d_v] fp32 (key-major)
 *   z0, z    [B, H, d_k] fp32 (LA_KATH only)
 * For decode N = 1 and the token arrays are [B, H, d] (respectively [B, H]).
 * The output o is rounded to nearest even from fp32 when io is bf16.
 *
 * Ownership and threading: the caller allocates every buffer in device memory and
 * passes plain device pointers and a hipStream_t (NULL = the default stream). The
 * library never allocates, frees or synchronizes; calls only enqueue work on the
 * given stream and return. It keeps no mutable global state and is re-entrant, apart
 * from the one device array per GPU that la_prefill_noalloc uses as its workspace.
 *
 * Errors: every entry point validates all arguments first. On any error it returns
 * a nonzero status, enqueues nothing and touches no output. No exception crosses
 * the ABI. LA_ERR_HIP means a kernel launch failed (hipGetLastError); work enqueued
 * before the failing launch of the same call may have run.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 1

/* status codes */
enum {
    LA_OK = 0,
    LA_ERR_INVALID = 1,      /* null required pointer, bad enum, negative size, misaligned
                                pointer (16 bytes for q, k, v, o, GLA g, S and z; element
                                alignment for GDN alpha, SSD a and GDN / KDA beta; 256 bytes for the
                                workspace), overlap of an output with any other buffer,
                                gate passed / missing for the variant, N != 1 for decode */
    LA_ERR_UNSUPPORTED = 2,  /* d_k or d_v not in {16, 32, 64, 128}, or a requested path /
                                chunk size that this shape or dtype does not support */
    LA_ERR_HIP = 3,          /* a kernel launch failed */
    LA_ERR_WORKSPACE = 4     /* workspace missing or smaller than la_prefill_workspace_size */
};

/* variants */
enum { LA_KATH = 0, LA_GLA = 1, LA_GDN = 2, LA_KDA = 3, LA_SSD = 4 };

/* storage dtypes */
enum { LA_F32 = 0, LA_BF16 = 1 };

/* kernel path selection (semantics never depend on it) */
enum {
    LA_PATH_AUTO = 0, /* bf16 MFMA kernels where the shape allows, else the fp32 VALU kernels */
    LA_PATH_VALU = 1, /* fp32 arithmetic on the vector ALUs (chunk 16) */
    LA_PATH_MFMA = 2  /* bf16 matrix cores with fp32 accumulation and fp32 state (chunk 64);
                         needs bf16 q / k / v and d_k = 128 */
};

typedef struct la_desc {
    int32_t B, H, N;      /* batch, heads, tokens per sequence (N = 1 for decode) */
    int32_t dk, dv;       /* key and value dims, each in {16, 32, 64, 128} */
    int32_t variant;      /* LA_KATH | LA_GLA | LA_GDN | LA_KDA | LA_SSD */
    int32_t io_dtype;     /* LA_F32 | LA_BF16: q, k, v, o */
    int32_t gate_dtype;   /* LA_F32 | LA_BF16: g / alpha, beta (ignored for LA_KATH) */
    float eps;            /* LA_KATH denominator epsilon, finite and >= 0 */
    int32_t path;         /* LA_PATH_* */
    int32_t chunk;        /* 0 = the path's chunk size; otherwise it must equal it */
    int32_t segments;     /* 0 = automatic. LA_KATH / LA_GLA / LA_SSD on the MFMA path split each
                             sequence into this many segments that run in parallel and
                             are joined by a scan of their state summaries */
} la_desc;

/* Bytes of device workspace la_prefill needs for this descriptor (0 if none).
 * Returns LA_OK and writes *bytes, or an error status for an invalid descriptor. */
int la_prefill_workspace_size(const la_desc* d, size_t* bytes);

/* Whole-sequence forward.
 *   q, k, v, g, beta   inputs as laid out above; g and beta must be NULL when the
 *                      variant does not take them.
 *   S0, z0             initial state, or NULL for zeros; z0 must be NULL unless LA_KATH.
 *   o                  output [B, H, N, d_v] io; must not overlap any other buffer.
 *   S_final            final state [B, H, d_k, d_v] fp32, required. It may be the same
 *                      pointer as S0 (in-place carry) but must not otherwise overlap.
 *   z_final            final normalizer [B, H, d_k] fp32: required for LA_KATH (may equal
 *                      z0), NULL otherwise.
 *   workspace          device scratch of at least la_prefill_workspace_size bytes,
 *                      256-byte aligned, owned by the caller, not read as input; NULL
 *                      when the size is 0. Contents on return are unspecified.
 *   stream             hipStream_t.
 * N = 0 is accepted: o is untouched and S_final / z_final receive S0 / z0 (or zeros).
 * B * H = 0 is accepted and does nothing. */
int la_prefill(const la_desc* d, const void* q, const void* k, const void* v,
               const void* g, const void* beta, const float* S0, const float* z0,
               void* o, float* S_final, float* z_final,
               void* workspace, size_t workspace_bytes, void* stream);

/* Variable-length batch. The implementation checklist of "状态空间与线性注意力" asks
 * whether sequence resets and padding positions update the state, and its failure modes
 * name state carried across request boundaries; here sequences are packed (no padding
 * is stored) and the state restarts at every boundary. nseq
 * sequences concatenated along the token axis of one [1, H, N, d] layout. Sequence s
 * occupies tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of every head, starts from
 * S0[s] (z0[s]) or zeros, and ends in S_final[s] (z_final[s]): the state resets at
 * every boundary, and the result for each sequence is that of la_prefill on it alone.
 *   d->B must be 1; d->N is the total token count; q, k, v, o, g, beta as in la_prefill
 *   with B = 1.
 *   cu_seqlens   device int32 [nseq + 1], nondecreasing, cu_seqlens[0] = 0,
 *                cu_seqlens[nseq] <= N; 4-byte aligned. Read only by the kernels: the
 *                host does not check its contents. Offsets outside [0, N] are clamped
 *                and lengths capped at max_seqlen, so no access leaves the buffers, but
 *                the results for such values are unspecified.
 *   max_seqlen   host value >= every sequence length, <= N; sizes the launch and the
 *                workspace.
 *   S0, S_final  [nseq, H, d_k, d_v] fp32; z0, z_final [nseq, H, d_k] fp32 (LA_KATH).
 *   workspace    at least la_prefill_varlen_workspace_size bytes (as for la_prefill).
 * Errors as for la_prefill; nseq = 0 does nothing. */
int la_prefill_varlen_workspace_size(const la_desc* d, int32_t nseq, int32_t max_seqlen,
                                     size_t* bytes);
int la_prefill_varlen(const la_desc* d, int32_t nseq, const int32_t* cu_seqlens,
                      int32_t max_seqlen, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S0, const float* z0, void* o,
                      float* S_final, float* z_final, void* workspace, size_t workspace_bytes,
                      void* stream);

/* One decode step, in place: the per-token step of "Linear / RNN 路线", section 2.1,
 * applied to the carried state; the decode carry of "线性注意力与 SSM", section 01, is
 * the final recurrent state only, so the cost of a step does not depend on how many
 * tokens came before.
 *   d->N must be 1. q, k [B, H, d_k]; v [B, H, d_v]; g (GLA [B, H, d_k], GDN alpha
 *   [B, H], KDA alpha [B, H, d_k]); beta (GDN / KDA [B, H]); S [B, H, d_k, d_v] fp32
 *   read and overwritten;
 *   z [B, H, d_k] fp32 read and overwritten (LA_KATH, NULL otherwise);
 *   o [B, H, d_v] io written. o must not overlap S, z or any input. */
int la_decode_step(const la_desc* d, const void* q, const void* k, const void* v,
                   const void* g, const void* beta, float* S, float* z, void* o,
                   void* stream);

/* Backward of la_prefill: the gradients of every input for a loss with dL/do = dO,
 * dL/dS_final = dS_final and, for KATH, dL/dz_final = dz_final (NULL: zero), by
 * reverse-mode differentiation of the recurrence (the training side of the same prefill;
 * "线性注意力与 SSM" notes that training keeps length-N activations and may recompute
 * states, which this does: the chunk-entering states, and for KATH the forward's
 * denominators, are recomputed into the workspace). Every variant is taken. SSD with bf16
 * io, d_k = 128 and d_v = 64 runs on the matrix cores (bf16 operands, fp32 accumulation,
 * chunk 64) for d->path LA_PATH_AUTO or LA_PATH_MFMA; every other case (and
 * LA_PATH_VALU) runs in fp32 on the vector ALUs (chunk 16) for any supported d_k, d_v and
 * either io dtype. LA_PATH_MFMA for a shape the matrix cores do not take is
 * LA_ERR_UNSUPPORTED; a chunk other than 0 or the path's is LA_ERR_UNSUPPORTED. The gate
 * gradients (dg, GDN's dalpha, KDA's per-key-dim dalpha) are formed directly from pairs of
 * token states, not through log-gate sums, so tiny gates keep fp32 accuracy.
 *   q, k, v, g, beta, S0, z0   the forward's inputs (S0, z0 may be NULL; g is NULL for
 *                      KATH, beta for every variant but GDN and KDA, z0 for all but KATH)
 *   dO                 [B, H, N, d_v] io
 *   dq, dk             [B, H, N, d_k] io, written;  dv [B, H, N, d_v] io, written
 *   dg                 shaped like g (gate dtype), written: dL/dg for the gate as given
 *                      (NULL for KATH)
 *   dbeta              [B, H, N] gate dtype, written (GDN, KDA; NULL otherwise)
 *   dS0                [B, H, d_k, d_v] fp32, written (also when S0 is NULL: the gradient
 *                      with respect to the zero initial state)
 *   dz_final, dz0      KATH: [B, H, d_k] fp32 (dz_final may be NULL), dz0 written; NULL
 *                      for the other variants
 *   workspace          at least la_prefill_backward_workspace_size bytes, 256-byte aligned
 * Outputs overlap nothing (no input, no other output, not the workspace). Alignment as for
 * la_prefill (dq, dk as q; dv and dO as v; dg as g; dbeta as beta; dz0, dz_final 16
 * bytes). Errors as for la_prefill. */
int la_prefill_backward_workspace_size(const la_desc* d, size_t* bytes);
int la_prefill_backward(const la_desc* d, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const float* S0, const float* z0,
                        const void* dO, const float* dS_final, const float* dz_final, void* dq,
                        void* dk, void* dv, void* dg, void* dbeta, float* dS0, float* dz0,
                        void* workspace, size_t workspace_bytes, void* stream);

/* la_prefill without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as la_prefill, minus the workspace: the workspace
 * comes from one fixed array of LA_NOALLOC_SCRATCH_BYTES in the library's device code,
 * one copy per GPU, held until the process ends. The call allocates nothing and calls no
 * allocating routine.
 *   A descriptor whose la_prefill_workspace_size exceeds LA_NOALLOC_SCRATCH_BYTES is
 *   rejected with LA_ERR_WORKSPACE before anything is enqueued.
 *   The stream must belong to the current device (LA_ERR_INVALID otherwise); NULL is the
 *   current device's default stream.
 *   Every call on one GPU uses that GPU's one array: calls whose work overlaps in time on
 *   one GPU (different streams, or host threads) race on it and must be serialised by the
 *   caller. Calls in order on one stream are safe; nothing in the array carries over from
 *   one call to the next. */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
int la_prefill_noalloc(const la_desc* d, const void* q, const void* k, const void* v,
                       const void* g, const void* beta, const float* S0, const float* z0,
                       void* o, float* S_final, float* z_final, void* stream);

/* ------------------------------------------------------------------------------------
 * Selective scan (Mamba-1 / S6): "Linear / RNN 路线", section 3.5 (the boxed
 * discretisation Abar_t = exp(Delta_t A), Bbar_t = Delta_t B_t with Delta, B and C
 * computed from the input) and the simplified block's forward in section 3.6;
 * "状态空间与线性注意力", sections Selective SSM (h_t = Abar_t h_{t-1} + Bbar_t x_t,
 * y_t = C_t h_t) and 卷积与递推的等价 (the D x_t skip). Every batch row b and channel d
 * carries a state h_{b,d} in R^n, one decay rate per (channel, state entry):
 *   Delta = softplus(dt_{t,d} + dt_bias_d)      (dt_softplus = 1; dt + dt_bias when 0)
 *   h_{d,i} <- exp(Delta A_{d,i}) h_{d,i} + Delta B_{t,i} x_{t,d}      (i < n)
 *   y_{t,d}  = sum_i C_{t,i} h_{d,i} + D_d x_{t,d}
 * B_t and C_t are shared by all channels of a row. The arithmetic is fp32 with an fp32
 * state; exp is the hardware base-2 exponential of Delta A log2(e).
 * ------------------------------------------------------------------------------------ */
typedef struct la_scan_desc {
    int32_t Bt;           /* batch rows */
    int32_t T;            /* tokens per row; T = 1 with h_final == h0 is one decode step */
    int32_t D;            /* channels */
    int32_t n;            /* state entries per channel: 16, 32, 64 or 128 */
    int32_t io_dtype;     /* LA_F32 | LA_BF16: dt, B, C, x and y */
    int32_t dt_softplus;  /* 1: Delta = softplus(dt + dt_bias); 0: Delta = dt + dt_bias */
} la_scan_desc;

/* Whole-sequence selective scan.
 *   dt, x     [Bt, T, D] io            A        [D, n] fp32 (negative for a decay)
 *   Bm, Cm    [Bt, T, n] io            Dskip    [D] fp32, or NULL for no skip
 *   dt_bias   [D] fp32, or NULL (zero) h0       [Bt, D, n] fp32, or NULL (zeros)
 *   y         [Bt, T, D] io, written (bf16: rounded to nearest even from fp32)
 *   h_final   [Bt, D, n] fp32, written; may be the same pointer as h0 (in place) but
 *             must not otherwise overlap anything; y must not overlap any buffer.
 * Alignment: Bm, Cm, A, h0 and h_final 16 bytes; dt, x and y their element size; Dskip
 * and dt_bias 4 bytes. All buffers are device memory owned by the caller; the call only
 * enqueues work on the stream. T = 0 copies h0 (or zeros) to h_final; Bt * D = 0 does
 * nothing. Errors as for la_prefill: LA_ERR_INVALID (null required pointer, bad dtype or
 * flag, negative size, misalignment, overlap), LA_ERR_UNSUPPORTED (n, or one batch row of
 * dt / x / y or of B / C reaching 2 GiB), LA_ERR_HIP. */
int la_selective_scan(const la_scan_desc* d, const void* dt, const float* A, const void* Bm,
                      const void* Cm, const void* x, const float* Dskip, const float* dt_bias,
                      const float* h0, void* y, float* h_final, void* stream);

/* The in-place streaming ceiling of a decode step. Decode is a read-modify-write of the
 * carried state and nothing else of size ("线性注意力与 SSM", sections 01 and 02: its cost
 * follows the state's size), so the fastest plain in-place pass over the same bytes bounds
 * it. This call makes that pass: x[i] <- a * x[i] for i < n, fp32, in place, every element
 * read once and written once with 16-byte accesses (a grid of two workgroups per compute
 * unit walks 16 KiB tiles, loading the next tile before storing the current one).
 *   x   n floats of device memory owned by the caller, 16-byte aligned; n a multiple of 4.
 * Only enqueues work on the stream. Errors: LA_ERR_INVALID (x NULL with n > 0, n not a
 * multiple of 4, x misaligned), LA_ERR_HIP. n = 0 does nothing. */
int la_stream_rmw(float* x, uint64_t n, float a, void* stream);

/* Static description of a status code (never NULL). */
const char* la_status_str(int status);

/* LA_ABI_VERSION of the built library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
