/*
 * Oracle for the causal linear-attention state recurrence: plain, slow, fp64,
 * token by token, on the host.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * links, calls or includes anything from here, and nothing here comes from
 * the GPU library: the two share no code, tables or constants.
 *
 * What it computes, for every (b, h) sequence independently and t = 1..N,
 * with S_0 = S0 (or zeros) and z_0 = z0 (or zeros). The state is key-major,
 * S in R^{d_k x d_v}:
 *
 *  KATH  "Linear / RNN 路线" (walkerchi.com playbook), section 2.1, the
 *        recurrence and the step function; "线性注意力与 SSM" (ailearn), section
 *        02; "状态空间与线性注意力" (wineandchord), section 线性注意力, normalized
 *        output with epsilon:
 *          phi(x) = x + 1 (x > 0), exp(x) (x <= 0)      [ELU with alpha 1, plus 1]
 *          S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t)
 *          o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps)
 *  GLA   "Linear / RNN 路线", section 2.2, boxed equation:
 *          S_t = diag(g_t) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t
 *  GDN   "线性注意力与 SSM", section GDN (gated delta rule), which writes the
 *        state value-major as S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T
 *        and notes that the write equals a correction by v_t - a_t S_{t-1} k_t.
 *        Key-major this is S_t = a_t S_{t-1} + k_t u_t^T with
 *          u_t = b_t (v_t - a_t S_{t-1}^T k_t),   o_t = S_t^T q_t.
 *  SSD   "Linear / RNN 路线", sections 3.6 and 4.1 (Mamba-2): the selective state
 *        space recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t with a scalar
 *        A_t per head, unrolled into linear attention with k = B, v = x, q = C:
 *          S_t = a_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
 *  KDA   "状态空间与线性注意力" (wineandchord), section KDA: a retention per key
 *        channel a_t in (0,1)^{d_k} decays the old state first, then the current
 *        key asks what the decayed state already predicts and writes the error:
 *          Sbar = Diag(a_t) S_{t-1}        [row i scaled by a_{t,i}]
 *          S_t = Sbar + b_t k_t (v_t - Sbar^T k_t)^T,   o_t = S_t^T q_t.
 *
 * Every variant reads the state after the token's update (the post-update
 * read of the output equations on every page).
 *
 * Selective scan (Mamba-1, S6), a separate entry point: "Linear / RNN 路线"
 * section 3.5 (boxed discretisation) and the Mamba2Block forward of section 3.6;
 * "状态空间与线性注意力" sections Selective SSM and 卷积与递推的等价 (the D x_t skip).
 * For each batch row b and channel d, a state h_d in R^{n} (one entry per state
 * dimension), with
 *     Delta_t = softplus(dt_t + bias_d)    (or dt_t itself when no softplus is asked)
 *     h_d <- exp(Delta_t A_{d,i}) h_{d,i} + Delta_t B_{t,i} x_{t,d}     for each i < n
 *     y_{t,d} = sum_i C_{t,i} h_{d,i} + D_d x_{t,d}.
 * B_t and C_t are shared by all channels of a row; A is fixed per (channel, state).
 *
 * Decode is the same per-token body applied once, in place.
 *
 * Backward (the training side of the same prefill; the pages note that training keeps
 * length-N activations and may recompute states): for a loss L with given dL/do_t and
 * dL/dS_final (and dL/dz_final for KATH), the gradients with respect to every input,
 * by reverse-mode differentiation of the token recurrence above, step by step in
 * reverse token order with every state of the forward pass kept. With dS = dL/dS_t
 * (everything after token t, plus the output path q_t dO_t^T added at token t):
 *   GLA   dq = S_t dO; dk = dS v; dv = dS^T k; dg_i = sum_j dS_ij S_{t-1,ij};
 *         dS_{t-1} = diag(g) dS
 *   SSD   as GLA with one decay: da = sum_ij dS_ij S_{t-1,ij}; dS_{t-1} = a dS
 *   GDN   p = S_{t-1}^T k, u = b (v - a p): du = dS^T k; dk = dS u + S_{t-1} dp with
 *         dp = -a b du; dv = b du; db = du . (v - a p); da = <dS, S_{t-1}> - b du . p;
 *         dS_{t-1} = a dS + k dp^T
 *   KDA   Sbar = Diag(a) S_{t-1}, p = Sbar^T k, u = b (v - p): du = dS^T k; dv = b du;
 *         db = du . (v - p); dp = -b du; dSbar = dS + k dp^T; dk = dS u + Sbar dp;
 *         da_i = sum_j dSbar_ij S_{t-1,ij}; dS_{t-1} = Diag(a) dSbar
 *   KATH  o = n / d with n = S_t^T phi(q), d = phi(q) . z_t + eps: dn = dO / d,
 *         dd = -(dO . o) / d; dphi(q) = S_t dn + z_t dd; dS += phi(q) dn^T;
 *         dz += phi(q) dd; dphi(k) = dS v + dz; dv = dS^T phi(k); dS_{t-1} = dS,
 *         dz_{t-1} = dz; dq = dphi(q) phi'(q), dk = dphi(k) phi'(k)
 * and dS0 = dS_0 (dz0 = dz_0).
 *
 * Counters (work accounting, "线性注意力与 SSM" section 02 hand count): each
 * state-update multiply-add and each state-read multiply-add is counted as it
 * is executed.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_KATH = 0, OR_GLA = 1, OR_GDN = 2, OR_KDA = 3, OR_SSD = 4 };

typedef struct {
    uint64_t state_update_macs; /* multiply-adds that write S */
    uint64_t state_read_macs;   /* multiply-adds that read S into an output */
    uint64_t norm_update_adds;  /* additions into z (KATH) */
    uint64_t norm_read_macs;    /* multiply-adds of phi(q)^T z (KATH) */
    uint64_t tokens;            /* token-heads processed */
} oracle_counts;

static double elu_plus_one(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* One token of one head. S: dk x dv (row i = key dim i), z: dk (KATH only).
 * work: scratch of at least 2*dk + dv doubles. */
static void token_step(int variant, int dk, int dv, const double *q, const double *k,
                       const double *v, const double *g, double beta, double eps,
                       double *S, double *z, double *o, double *work, oracle_counts *c)
{
    int i, j;
    if (variant == OR_KATH) {
        double *fq = work, *fk = work + dk;
        double den = 0.0;
        for (i = 0; i < dk; ++i) {
            fq[i] = elu_plus_one(q[i]);
            fk[i] = elu_plus_one(k[i]);
        }
        for (i = 0; i < dk; ++i) {
            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += fk[i] * v[j];
            c->state_update_macs += (uint64_t)dv;
            z[i] += fk[i];
        }
        c->norm_update_adds += (uint64_t)dk;
        for (i = 0; i < dk; ++i) den += fq[i] * z[i];
        c->norm_read_macs += (uint64_t)dk;
        den += eps;
        for (j = 0; j < dv; ++j) {
            double num = 0.0;
            for (i = 0; i < dk; ++i) num += fq[i] * S[(size_t)i * dv + j];
            o[j] = num / den;
        }
        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;
    } else if (variant == OR_GLA) {
        /* row i of S is scaled by the gate of key dim i, then the outer product is added */
        for (i = 0; i < dk; ++i) {
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = g[i] * S[(size_t)i * dv + j] + k[i] * v[j];
            c->state_update_macs += (uint64_t)dv;
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
            o[j] = acc;
        }
        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;
    } else if (variant == OR_SSD) { /* g[0]: the token's scalar decay */
        const double a = g[0];
        for (i = 0; i < dk; ++i) {
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + k[i] * v[j];
            c->state_update_macs += (uint64_t)dv;
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
            o[j] = acc;
        }
        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;
    } else if (variant == OR_KDA) { /* g: retention per key channel */
        double *u = work; /* dv */
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= g[i];   /* decay first */
        for (j = 0; j < dv; ++j) {
            double pred = 0.0; /* (Sbar^T k_t)_j: what the decayed state recalls for k_t */
            for (i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * k[i];
            u[j] = beta * (v[j] - pred);
        }
        for (i = 0; i < dk; ++i) {
            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * u[j];
            c->state_update_macs += (uint64_t)dv;
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
            o[j] = acc;
        }
        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;
    } else { /* OR_GDN: alpha is g[0] */
        double alpha = g[0];
        double *u = work; /* dv */
        for (j = 0; j < dv; ++j) {
            double pred = 0.0; /* (S_{t-1}^T k_t)_j: what the old state recalls for k_t */
            for (i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * k[i];
            u[j] = beta * (v[j] - alpha * pred);
        }
        for (i = 0; i < dk; ++i) {
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = alpha * S[(size_t)i * dv + j] + k[i] * u[j];
            c->state_update_macs += (uint64_t)dv;
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
            o[j] = acc;
        }
        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;
    }
    c->tokens += 1;
}

static int check_args(int variant, int B, int H, int N, int dk, int dv)
{
    if (variant < OR_KATH || variant > OR_SSD) return 1;
    if (B < 0 || H < 0 || N < 0 || dk < 1 || dv < 1) return 1;
    return 0;
}

/*
 * Whole-sequence forward.
 *   q, k: [B,H,N,dk]   v: [B,H,N,dv]
 *   g:    GLA [B,H,N,dk]; GDN alpha [B,H,N]; KDA alpha [B,H,N,dk]; SSD decay [B,H,N];
 *         KATH unused (may be NULL)
 *   beta: GDN and KDA [B,H,N]; otherwise unused
 *   S0:   [B,H,dk,dv] or NULL (zeros);   z0: [B,H,dk] or NULL (zeros), KATH only
 *   o:    [B,H,N,dv] out;  S: [B,H,dk,dv] out (final state);  z: [B,H,dk] out (KATH, may be NULL otherwise)
 *   counts: optional, summed over all sequences.
 *   threads: OpenMP threads over the B*H sequences (<= 0: runtime default).
 * Returns 0, or 1 on a bad argument.
 */
int oracle_prefill(int variant, int B, int H, int N, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   const double *S0, const double *z0, double eps,
                   double *o, double *S, double *z, int threads, oracle_counts *counts)
{
    long long seq, nseq;
    oracle_counts total;
    if (check_args(variant, B, H, N, dk, dv)) return 1;
    if (variant == OR_KATH && z == NULL) return 1;
    if (variant != OR_KATH && g == NULL) return 1;
    if ((variant == OR_GDN || variant == OR_KDA) && beta == NULL) return 1;
    memset(&total, 0, sizeof(total));
    nseq = (long long)B * H;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        oracle_counts c;
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * dk + dv));
        memset(&c, 0, sizeof(c));
#pragma omp for schedule(dynamic, 1)
        for (seq = 0; seq < nseq; ++seq) {
            double *Sh = S + (size_t)seq * dk * dv;
            double *zh = (variant == OR_KATH) ? z + (size_t)seq * dk : NULL;
            int t;
            if (S0) memcpy(Sh, S0 + (size_t)seq * dk * dv, sizeof(double) * (size_t)dk * dv);
            else memset(Sh, 0, sizeof(double) * (size_t)dk * dv);
            if (zh) {
                if (z0) memcpy(zh, z0 + (size_t)seq * dk, sizeof(double) * (size_t)dk);
                else memset(zh, 0, sizeof(double) * (size_t)dk);
            }
            for (t = 0; t < N; ++t) {
                size_t tok = (size_t)seq * N + t;
                const double *gt = NULL;
                double bt = 0.0;
                if (variant == OR_GLA) gt = g + tok * dk;
                if (variant == OR_GDN) { gt = g + tok; bt = beta[tok]; }
                if (variant == OR_KDA) { gt = g + tok * dk; bt = beta[tok]; }
                if (variant == OR_SSD) gt = g + tok;
                token_step(variant, dk, dv, q + tok * dk, k + tok * dk, v + tok * dv, gt, bt,
                           eps, Sh, zh, o + tok * dv, work, &c);
            }
        }
#pragma omp critical
        {
            total.state_update_macs += c.state_update_macs;
            total.state_read_macs += c.state_read_macs;
            total.norm_update_adds += c.norm_update_adds;
            total.norm_read_macs += c.norm_read_macs;
            total.tokens += c.tokens;
        }
        free(work);
    }
    if (counts) *counts = total;
    return 0;
}

/*
 * One decode step for B*H independent states, in place.
 *   q, k: [B,H,dk]  v: [B,H,dv]  g: GLA [B,H,dk] / GDN alpha [B,H] / KDA alpha [B,H,dk] /
 *   SSD decay [B,H]
 *   beta: GDN and KDA [B,H]
 *   S: [B,H,dk,dv] in/out;  z: [B,H,dk] in/out (KATH);  o: [B,H,dv] out.
 */
int oracle_decode_step(int variant, int B, int H, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta, double eps,
                       double *S, double *z, double *o, int threads)
{
    long long seq, nseq;
    if (check_args(variant, B, H, 1, dk, dv)) return 1;
    if (variant == OR_KATH && z == NULL) return 1;
    if (variant != OR_KATH && g == NULL) return 1;
    if ((variant == OR_GDN || variant == OR_KDA) && beta == NULL) return 1;
    nseq = (long long)B * H;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        oracle_counts c;
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * dk + dv));
        memset(&c, 0, sizeof(c));
#pragma omp for schedule(static)
        for (seq = 0; seq < nseq; ++seq) {
            const double *gt = NULL;
            double bt = 0.0;
            if (variant == OR_GLA) gt = g + (size_t)seq * dk;
            if (variant == OR_GDN) { gt = g + seq; bt = beta[seq]; }
            if (variant == OR_KDA) { gt = g + (size_t)seq * dk; bt = beta[seq]; }
            if (variant == OR_SSD) gt = g + seq;
            token_step(variant, dk, dv, q + (size_t)seq * dk, k + (size_t)seq * dk,
                       v + (size_t)seq * dv, gt, bt, eps, S + (size_t)seq * dk * dv,
                       variant == OR_KATH ? z + (size_t)seq * dk : NULL,
                       o + (size_t)seq * dv, work, &c);
        }
        free(work);
    }
    return 0;
}

static double softplus(double u) { return u > 30.0 ? u : log1p(exp(u)); }

/*
 * Selective scan over whole sequences (see the header for the equations).
 *   dt, x: [Bt,T,D]   A: [D,n]   Bm, Cm: [Bt,T,n]
 *   Dskip: [D] or NULL (no skip)   dt_bias: [D] or NULL (zero)   dt_softplus: 0 or 1
 *   h0: [Bt,D,n] or NULL (zeros)
 *   y: [Bt,T,D] out;   hT: [Bt,D,n] out (final state).
 * Returns 0, or 1 on a bad argument.
 */
int oracle_selective_scan(int Bt, int T, int D, int n, const double *dt, const double *A,
                          const double *Bm, const double *Cm, const double *x,
                          const double *Dskip, const double *dt_bias, int dt_softplus,
                          const double *h0, double *y, double *hT, int threads)
{
    long long row;
    if (Bt < 0 || T < 0 || D < 1 || n < 1 || dt == NULL || A == NULL || Bm == NULL ||
        Cm == NULL || x == NULL || y == NULL || hT == NULL)
        return 1;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (row = 0; row < (long long)Bt * D; ++row) {
        const long long b = row / D;
        const int d = (int)(row % D);
        double *h = hT + (size_t)row * n;
        int t, i;
        if (h0) memcpy(h, h0 + (size_t)row * n, sizeof(double) * (size_t)n);
        else memset(h, 0, sizeof(double) * (size_t)n);
        for (t = 0; t < T; ++t) {
            const size_t tok = (size_t)b * T + t;
            const double xt = x[tok * D + d];
            double delta = dt[tok * D + d] + (dt_bias ? dt_bias[d] : 0.0);
            double acc = 0.0;
            if (dt_softplus) delta = softplus(delta);
            for (i = 0; i < n; ++i) {
                const double abar = exp(delta * A[(size_t)d * n + i]);
                const double bbar = delta * Bm[tok * n + i];
                h[i] = abar * h[i] + bbar * xt;
            }
            for (i = 0; i < n; ++i) acc += Cm[tok * n + i] * h[i];
            y[tok * D + d] = acc + (Dskip ? Dskip[d] * xt : 0.0);
        }
    }
    return 0;
}

/* Backward of one token: S_prev / z_prev the state before the token, S_post / z_post
 * after it; dS / dz hold dL/dS_post (without this token's output path) on entry and
 * dL/dS_prev on return. work: at least 2 dk + 3 dv doubles. */
static void token_backward(int variant, int dk, int dv, const double *q, const double *k,
                           const double *v, const double *g, double beta, double eps,
                           const double *S_prev, const double *S_post, const double *z_post,
                           const double *dO, double *dS, double *dz, double *dq, double *dk_,
                           double *dv_, double *dg, double *dbeta, double *work)
{
    int i, j;
    if (variant == OR_KATH) {
        double *fq = work, *fk = work + dk, *dn = work + 2 * dk, *o = work + 2 * dk + dv;
        double den = eps, dd = 0.0;
        for (i = 0; i < dk; ++i) {
            fq[i] = elu_plus_one(q[i]);
            fk[i] = elu_plus_one(k[i]);
            den += fq[i] * z_post[i];
        }
        for (j = 0; j < dv; ++j) {
            double num = 0.0;
            for (i = 0; i < dk; ++i) num += fq[i] * S_post[(size_t)i * dv + j];
            o[j] = num / den;
            dn[j] = dO[j] / den;
            dd -= dO[j] * o[j] / den;
        }
        for (i = 0; i < dk; ++i) {
            double dfq = z_post[i] * dd;
            for (j = 0; j < dv; ++j) dfq += S_post[(size_t)i * dv + j] * dn[j];
            dq[i] = dfq * (q[i] > 0.0 ? 1.0 : exp(q[i]));
            for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += fq[i] * dn[j];
            dz[i] += fq[i] * dd;
        }
        for (i = 0; i < dk; ++i) {
            double dfk = dz[i];
            for (j = 0; j < dv; ++j) dfk += dS[(size_t)i * dv + j] * v[j];
            dk_[i] = dfk * (k[i] > 0.0 ? 1.0 : exp(k[i]));
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += dS[(size_t)i * dv + j] * fk[i];
            dv_[j] = acc;
        }
        return;   /* dS and dz pass through unchanged: S_t = S_{t-1} + ..., z_t = z_{t-1} + ... */
    }
    /* the output read o = S_post^T q */
    for (i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (j = 0; j < dv; ++j) acc += S_post[(size_t)i * dv + j] * dO[j];
        dq[i] = acc;
        for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += q[i] * dO[j];
    }
    if (variant == OR_GLA || variant == OR_SSD) {
        double dsum = 0.0;
        for (i = 0; i < dk; ++i) {
            double acc = 0.0, gi = variant == OR_GLA ? g[i] : g[0];
            for (j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * v[j];
            dk_[i] = acc;
            acc = 0.0;
            for (j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * S_prev[(size_t)i * dv + j];
            if (variant == OR_GLA) dg[i] = acc;
            else dsum += acc;
            (void)gi;
        }
        if (variant == OR_SSD) dg[0] = dsum;
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += dS[(size_t)i * dv + j] * k[i];
            dv_[j] = acc;
        }
        for (i = 0; i < dk; ++i) {
            const double gi = variant == OR_GLA ? g[i] : g[0];
            for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= gi;
        }
        return;
    }
    {
        /* delta rule: p = Sdec^T k with Sdec = alpha S_prev (GDN: alpha scalar; KDA:
         * Diag(alpha) S_prev), u = beta (v - p); S_post = Sdec + k u^T */
        double *u = work, *du = work + dv, *dp = work + 2 * dv, *p = work + 3 * dv;
        double da = 0.0, db = 0.0;
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) {
                const double ai = variant == OR_GDN ? g[0] : g[i];
                acc += ai * S_prev[(size_t)i * dv + j] * k[i];
            }
            p[j] = acc;
            u[j] = beta * (v[j] - acc);
        }
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i) acc += dS[(size_t)i * dv + j] * k[i];
            du[j] = acc;
            dv_[j] = beta * acc;
            db += acc * (v[j] - p[j]);
            dp[j] = -beta * acc;
        }
        *dbeta = db;
        for (i = 0; i < dk; ++i) {
            const double ai = variant == OR_GDN ? g[0] : g[i];
            double acc = 0.0, accp = 0.0;
            for (j = 0; j < dv; ++j) {
                acc += dS[(size_t)i * dv + j] * u[j];
                accp += ai * S_prev[(size_t)i * dv + j] * dp[j];
            }
            dk_[i] = acc + accp;
        }
        /* dSdec = dS + k dp^T; dalpha from Sdec = alpha S_prev; dS_prev = alpha dSdec */
        for (i = 0; i < dk; ++i) {
            const double ai = variant == OR_GDN ? g[0] : g[i];
            double acc = 0.0;
            for (j = 0; j < dv; ++j) {
                const double dsd = dS[(size_t)i * dv + j] + k[i] * dp[j];
                acc += dsd * S_prev[(size_t)i * dv + j];
                dS[(size_t)i * dv + j] = ai * dsd;
            }
            if (variant == OR_GDN) da += acc;
            else dg[i] = acc;
        }
        if (variant == OR_GDN) dg[0] = da;
    }
}

/*
 * Whole-sequence backward (reverse-mode derivative of oracle_prefill).
 * Inputs as for oracle_prefill, plus
 *   dO: [B,H,N,dv]; dS_final: [B,H,dk,dv] or NULL (zero); dz_final: [B,H,dk] or NULL (KATH)
 * Outputs (all required unless noted):
 *   dq, dk: [B,H,N,dk]; dv: [B,H,N,dv]; dg: shaped like g (NULL for KATH);
 *   dbeta: [B,H,N] (GDN, KDA; NULL otherwise); dS0: [B,H,dk,dv]; dz0: [B,H,dk] (KATH)
 * Returns 0, or 1 on a bad argument.
 */
int oracle_prefill_backward(int variant, int B, int H, int N, int dk, int dv,
                            const double *q, const double *k, const double *v,
                            const double *g, const double *beta,
                            const double *S0, const double *z0, double eps,
                            const double *dO, const double *dS_final, const double *dz_final,
                            double *dq, double *dk_, double *dv_, double *dg, double *dbeta,
                            double *dS0, double *dz0, int threads)
{
    long long seq, nseq;
    const int gw = (variant == OR_GLA || variant == OR_KDA) ? dk : 1;
    if (check_args(variant, B, H, N, dk, dv)) return 1;
    if (!dO || !dq || !dk_ || !dv_ || !dS0) return 1;
    if (variant != OR_KATH && (!g || !dg)) return 1;
    if ((variant == OR_GDN || variant == OR_KDA) && (!beta || !dbeta)) return 1;
    if (variant == OR_KATH && !dz0) return 1;
    nseq = (long long)B * H;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        oracle_counts c;
        const size_t SS = (size_t)dk * dv;
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * dk + 4 * dv + 8));
        double *states = (double *)malloc(sizeof(double) * SS * (size_t)(N + 1));
        double *zs = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)(N + 1));
        double *ot = (double *)malloc(sizeof(double) * (size_t)(dv + 1));
        double *dS = (double *)malloc(sizeof(double) * SS);
        double *dz = (double *)malloc(sizeof(double) * (size_t)dk);
        memset(&c, 0, sizeof(c));
#pragma omp for schedule(dynamic, 1)
        for (seq = 0; seq < nseq; ++seq) {
            int t;
            if (S0) memcpy(states, S0 + (size_t)seq * SS, sizeof(double) * SS);
            else memset(states, 0, sizeof(double) * SS);
            if (variant == OR_KATH && z0) memcpy(zs, z0 + (size_t)seq * dk, sizeof(double) * (size_t)dk);
            else memset(zs, 0, sizeof(double) * (size_t)dk);
            /* forward, keeping every state */
            for (t = 0; t < N; ++t) {
                const size_t tok = (size_t)seq * N + t;
                const double *gt = g ? g + tok * gw : NULL;
                const double bt = beta ? beta[tok] : 0.0;
                memcpy(states + SS * (size_t)(t + 1), states + SS * (size_t)t, sizeof(double) * SS);
                memcpy(zs + (size_t)dk * (t + 1), zs + (size_t)dk * t, sizeof(double) * (size_t)dk);
                token_step(variant, dk, dv, q + tok * dk, k + tok * dk, v + tok * dv, gt, bt, eps,
                           states + SS * (size_t)(t + 1), zs + (size_t)dk * (t + 1), ot, work, &c);
            }
            /* backward */
            if (dS_final) memcpy(dS, dS_final + (size_t)seq * SS, sizeof(double) * SS);
            else memset(dS, 0, sizeof(double) * SS);
            if (variant == OR_KATH && dz_final) memcpy(dz, dz_final + (size_t)seq * dk, sizeof(double) * (size_t)dk);
            else memset(dz, 0, sizeof(double) * (size_t)dk);
            for (t = N - 1; t >= 0; --t) {
                const size_t tok = (size_t)seq * N + t;
                const double *gt = g ? g + tok * gw : NULL;
                const double bt = beta ? beta[tok] : 0.0;
                double dbt = 0.0;
                token_backward(variant, dk, dv, q + tok * dk, k + tok * dk, v + tok * dv, gt, bt, eps,
                               states + SS * (size_t)t, states + SS * (size_t)(t + 1),
                               zs + (size_t)dk * (t + 1), dO + tok * dv, dS, dz, dq + tok * dk,
                               dk_ + tok * dk, dv_ + tok * dv, dg ? dg + tok * gw : NULL, &dbt, work);
                if (dbeta) dbeta[tok] = dbt;
            }
            memcpy(dS0 + (size_t)seq * SS, dS, sizeof(double) * SS);
            if (variant == OR_KATH) memcpy(dz0 + (size_t)seq * dk, dz, sizeof(double) * (size_t)dk);
        }
        free(work); free(states); free(zs); free(ot); free(dS); free(dz);
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
