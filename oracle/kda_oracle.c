/*
 * KDA reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential fp64 evaluation of Kimi Delta Attention (KDA), the
 * channel-wise gated delta rule.  Only the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load this code; the GPU library
 * never links or calls it, and it shares no source with it.
 *
 * Sources (cited by page title and section):
 *  [A] "Kimi K3 -- the architecture and infrastructure, explained",
 *      section "How the delta rule actually works": the delta-rule update
 *      S <- S - beta (S k - v) k^T with the recall v_hat = S k (S there is
 *      d_v x d_k; here it is stored transposed, d_k x d_v).
 *  [B] same page, section "Kimi Delta Attention: the load-bearing choice":
 *      the gate is channel-wise, each state dimension decays on its own.
 *  [C] "Inside Kimi K3: How Moonshot AI Built the Largest Open-Source Model",
 *      section "Technical Details": per head 128 forgetting dials, beta is the
 *      writing strength, alpha the forgetting factor, "erase then write".
 *  [D] marketersindex.com Kimi K3 article, section "Architectural Innovations:
 *      Kimi Delta Attention (KDA)": recall / compare / correct, and channels
 *      (rows of the memory state) decaying at different speeds.
 *
 * What it computes, for every sequence n and head h independently:
 *     S <- initial state (or zeros)                       d_k x d_v
 *     for each token t of the sequence, in order:
 *       a_i = exp(log_alpha[t,h,i])        forgetting factor per channel [B][C]
 *       S   = Diag(a) S                    channel-wise decay, rows = channels [D]
 *       p   = S^T k_t                      recall [A][D]
 *       u   = beta_t (v_t - p)             compare, scaled by the write strength [A][C]
 *       S   = S + k_t u^T                  correct [A][D]
 *       o_t = S^T q_t                      read-out from the updated state
 *     final state <- S
 * Optionally also, per token, the magnitude of the read-out's terms,
 * m_t = |S_t|^T |q_t| (elementwise absolute values): the scale against which
 * rounding in a finite-precision evaluation of o_t = S_t^T q_t is measured
 * (o_t can be far smaller than m_t when its terms cancel).
 * i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 * Readings where the pages are silent: decay comes before the erase/write;
 * beta is one scalar per (token, head) and alpha the per-channel gate; no
 * query scaling and no normalisation happen inside the operation; the
 * read-out uses the state after the token's update.
 *
 * Addressing.  Inputs are "token rows": a row holds H heads, each head holding
 * d_k (q, k, log_alpha), d_v (v, o) or 1 (beta) values, contiguous.  Token t
 * of sequence n lives in row  row0[n] + t * row_step.  This one scheme covers
 * a dense [B,T,H,*] batch (row0[n] = n*T, step 1), a packed variable-length
 * batch (row0[n] = cu_seqlens[n], step 1) and a chain of single-token decode
 * steps stored [steps, N, H, *] (row0[n] = n, step N).
 *
 * Inputs arrive as fp32 (bf16 inputs are widened exactly by the caller) and
 * are widened to fp64 here; all arithmetic is fp64 in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_abi_version(void) { return 1; }

/* Returns the number of threads the parallel loop over (sequence, head) units
 * may use, for reporting. */
int kda_oracle_max_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0) return n_threads;
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/* One (sequence, head) unit, token by token.  S is a dk*dv scratch matrix. */
static void run_unit(int64_t n, int64_t h, const int64_t *row0, const int64_t *len,
                     int64_t row_step, int64_t H, int64_t dk, int64_t dv,
                     const float *q, const float *k, const float *v,
                     const float *beta, const float *log_alpha,
                     const double *s0, double *o, double *o_mag, double *s_final,
                     double *S, double *a, double *p, double *u)
{
    const int64_t unit = n * H + h;
    if (s0) memcpy(S, s0 + unit * dk * dv, (size_t)(dk * dv) * sizeof(double));
    else memset(S, 0, (size_t)(dk * dv) * sizeof(double));

    for (int64_t t = 0; t < len[n]; ++t) {
        const int64_t row = row0[n] + t * row_step;
        const float *qt = q + (row * H + h) * dk;
        const float *kt = k + (row * H + h) * dk;
        const float *lat = log_alpha + (row * H + h) * dk;
        const float *vt = v + (row * H + h) * dv;
        const double bt = (double)beta[row * H + h];
        double *ot = o + (row * H + h) * dv;

        /* forgetting factors, one per channel (row of S) */
        for (int64_t i = 0; i < dk; ++i) a[i] = exp((double)lat[i]);

        /* decay: S <- Diag(a) S */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a[i];

        /* recall: p = S^T k */
        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * (double)kt[i];

        /* compare: u = beta (v - p) */
        for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);

        /* correct: S <- S + k u^T */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += (double)kt[i] * u[j];

        /* read-out: o = S^T q */
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * (double)qt[i];

        /* magnitude of the read-out's terms: m = |S|^T |q| */
        if (o_mag) {
            double *mt = o_mag + (row * H + h) * dv;
            for (int64_t j = 0; j < dv; ++j) mt[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) mt[j] += fabs(S[i * dv + j]) * fabs((double)qt[i]);
        }
    }
    memcpy(s_final + unit * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
}

/*
 * Run the recurrence for n_seq sequences x H heads.
 *   row0[n_seq], len[n_seq] : token-row addressing (see above)
 *   q, k, log_alpha : rows x H x dk  (fp32)
 *   v               : rows x H x dv  (fp32)
 *   beta            : rows x H       (fp32)
 *   s0              : [n_seq, H, dk, dv] fp64, or NULL for zeros
 *   o               : rows x H x dv  fp64, written for every token visited
 *   o_mag           : rows x H x dv  fp64 (|S_t|^T |q_t| per token), or NULL
 *   s_final         : [n_seq, H, dk, dv] fp64
 *   n_threads       : <= 0 means the OpenMP default
 * Returns 0 on success, -1 on bad sizes, -2 on allocation failure.
 */
int kda_oracle_run(int64_t n_seq, const int64_t *row0, const int64_t *len, int64_t row_step,
                   int64_t H, int64_t dk, int64_t dv,
                   const float *q, const float *k, const float *v,
                   const float *beta, const float *log_alpha,
                   const double *s0, double *o, double *o_mag, double *s_final, int n_threads)
{
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (len[n] < 0 || row0[n] < 0) return -1;

    const int64_t units = n_seq * H;
    int failed = 0;
#ifdef _OPENMP
    /* per-call thread count; the process-wide default is left alone */
    const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel reduction(| : failed) num_threads(nt)
#endif
    {
        double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
        double *a = (double *)malloc((size_t)dk * sizeof(double));
        double *p = (double *)malloc((size_t)dv * sizeof(double));
        double *u = (double *)malloc((size_t)dv * sizeof(double));
        const int ok = S && a && p && u;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t w = 0; w < units; ++w) {
            if (!ok) { failed = 1; continue; }
            run_unit(w / H, w % H, row0, len, row_step, H, dk, dv, q, k, v, beta,
                     log_alpha, s0, o, o_mag, s_final, S, a, p, u);
        }
        free(S); free(a); free(p); free(u);
    }
    return failed ? -2 : 0;
}

/*
 * Input preparation from raw projections (the oracle of the library's "raw"
 * entry points).  The pages say KDA has two learned gate parameters -- beta,
 * the writing strength, and alpha, the forgetting factor ("Inside Kimi K3:
 * How Moonshot AI Built the Largest Open-Source Model", section "Technical
 * Details") -- but not how they are parameterised; the readings here are the
 * plainest ones that keep beta in (0, 1) and alpha in (0, 1):
 *   beta      = 1 / (1 + exp(-b_raw))                  (logistic sigmoid)
 *   log_alpha = -log(1 + exp(a_raw))                   (minus softplus)
 * and q and k are unit vectors per (row, head):
 *   q = q_raw / ||q_raw||_2,  k = k_raw / ||k_raw||_2  (a zero vector stays zero)
 * With round_bf16 set, the normalised q and k are rounded to bfloat16 (8
 * significant bits, round to nearest, ties to even), as they are when the
 * library stages bf16 inputs.  All arithmetic is fp64; results are stored as
 * fp32 (q and k then hold exact bf16 values).
 *   q_raw, k_raw : rows x H x dk;  b_raw : rows x H;  a_raw : rows x H x dk
 * Returns 0, or -1 on bad sizes.
 */
static double round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    const double m = frexp(x, &e);          /* x = m 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);  /* 8 significant bits, ties to even */
}

static void unit_vector(const float *x, int64_t dk, int round, float *out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < dk; ++i) ss += (double)x[i] * (double)x[i];
    const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
    for (int64_t i = 0; i < dk; ++i) {
        const double y = (double)x[i] * inv;
        out[i] = (float)(round ? round_bf16(y) : y);
    }
}

int kda_oracle_prepare(int64_t rows, int64_t H, int64_t dk,
                       const float *q_raw, const float *k_raw, const float *b_raw,
                       const float *a_raw, int round, float *q, float *k, float *beta,
                       float *log_alpha)
{
    if (rows < 0 || H <= 0 || dk <= 0) return -1;
    for (int64_t rh = 0; rh < rows * H; ++rh) {
        /* normalise each (row, head) vector on its own */
        unit_vector(q_raw + rh * dk, dk, round, q + rh * dk);
        unit_vector(k_raw + rh * dk, dk, round, k + rh * dk);
        /* write strength */
        beta[rh] = (float)(1.0 / (1.0 + exp(-(double)b_raw[rh])));
        /* forgetting gate: log_alpha = -softplus(a), evaluated without overflow */
        for (int64_t i = 0; i < dk; ++i) {
            const double a = (double)a_raw[rh * dk + i];
            const double sp = a > 0.0 ? a + log1p(exp(-a)) : log1p(exp(a));
            log_alpha[rh * dk + i] = (float)(-sp);
        }
    }
    return 0;
}

/*
 * Gradients (the adjoint of kda_oracle_run), for a later backward pass: the
 * chain rule applied to the forward steps above in reverse order, token by
 * token.  For the scalar loss
 *     L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * (dO = d_o, dS_T = d_sT or zero) and G the gradient with respect to the
 * current state, initialised to dS_T, each token t from the last back:
 *     G    += q_t dO_t^T                    read-out o_t = S_t^T q_t
 *     dq_t  = S_t dO_t
 *     du    = G^T k_t                       correct  S_t = S' + k_t u^T
 *     dk_t  = G u
 *     dbeta_t = du . (v_t - p),  dv_t = beta_t du,  dp = -beta_t du
 *     G'    = G + k_t dp^T                  recall   p = S'^T k_t
 *     dk_t += S' dp
 *     dlog_alpha_t[i] = sum_j G'[i][j] S'[i][j]   decay S' = Diag(a) S_{t-1}, a = exp(log_alpha)
 *     G     = Diag(a) G'
 * and finally dS_0 = G.  The entering state of every token is recomputed from
 * checkpoints taken every CK tokens, so memory stays (len/CK + CK) states per
 * (sequence, head).  Same addressing as kda_oracle_run; gradients are fp64 in
 * the layout of their inputs.  Returns 0, -1 on bad sizes, -2 on allocation
 * failure.
 */
#define CK 64

static void backward_unit(int64_t n, int64_t h, const int64_t *row0, const int64_t *len,
                          int64_t row_step, int64_t H, int64_t dk, int64_t dv,
                          const float *q, const float *k, const float *v,
                          const float *beta, const float *log_alpha, const double *s0,
                          const double *d_o, const double *d_sT,
                          double *dq, double *dkk, double *dvv, double *dbeta, double *dla,
                          double *ds0, double *ckpt, double *blk, double *S, double *G,
                          double *a, double *p, double *u, double *du, double *dp)
{
    const int64_t unit = n * H + h;
    const int64_t L = len[n], SZ = dk * dv;
    /* forward pass: the state entering token t for every t = 0 (mod CK) */
    if (s0) memcpy(S, s0 + unit * SZ, (size_t)SZ * sizeof(double));
    else memset(S, 0, (size_t)SZ * sizeof(double));
    for (int64_t t = 0; t < L; ++t) {
        if (t % CK == 0) memcpy(ckpt + (t / CK) * SZ, S, (size_t)SZ * sizeof(double));
        const int64_t row = row0[n] + t * row_step;
        const float *kt = k + (row * H + h) * dk;
        const float *vt = v + (row * H + h) * dv;
        const float *lat = log_alpha + (row * H + h) * dk;
        const double bt = (double)beta[row * H + h];
        for (int64_t i = 0; i < dk; ++i) {
            const double ai = exp((double)lat[i]);
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= ai;
        }
        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * (double)kt[i];
        for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += (double)kt[i] * u[j];
    }

    /* backward pass */
    if (d_sT) memcpy(G, d_sT + unit * SZ, (size_t)SZ * sizeof(double));
    else memset(G, 0, (size_t)SZ * sizeof(double));
    for (int64_t b0 = ((L - 1) / CK) * CK; L > 0 && b0 >= 0; b0 -= CK) {
        const int64_t b1 = b0 + CK < L ? b0 + CK : L;
        /* entering states of tokens b0 .. b1-1, recomputed from the checkpoint */
        memcpy(blk, ckpt + (b0 / CK) * SZ, (size_t)SZ * sizeof(double));
        for (int64_t t = b0; t + 1 < b1; ++t) {
            double *cur = blk + (t - b0) * SZ, *nxt = cur + SZ;
            const int64_t row = row0[n] + t * row_step;
            const float *kt = k + (row * H + h) * dk;
            const float *vt = v + (row * H + h) * dv;
            const float *lat = log_alpha + (row * H + h) * dk;
            const double bt = (double)beta[row * H + h];
            for (int64_t i = 0; i < dk; ++i) {
                const double ai = exp((double)lat[i]);
                for (int64_t j = 0; j < dv; ++j) nxt[i * dv + j] = cur[i * dv + j] * ai;
            }
            for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += nxt[i * dv + j] * (double)kt[i];
            for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) nxt[i * dv + j] += (double)kt[i] * u[j];
        }
        for (int64_t t = b1 - 1; t >= b0; --t) {
            const double *Sin = blk + (t - b0) * SZ;  /* S_{t-1} */
            const int64_t row = row0[n] + t * row_step;
            const float *qt = q + (row * H + h) * dk;
            const float *kt = k + (row * H + h) * dk;
            const float *vt = v + (row * H + h) * dv;
            const float *lat = log_alpha + (row * H + h) * dk;
            const double bt = (double)beta[row * H + h];
            const double *dot = d_o + (row * H + h) * dv;
            double *dqt = dq + (row * H + h) * dk;
            double *dkt = dkk + (row * H + h) * dk;
            double *dvt = dvv + (row * H + h) * dv;
            double *dlat = dla + (row * H + h) * dk;

            /* the token's forward quantities: S' = Diag(a) S_{t-1} (in S), p and u;
               S_t = S' + k u^T is formed where it is used */
            for (int64_t i = 0; i < dk; ++i) {
                a[i] = exp((double)lat[i]);
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = Sin[i * dv + j] * a[i];
            }
            for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * (double)kt[i];
            for (int64_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);

            /* read-out: G += q dO^T;  dq = S_t dO with S_t = S' + k u^T */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) G[i * dv + j] += (double)qt[i] * dot[j];
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j)
                    acc += (S[i * dv + j] + (double)kt[i] * u[j]) * dot[j];
                dqt[i] = acc;
            }
            /* correct: du = G^T k, dk = G u */
            for (int64_t j = 0; j < dv; ++j) du[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) du[j] += G[i * dv + j] * (double)kt[i];
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += G[i * dv + j] * u[j];
                dkt[i] = acc;
            }
            /* compare: u = beta (v - p) */
            double db = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
                db += du[j] * ((double)vt[j] - p[j]);
                dvt[j] = bt * du[j];
                dp[j] = -bt * du[j];
            }
            dbeta[row * H + h] = db;
            /* recall: p = S'^T k  ->  G' = G + k dp^T,  dk += S' dp */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    G[i * dv + j] += (double)kt[i] * dp[j];
                    acc += S[i * dv + j] * dp[j];
                }
                dkt[i] += acc;
            }
            /* decay: S' = Diag(a) S_{t-1} */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += G[i * dv + j] * S[i * dv + j];
                dlat[i] = acc;
                for (int64_t j = 0; j < dv; ++j) G[i * dv + j] *= a[i];
            }
        }
    }
    memcpy(ds0 + unit * SZ, G, (size_t)SZ * sizeof(double));
}

int kda_oracle_backward(int64_t n_seq, const int64_t *row0, const int64_t *len, int64_t row_step,
                        int64_t H, int64_t dk, int64_t dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *log_alpha, const double *s0,
                        const double *d_o, const double *d_sT,
                        double *dq, double *dkk, double *dvv, double *dbeta, double *dla,
                        double *ds0, int n_threads)
{
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    int64_t longest = 0;
    for (int64_t n = 0; n < n_seq; ++n) {
        if (len[n] < 0 || row0[n] < 0) return -1;
        if (len[n] > longest) longest = len[n];
    }
    const int64_t units = n_seq * H, SZ = dk * dv;
    const int64_t nck = longest / CK + 1;
    int failed = 0;
#ifdef _OPENMP
    /* per-call thread count; the process-wide default is left alone */
    const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel reduction(| : failed) num_threads(nt)
#endif
    {
        double *ckpt = (double *)malloc((size_t)(nck * SZ) * sizeof(double));
        double *blk = (double *)malloc((size_t)(CK * SZ) * sizeof(double));
        double *S = (double *)malloc((size_t)SZ * sizeof(double));
        double *G = (double *)malloc((size_t)SZ * sizeof(double));
        double *a = (double *)malloc((size_t)dk * sizeof(double));
        double *p = (double *)malloc((size_t)dv * sizeof(double));
        double *u = (double *)malloc((size_t)dv * sizeof(double));
        double *du = (double *)malloc((size_t)dv * sizeof(double));
        double *dp = (double *)malloc((size_t)dv * sizeof(double));
        const int ok = ckpt && blk && S && G && a && p && u && du && dp;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t w = 0; w < units; ++w) {
            if (!ok) { failed = 1; continue; }
            backward_unit(w / H, w % H, row0, len, row_step, H, dk, dv, q, k, v, beta, log_alpha,
                          s0, d_o, d_sT, dq, dkk, dvv, dbeta, dla, ds0, ckpt, blk, S, G, a, p, u,
                          du, dp);
        }
        free(ckpt); free(blk); free(S); free(G); free(a); free(p); free(u); free(du); free(dp);
    }
    return failed ? -2 : 0;
}
