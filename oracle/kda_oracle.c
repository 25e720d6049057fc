/*
 * kda_oracle.c -- fp64 CPU oracle for the Kimi Delta Attention forward pass.
 *
 * TEST INFRASTRUCTURE. This file is the correctness reference that the GPU
 * library is checked against. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. The product path (the HIP
 * library and its Python binding) never links, imports or calls it, and it
 * shares no code, headers, tables or helpers with that path.
 *
 * What it computes (source: "You Could Have Come Up with Kimi Delta
 * Attention", Doubleword blog, section 4, boxed KDA equations; section 4.1 for
 * the log-decay storage g = log(alpha)):
 *
 *   for every token t of a sequence, one head at a time, state S is V x K
 *   (row = value channel, column = key channel):
 *     S~  = S . Diag(alpha_t)         forget each key channel
 *     vh  = S~ k_t                    predict
 *     e   = beta_t (v_t - vh)         correct
 *     S   = S~ + e k_t^T              write
 *     o_t = S (s q_t),  s = scale     read (after the write)
 *
 * The activations in front of the recurrence follow the FlashKDA pages
 * (instagit summary of FlashKDA, "Chunked Token Processing"; DocSearch digest
 * of FlashKDA, "Configure fla_chunk_kda" and "flash_kda.fwd API reference"):
 *     alpha_t = exp(g_t),  g_t = lower_bound * sigmoid(g_raw_t)  (per channel)
 *     beta_t  = sigmoid(beta_raw_t)
 *     q, k L2-normalised per token: x / sqrt(sum x^2 + eps)
 * The epsilon is not given on the pages; the caller passes it (1e-6 is the
 * reading used throughout this project).
 *
 * Everything is plain fp64 in the order written above: no blocking, no
 * chunking, no fusion. OpenMP only splits independent (sequence, head) pairs
 * over threads; each pair is stepped strictly token by token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Logistic sigmoid 1/(1+e^-x), evaluated in the branch that cannot overflow. */
double kda_oracle_sigmoid(double x)
{
    if (x >= 0.0) {
        double e = exp(-x);
        return 1.0 / (1.0 + e);
    }
    double e = exp(x);
    return e / (1.0 + e);
}

/*
 * The recurrence for one (sequence, head) on already-activated inputs.
 *   q, k : [T][dk] rows with row stride sq / sk (doubles); used as given
 *   v    : [T][dv] rows with stride sv
 *   alpha: [T][dk] retention factors, stride sa
 *   beta : [T] with stride sb
 *   S    : [dv][dk] state, updated in place (holds the initial state on entry)
 *   o    : [T][dv] output rows with stride so
 *   work : scratch of dv doubles
 */
static void core_pair(int64_t T, int64_t dk, int64_t dv,
                      const double *q, int64_t sq,
                      const double *k, int64_t sk,
                      const double *v, int64_t sv,
                      const double *alpha, int64_t sa,
                      const double *beta, int64_t sb,
                      double scale, double *S,
                      double *o, int64_t so, double *work)
{
    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * sq;
        const double *kt = k + t * sk;
        const double *vt = v + t * sv;
        const double *at = alpha + t * sa;
        const double bt = beta[t * sb];
        double *ot = o + t * so;
        /* forget: scale key column j by alpha_t[j] */
        for (int64_t i = 0; i < dv; ++i)
            for (int64_t j = 0; j < dk; ++j)
                S[i * dk + j] *= at[j];
        /* predict and correct: e = beta (v - S~ k) */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * kt[j];
            work[i] = bt * (vt[i] - acc);
        }
        /* write: S += e k^T */
        for (int64_t i = 0; i < dv; ++i)
            for (int64_t j = 0; j < dk; ++j)
                S[i * dk + j] += work[i] * kt[j];
        /* read after write: o = S (scale q) */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * (scale * qt[j]);
            ot[i] = acc;
        }
    }
}

/*
 * Recurrence on pre-activated inputs for a single (sequence, head):
 * q, k used as given (no normalisation), alpha and beta given directly.
 * Contiguous rows: q,k,alpha [T][dk], v,o [T][dv], beta [T], S [dv][dk].
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_core(int64_t T, int64_t dk, int64_t dv,
                    const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta, double scale,
                    double *S, double *o)
{
    if (T < 0 || dk < 1 || dv < 1 || !S || (T > 0 && (!q || !k || !v || !alpha || !beta || !o)))
        return -1;
    double *work = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!work) return -1;
    core_pair(T, dk, dv, q, dk, k, dk, v, dv, alpha, dk, beta, 1, scale, S, o, dv, work);
    free(work);
    return 0;
}

/*
 * Full forward on raw inputs, packed layout as in the FlashKDA API
 * (DocSearch digest of FlashKDA, "flash_kda.fwd API reference"):
 *   q, k, g_raw : [T_tot][H][dk]     v, out : [T_tot][H][dv]
 *   beta_raw    : [T_tot][H]
 *   seq_offsets : N+1 token offsets; sequence n is [off[n], off[n+1])
 *   initial_state, final_state : [N][H][dv][dk] or NULL (NULL initial = zeros)
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_fwd(int64_t num_seqs, const int64_t *seq_offsets,
                   int64_t num_heads, int64_t dk, int64_t dv,
                   const double *q, const double *k, const double *v,
                   const double *g_raw, const double *beta_raw,
                   const double *initial_state,
                   double lower_bound, double scale, double l2_eps,
                   double *out, double *final_state, int num_threads)
{
    if (num_seqs < 0 || num_heads < 1 || dk < 1 || dv < 1 || !seq_offsets)
        return -1;
    if (seq_offsets[0] != 0) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (seq_offsets[n + 1] < seq_offsets[n]) return -1;
    const int64_t T_tot = seq_offsets[num_seqs];
    if (T_tot > 0 && (!q || !k || !v || !g_raw || !beta_raw || !out)) return -1;

    const int64_t pairs = num_seqs * num_heads;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / num_heads, h = p % num_heads;
        const int64_t t0 = seq_offsets[n], T = seq_offsets[n + 1] - t0;
        double *S = (double *)calloc((size_t)(dv * dk), sizeof(double));
        double *qn = (double *)malloc(sizeof(double) * (size_t)(T * dk + 1));
        double *kn = (double *)malloc(sizeof(double) * (size_t)(T * dk + 1));
        double *al = (double *)malloc(sizeof(double) * (size_t)(T * dk + 1));
        double *be = (double *)malloc(sizeof(double) * (size_t)(T + 1));
        double *work = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !qn || !kn || !al || !be || !work) {
            bad = 1;
        } else {
            if (initial_state)
                memcpy(S, initial_state + p * dv * dk, sizeof(double) * (size_t)(dv * dk));
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (t0 + t) * num_heads + h;
                const double *qs = q + row * dk, *ks = k + row * dk, *gs = g_raw + row * dk;
                double nq = 0.0, nk = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    nq += qs[j] * qs[j];
                    nk += ks[j] * ks[j];
                }
                const double rq = 1.0 / sqrt(nq + l2_eps), rk = 1.0 / sqrt(nk + l2_eps);
                for (int64_t j = 0; j < dk; ++j) {
                    qn[t * dk + j] = qs[j] * rq;
                    kn[t * dk + j] = ks[j] * rk;
                    al[t * dk + j] = exp(lower_bound * kda_oracle_sigmoid(gs[j]));
                }
                be[t] = kda_oracle_sigmoid(beta_raw[row]);
            }
            /* v and out rows are strided by H*dv in the packed layout */
            core_pair(T, dk, dv, qn, dk, kn, dk,
                      v + (t0 * num_heads + h) * dv, num_heads * dv,
                      al, dk, be, 1, scale, S,
                      out + (t0 * num_heads + h) * dv, num_heads * dv, work);
            if (final_state)
                memcpy(final_state + p * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        }
        free(S); free(qn); free(kn); free(al); free(be); free(work);
    }
    return bad ? -1 : 0;
}

/* Threads an OpenMP region will use by default (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
