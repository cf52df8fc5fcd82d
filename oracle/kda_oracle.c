/*
 * KDA oracle: the gated delta rule with a per-channel decay, evaluated one
 * token at a time in fp64 on the host.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle for the HIP
 * library.  It shares no code, header, table or constant with the GPU path,
 * and the GPU path never links or calls it.  Only tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.
 *
 * What it computes (Kimi K3 architecture blog post, section on the lower
 * bound on the log-decay: a fixed-size recurrent state that forgets as it
 * goes; section on the serving stack: the state is updated serially and in
 * place).  For one head of one sequence, with state S (dk x dv), starting
 * from S = h0 (or zero), for every token t in order:
 *
 *     S   <- Diag(exp(g_t)) S                     decay first
 *     S   <- S - beta_t k_t (k_t^T S)             erase  (I - beta k k^T)
 *     S   <- S + beta_t k_t v_t^T                 write
 *     o_t  = S^T q_t                              read after the update
 *
 * and ht = S after the last token.  This is the plain definition; the
 * chunked method reaches the same result up to rounding order, so the
 * oracle is the definition written out, with no blocking and no fusion.
 *
 * Inputs are float32 (every bf16 value is exactly representable in
 * float32, so a bf16 input upcast to float32 is the exact value the GPU
 * sees); all arithmetic and all outputs are fp64.
 *
 * Pins: see tests/test_oracle_pins.py (brute-force transition products,
 * closed forms for beta = 0, one-hot and orthonormal keys, the write-then-
 * read identity, affine segment composition, neutral padding, varlen,
 * resume and prefill = repeated decode).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle-only ablation: skip the erase term (gated linear attention). */
#define KDA_ORACLE_NO_ERASE 1u

/* One token on one (sequence, head) state, in place.  kS is dv scratch. */
static void oracle_token(double *S, const float *q, const float *k,
                         const float *v, const float *g, double beta, int dk,
                         int dv, int erase, double *kS, double *out)
{
    /* decay: row c of S is scaled by exp(g[c]) */
    for (int c = 0; c < dk; ++c) {
        double f = exp((double)g[c]);
        double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j)
            row[j] *= f;
    }
    /* erase: S -= beta k (k^T S) */
    if (erase) {
        for (int j = 0; j < dv; ++j)
            kS[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            double kc = (double)k[c];
            const double *row = S + (size_t)c * dv;
            for (int j = 0; j < dv; ++j)
                kS[j] += kc * row[j];
        }
        for (int c = 0; c < dk; ++c) {
            double a = beta * (double)k[c];
            double *row = S + (size_t)c * dv;
            for (int j = 0; j < dv; ++j)
                row[j] -= a * kS[j];
        }
    }
    /* write: S += beta k v^T */
    for (int c = 0; c < dk; ++c) {
        double a = beta * (double)k[c];
        double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j)
            row[j] += a * (double)v[j];
    }
    /* read: out = S^T q */
    for (int j = 0; j < dv; ++j)
        out[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
        double qc = (double)q[c];
        const double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j)
            out[j] += qc * row[j];
    }
}

/*
 * Packed prefill.  Rows are tokens of all sequences concatenated; sequence n
 * owns rows [cu[n], cu[n+1]).
 *   q, k : [T][H][dk]   v : [T][H][dv]   g : [T][H][dk]   beta : [T][H]
 *   h0   : [N][H][dk][dv] or NULL (zero state)
 *   o    : [T][H][dv] (fp64 out)   ht : [N][H][dk][dv] (fp64 out) or NULL
 * Chains (n, h) are independent; they are spread over nthreads OpenMP
 * threads (<= 0 means the OpenMP default).  Returns 0, or -1 on bad args.
 */
int kda_oracle_prefill(const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const double *h0,
                       const int64_t *cu, int64_t N, int64_t H, int64_t dk,
                       int64_t dv, unsigned flags, double *o, double *ht,
                       int nthreads)
{
    if (!q || !k || !v || !g || !beta || !cu || !o || N < 0 || H <= 0 ||
        dk <= 0 || dv <= 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return -1;
    const int erase = (flags & KDA_ORACLE_NO_ERASE) ? 0 : 1;
    const int64_t chains = N * H;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t ch = 0; ch < chains; ++ch) {
        const int64_t n = ch / H, h = ch % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        if (h0)
            memcpy(S, h0 + (size_t)ch * dk * dv, sizeof(double) * dk * dv);
        else
            memset(S, 0, sizeof(double) * dk * dv);
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const size_t r = (size_t)t * H + h;
            oracle_token(S, q + r * dk, k + r * dk, v + r * dv, g + r * dk,
                         (double)beta[r], (int)dk, (int)dv, erase, kS,
                         o + r * dv);
        }
        if (ht)
            memcpy(ht + (size_t)ch * dk * dv, S, sizeof(double) * dk * dv);
        free(kS);
        free(S);
    }
    return 0;
}

/*
 * One decode step for N independent sequences: the same token update on a
 * state held by the caller, in place (the serving-stack section: the state
 * is updated in place).
 *   q, k : [N][H][dk]  v : [N][H][dv]  g : [N][H][dk]  beta : [N][H]
 *   state: [N][H][dk][dv] fp64, in/out      o : [N][H][dv] fp64 out
 */
int kda_oracle_decode_step(const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *state,
                           int64_t N, int64_t H, int64_t dk, int64_t dv,
                           double *o, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !state || !o || N < 0 || H <= 0 ||
        dk <= 0 || dv <= 0)
        return -1;
    const int64_t chains = N * H;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t ch = 0; ch < chains; ++ch) {
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        oracle_token(state + (size_t)ch * dk * dv, q + (size_t)ch * dk,
                     k + (size_t)ch * dk, v + (size_t)ch * dv,
                     g + (size_t)ch * dk, (double)beta[ch], (int)dk, (int)dv,
                     1, kS, o + (size_t)ch * dv);
        free(kS);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use by default. */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
