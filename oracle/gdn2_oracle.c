/*
 * Plain FP64 token-by-token oracle for the Gated DeltaNet-2 forward pass.
 *
 * TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark load this library. It shares no code, header or
 * constant with the GPU library.
 *
 * Definition: FlashInfer chunk_gated_delta_rule2 docs, recurrence display
 * equation. Per (sequence, value head), state S is K x V, and per token t:
 *     S      = diag(exp(g_t)) S
 *     vnew   = w_t * v_t - (beta_t * k_t)^T S
 *     S     += k_t vnew^T
 *     o_t    = scale * q_t^T S
 * Same readings as oracle/recurrence.py (defaults, contiguous value-head
 * groups, K-major state, packed varlen sequences). The caller passes the
 * already resolved scale.
 *
 * Inputs may be float64, float32 or bfloat16 (raw 16-bit patterns); every
 * value is widened exactly to double before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

static double ld(const void *p, int dtype, int64_t i)
{
    if (dtype == ORC_F64)
        return ((const double *)p)[i];
    if (dtype == ORC_F32)
        return (double)((const float *)p)[i];
    /* bfloat16: the upper 16 bits of an IEEE float32 */
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Shapes (row-major, contiguous):
 *   q, k [T, H, K]; v, w [T, HV, V]; g, beta [T, HV, K];
 *   initial_state [N, HV, K, V] (may be NULL = zeros);
 *   g NULL = 0, beta NULL = 1, w NULL = 1.
 *   cu_seqlens [N+1] (NULL = one sequence of T tokens, N must be 1).
 *   heads[nheads]: value heads to evaluate.
 * Outputs: out [T, nheads, V], final_state [N, nheads, K, V] (may be NULL).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int gdn2_oracle_fwd(const void *q, int q_dt, const void *k, int k_dt,
                    const void *v, int v_dt, const void *g, int g_dt,
                    const void *beta, int beta_dt, const void *w, int w_dt,
                    double scale, const void *initial_state, int s_dt,
                    const int32_t *cu_seqlens, int32_t N, int64_t T, int32_t H,
                    int32_t HV, int32_t K, int32_t V, const int32_t *heads,
                    int32_t nheads, double *out, double *final_state)
{
    if (!q || !k || !v || !out || !heads || H <= 0 || HV % H != 0 || K <= 0 ||
        V <= 0 || N <= 0 || nheads <= 0)
        return -1;
    if (!cu_seqlens && N != 1)
        return -1;
    const int32_t m = HV / H;
    const int64_t items = (int64_t)N * nheads;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t it = 0; it < items; ++it) {
        const int32_t n = (int32_t)(it / nheads);
        const int32_t hi = (int32_t)(it % nheads);
        const int32_t hv = heads[hi];
        const int32_t hk = hv / m;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;

        double *S = (double *)malloc(sizeof(double) * (size_t)K * (size_t)V);
        double *vn = (double *)malloc(sizeof(double) * (size_t)V);
        double *bk = (double *)malloc(sizeof(double) * (size_t)K);
        double *kk = (double *)malloc(sizeof(double) * (size_t)K);
        double *qq = (double *)malloc(sizeof(double) * (size_t)K);
        double *acc = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !vn || !bk || !kk || !qq || !acc) {
            failed = 1;
            free(S); free(vn); free(bk); free(kk); free(qq); free(acc);
            continue;
        }
        for (int32_t c = 0; c < K; ++c)
            for (int32_t j = 0; j < V; ++j)
                S[(int64_t)c * V + j] =
                    initial_state
                        ? ld(initial_state, s_dt,
                             (((int64_t)n * HV + hv) * K + c) * V + j)
                        : 0.0;

        for (int64_t t = t0; t < t1; ++t) {
            const int64_t qk_row = (t * H + hk) * K; /* q/k head hk */
            const int64_t gb_row = (t * HV + hv) * K; /* gates of value head hv */
            const int64_t vw_row = (t * HV + hv) * V;

            /* forget gate on the key axis */
            for (int32_t c = 0; c < K; ++c) {
                const double a = g ? exp(ld(g, g_dt, gb_row + c)) : 1.0;
                for (int32_t j = 0; j < V; ++j)
                    S[(int64_t)c * V + j] *= a;
                kk[c] = ld(k, k_dt, qk_row + c);
                qq[c] = ld(q, q_dt, qk_row + c);
                bk[c] = (beta ? ld(beta, beta_dt, gb_row + c) : 1.0) * kk[c];
            }
            /* vnew = w*v - (beta*k)^T S, S already decayed; the sum over
               key channels c runs in ascending c for every j */
            for (int32_t j = 0; j < V; ++j)
                acc[j] = 0.0;
            for (int32_t c = 0; c < K; ++c)
                for (int32_t j = 0; j < V; ++j)
                    acc[j] += bk[c] * S[(int64_t)c * V + j];
            for (int32_t j = 0; j < V; ++j) {
                const double wv =
                    (w ? ld(w, w_dt, vw_row + j) : 1.0) * ld(v, v_dt, vw_row + j);
                vn[j] = wv - acc[j];
            }
            /* rank-one write k vnew^T */
            for (int32_t c = 0; c < K; ++c)
                for (int32_t j = 0; j < V; ++j)
                    S[(int64_t)c * V + j] += kk[c] * vn[j];
            /* output from the updated state */
            for (int32_t j = 0; j < V; ++j)
                acc[j] = 0.0;
            for (int32_t c = 0; c < K; ++c)
                for (int32_t j = 0; j < V; ++j)
                    acc[j] += qq[c] * S[(int64_t)c * V + j];
            for (int32_t j = 0; j < V; ++j)
                out[(t * nheads + hi) * V + j] = scale * acc[j];
        }
        if (final_state)
            for (int32_t c = 0; c < K; ++c)
                for (int32_t j = 0; j < V; ++j)
                    final_state[(((int64_t)n * nheads + hi) * K + c) * V + j] =
                        S[(int64_t)c * V + j];
        free(S); free(vn); free(bk); free(kk); free(qq); free(acc);
    }
    return failed ? -1 : 0;
}

/* Threads an OpenMP parallel region would use (for reporting). */
int gdn2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward pass of the same recurrence: the reverse sweep of the chain rule
 * listed in oracle/recurrence_bwd.py, per (sequence, value head), in float64.
 * States are recomputed: the forward sweep keeps the state at the start of
 * every `block` tokens; the reverse sweep recomputes one block's states from
 * its checkpoint, then walks that block backwards.
 *
 * Inputs as gdn2_oracle_fwd (all value heads; g, beta and w required), plus
 * d_out [T, HV, V] and d_final [N, HV, K, V] (NULL = zero).
 * Outputs: dq, dk [T, HV, K] per value head (the caller sums the value heads
 * of each q/k head), dv, dw [T, HV, V], dg, dbeta [T, HV, K],
 * dS0 [N, HV, K, V]. Returns 0, or -1 on a bad argument or allocation
 * failure.
 */
int gdn2_oracle_bwd(const void *q, int q_dt, const void *k, int k_dt,
                    const void *v, int v_dt, const void *g, int g_dt,
                    const void *beta, int beta_dt, const void *w, int w_dt,
                    double scale, const void *initial_state, int s_dt,
                    const void *d_out, int do_dt, const void *d_final, int df_dt,
                    const int32_t *cu_seqlens, int32_t N, int64_t T, int32_t H,
                    int32_t HV, int32_t K, int32_t V, int32_t block,
                    double *dq, double *dk, double *dv, double *dw, double *dg,
                    double *dbeta, double *dS0)
{
    if (!q || !k || !v || !g || !beta || !w || !d_out || H <= 0 || HV % H != 0 ||
        K <= 0 || V <= 0 || N <= 0 || block <= 0 || !dq || !dk || !dv || !dw || !dg ||
        !dbeta || !dS0)
        return -1;
    if (!cu_seqlens && N != 1)
        return -1;
    const int32_t m = HV / H;
    const int64_t items = (int64_t)N * HV;
    const size_t KV = (size_t)K * (size_t)V;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t it = 0; it < items; ++it) {
        const int32_t n = (int32_t)(it / HV);
        const int32_t hv = (int32_t)(it % HV);
        const int32_t hk = hv / m;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
        const int64_t L = t1 - t0;
        const int64_t nblk = (L + block - 1) / block;

        double *ck = (double *)malloc(sizeof(double) * KV * (size_t)(nblk > 0 ? nblk : 1));
        double *Sp = (double *)malloc(sizeof(double) * KV * (size_t)block);
        double *S = (double *)malloc(sizeof(double) * KV);
        double *Sd = (double *)malloc(sizeof(double) * KV);
        double *dS = (double *)malloc(sizeof(double) * KV);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(8 * (K > V ? K : V)));
        if (!ck || !Sp || !S || !Sd || !dS || !vec) {
            failed = 1;
            free(ck); free(Sp); free(S); free(Sd); free(dS); free(vec);
            continue;
        }
        const int32_t D = K > V ? K : V;
        double *a = vec, *kk = vec + D, *qq = vec + 2 * D, *bk = vec + 3 * D;
        double *vn = vec + 4 * D, *dvn = vec + 5 * D, *dbk = vec + 6 * D, *dov = vec + 7 * D;

        for (size_t i = 0; i < KV; ++i)
            S[i] = initial_state ? ld(initial_state, s_dt, ((int64_t)n * HV + hv) * (int64_t)KV + (int64_t)i) : 0.0;

        /* one token of the forward recurrence on S; Sd receives the decayed
           state, vn the new value */
#define GDN2_ORACLE_STEP(t)                                                         \
        do {                                                                        \
            const int64_t qk_row = ((t) * H + hk) * K;                              \
            const int64_t gb_row = ((t) * HV + hv) * K;                             \
            const int64_t vw_row = ((t) * HV + hv) * V;                             \
            for (int32_t c = 0; c < K; ++c) {                                       \
                a[c] = exp(ld(g, g_dt, gb_row + c));                                \
                kk[c] = ld(k, k_dt, qk_row + c);                                    \
                qq[c] = ld(q, q_dt, qk_row + c);                                    \
                bk[c] = ld(beta, beta_dt, gb_row + c) * kk[c];                      \
                for (int32_t j = 0; j < V; ++j)                                     \
                    Sd[(int64_t)c * V + j] = a[c] * S[(int64_t)c * V + j];          \
            }                                                                       \
            for (int32_t j = 0; j < V; ++j) {                                       \
                double e = 0.0;                                                     \
                for (int32_t c = 0; c < K; ++c)                                     \
                    e += bk[c] * Sd[(int64_t)c * V + j];                            \
                vn[j] = ld(w, w_dt, vw_row + j) * ld(v, v_dt, vw_row + j) - e;      \
            }                                                                       \
            for (int32_t c = 0; c < K; ++c)                                         \
                for (int32_t j = 0; j < V; ++j)                                     \
                    S[(int64_t)c * V + j] = Sd[(int64_t)c * V + j] + kk[c] * vn[j]; \
        } while (0)

        /* forward sweep: checkpoints at block starts */
        for (int64_t t = t0; t < t1; ++t) {
            if ((t - t0) % block == 0)
                memcpy(ck + KV * (size_t)((t - t0) / block), S, sizeof(double) * KV);
            GDN2_ORACLE_STEP(t);
        }
        /* reverse sweep */
        for (size_t i = 0; i < KV; ++i)
            dS[i] = d_final ? ld(d_final, df_dt, ((int64_t)n * HV + hv) * (int64_t)KV + (int64_t)i) : 0.0;
        for (int64_t b = nblk - 1; b >= 0; --b) {
            const int64_t tb = t0 + b * block;
            const int64_t te = tb + block < t1 ? tb + block : t1;
            memcpy(S, ck + KV * (size_t)b, sizeof(double) * KV);
            for (int64_t t = tb; t < te; ++t) {
                memcpy(Sp + KV * (size_t)(t - tb), S, sizeof(double) * KV);
                GDN2_ORACLE_STEP(t);
            }
            for (int64_t t = te - 1; t >= tb; --t) {
                memcpy(S, Sp + KV * (size_t)(t - tb), sizeof(double) * KV);
                GDN2_ORACLE_STEP(t); /* refreshes a, kk, qq, bk, Sd, vn for token t; S = S_t */
                const int64_t gb_row = (t * HV + hv) * K;
                const int64_t vw_row = (t * HV + hv) * V;
                for (int32_t j = 0; j < V; ++j)
                    dov[j] = ld(d_out, do_dt, vw_row + j);
                /* o_t = scale S_t^T q_t */
                for (int32_t c = 0; c < K; ++c) {
                    double s = 0.0;
                    for (int32_t j = 0; j < V; ++j)
                        s += S[(int64_t)c * V + j] * dov[j];
                    dq[gb_row + c] = scale * s;
                    for (int32_t j = 0; j < V; ++j)
                        dS[(int64_t)c * V + j] += scale * qq[c] * dov[j];
                }
                /* S_t = Sd + k vnew^T ; vnew = w v - Sd^T (beta k) */
                for (int32_t j = 0; j < V; ++j) {
                    double s = 0.0;
                    for (int32_t c = 0; c < K; ++c)
                        s += dS[(int64_t)c * V + j] * kk[c];
                    dvn[j] = s;
                    dw[vw_row + j] = s * ld(v, v_dt, vw_row + j);
                    dv[vw_row + j] = s * ld(w, w_dt, vw_row + j);
                }
                for (int32_t c = 0; c < K; ++c) {
                    double s = 0.0, e = 0.0;
                    for (int32_t j = 0; j < V; ++j) {
                        s += dS[(int64_t)c * V + j] * vn[j];
                        e -= Sd[(int64_t)c * V + j] * dvn[j]; /* de = -dvnew */
                    }
                    dbk[c] = e;
                    dbeta[gb_row + c] = e * kk[c];
                    dk[gb_row + c] = s + e * ld(beta, beta_dt, gb_row + c);
                }
                /* dSd = dS + (beta k) de^T ; dg = rowsum(dSd * Sd) ; dS_{t-1} = a dSd */
                for (int32_t c = 0; c < K; ++c) {
                    double s = 0.0;
                    for (int32_t j = 0; j < V; ++j) {
                        const double x = dS[(int64_t)c * V + j] - bk[c] * dvn[j];
                        s += x * Sd[(int64_t)c * V + j];
                        dS[(int64_t)c * V + j] = a[c] * x;
                    }
                    dg[gb_row + c] = s;
                }
            }
        }
#undef GDN2_ORACLE_STEP
        for (size_t i = 0; i < KV; ++i)
            dS0[((int64_t)n * HV + hv) * (int64_t)KV + (int64_t)i] = dS[i];
        free(ck); free(Sp); free(S); free(Sd); free(dS); free(vec);
    }
    return failed ? -1 : 0;
}
