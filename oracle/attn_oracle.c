/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, fp64 CPU definition of attention that the GPU path is
 * checked against. Only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library; the product path never calls it and shares
 * no code with it.
 *
 * Source: the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与
 * TiledMMA" (tom-jerr.github.io), cited below as [CuTe-FA2].
 *   - [CuTe-FA2] §"先看全局：FA2 中的数据究竟去了哪里", first equation:
 *     one query tile computes S = Q Kᵀ, P = softmax(S), O = P V.
 *   - [CuTe-FA2] §"教学配置：一块 CTA 做什么", the equations for m_i, ℓ_i and õ_i:
 *     ℓ_i is the sum over processed keys of e^{s_ij - m_i}, and the output is
 *     O_i = õ_i / ℓ_i once every key has been seen. Over all keys this is the
 *     row softmax of S applied to V, which is what is written out here.
 *   - [CuTe-FA2] §"沿 C fragment 做 Online Softmax", last paragraph: the scores
 *     are multiplied by a positive softmax scale (1/8 for D = 64).
 *   - [CuTe-FA2] §"与官方 FA2 比较时，先对齐契约": tensors are [B,H,N,D]
 *     row-major, and the production kernel also returns the softmax
 *     log-sum-exp. Its base is not printed; the natural log is used, so that
 *     exp(scale*q_i.k_j - LSE_i) is the probability P_ij.
 *   - "causal" (named throughout [CuTe-FA2] with no formula): query i may
 *     attend key j only when j <= i (query and key lengths are equal).
 *
 * Definition computed, for every (b, h, i), with J_i = {0..S-1} (or {0..i}
 * when causal), in double precision, with no tiling and no online update:
 *     s_ij  = scale * sum_d q_id k_jd          for j in J_i
 *     M_i   = max_j s_ij
 *     l_i   = sum_j exp(s_ij - M_i)
 *     P_ij  = exp(s_ij - M_i) / l_i
 *     O_id  = sum_j P_ij v_jd
 *     LSE_i = M_i + log(l_i)
 * Subtracting M_i is the textbook way to evaluate softmax without overflow;
 * it does not change P (the factor e^{-M_i} cancels) and LSE adds it back.
 *
 * Inputs are double arrays holding the exact values of the fp16 inputs.
 * Layout: q, k, v, O are [B,H,S,D] row-major; LSE is [B,H,S].
 */
#include <math.h>
#include <stdlib.h>
#include <omp.h>

/* One query row: writes D outputs and the log-sum-exp. `s` and `p` are
 * caller-provided scratch arrays of at least S doubles. */
static void attend_row(const double *q, const double *k, const double *v,
                       long long S, long long D, long long i, int causal,
                       double scale, double *s, double *p,
                       double *o_row, double *lse_out)
{
    const double *qi = q + i * D;
    long long n_keys = causal ? i + 1 : S;   /* keys j in J_i are 0 .. n_keys-1 */

    /* scores */
    for (long long j = 0; j < n_keys; ++j) {
        const double *kj = k + j * D;
        double dot = 0.0;
        for (long long d = 0; d < D; ++d)
            dot += qi[d] * kj[d];
        s[j] = scale * dot;
    }

    /* row max */
    double M = s[0];
    for (long long j = 1; j < n_keys; ++j)
        if (s[j] > M)
            M = s[j];

    /* normaliser */
    double l = 0.0;
    for (long long j = 0; j < n_keys; ++j)
        l += exp(s[j] - M);

    /* probabilities */
    for (long long j = 0; j < n_keys; ++j)
        p[j] = exp(s[j] - M) / l;

    /* output row: O_i = sum_j P_ij v_j */
    for (long long d = 0; d < D; ++d) {
        double acc = 0.0;
        for (long long j = 0; j < n_keys; ++j)
            acc += p[j] * v[j * D + d];
        o_row[d] = acc;
    }

    *lse_out = M + log(l);
}

/* Full attention over every (b, h, i). Returns 0 on success, -1 on bad
 * arguments, -2 if scratch memory cannot be allocated. `nthreads` <= 0 means
 * the OpenMP default. */
int attn_oracle_f64(const double *q, const double *k, const double *v,
                    int B, int H, int S, int D, int causal, double scale,
                    double *O, double *LSE, int nthreads)
{
    if (!q || !k || !v || !O || !LSE || B < 1 || H < 1 || S < 1 || D < 1)
        return -1;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    long long rows = (long long)B * H * S;
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *p = (double *)malloc(sizeof(double) * (size_t)S);
        if (!s || !p) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < rows; ++r) {
            if (!s || !p)
                continue;
            long long head = r / S, i = r % S;
            const long long base = head * (long long)S * D;
            attend_row(q + base, k + base, v + base, S, D, i, causal, scale,
                       s, p, O + r * D, LSE + r);
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* The same definition for a list of rows only. rows[n] is the flat index
 * (b*H + h)*S + i of a query row; O is [nrows, D] and LSE is [nrows]. */
int attn_oracle_rows_f64(const double *q, const double *k, const double *v,
                         int B, int H, int S, int D, int causal, double scale,
                         const long long *rows, int nrows,
                         double *O, double *LSE, int nthreads)
{
    if (!q || !k || !v || !rows || !O || !LSE || B < 1 || H < 1 || S < 1 ||
        D < 1 || nrows < 0)
        return -1;
    long long total = (long long)B * H * S;
    for (int n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= total)
            return -1;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *p = (double *)malloc(sizeof(double) * (size_t)S);
        if (!s || !p) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int n = 0; n < nrows; ++n) {
            if (!s || !p)
                continue;
            long long r = rows[n];
            long long head = r / S, i = r % S;
            const long long base = head * (long long)S * D;
            attend_row(q + base, k + base, v + base, S, D, i, causal, scale,
                       s, p, O + (long long)n * D, LSE + n);
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* Number of threads a parallel region of this library uses by default. */
int attn_oracle_max_threads(void) { return omp_get_max_threads(); }
