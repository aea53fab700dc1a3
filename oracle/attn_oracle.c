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
 *
 * Extensions. [CuTe-FA2] §"哪些结论可以迁移，哪些只是本例特例" lists local
 * masks, variable-length sequences, dropout and GQA/MQA among the features of
 * the production kernel without defining them. The plain readings used here:
 *   - local window (wl, wr): J_i = { j : i - wl <= j <= i + wr, 0 <= j < S },
 *     a negative side being unbounded; (-1, 0) is causal, (-1, -1) is all keys.
 *   - GQA/MQA and variable-length sequences only select which q, k, v rows
 *     form one problem; attn_oracle_head_f64 below takes one (sequence, head)
 *     at a time and the Python wrapper does the selection.
 *   - dropout with probability p: after the softmax, P_ij is multiplied by
 *     z_ij / (1 - p) with z_ij in {0, 1}; l_i and LSE_i are those of the
 *     softmax before dropout. The 128-bit output of
 *     Philox4x32-10(counter = (floor(j/8), i, bh, offset), key = (k0, k1))
 *     is read as eight 16-bit draws, draw t being bits 16*(t mod 2) .. +15
 *     of word floor(t/2); z_ij = 1 when draw (j mod 8) is >= thr, with
 *     thr = floor(p * 2^16) clamped to 2^16 - 1 and bh the flat (sequence,
 *     head) index. Philox4x32-10 follows Salmon, Moraes, Dror and Shaw,
 *     "Parallel random numbers: as easy as 1, 2, 3" (SC 2011).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* Philox4x32-10 (Salmon et al., SC 2011): ten rounds on a 4-word counter. A
 * round multiplies words 0 and 2 by fixed 32-bit constants; the new word 0 is
 * the high half of the second product xor word 1 xor key word 0, the new word 1
 * its low half, the new word 2 the high half of the first product xor word 3
 * xor key word 1, and the new word 3 its low half. Between rounds each key word
 * grows by its Weyl constant (the golden ratio and sqrt(3) - 1, scaled to
 * 2^32). */
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += weyl0;
            k1 += weyl1;
        }
        const uint64_t prod0 = (uint64_t)mult0 * x[0];
        const uint64_t prod1 = (uint64_t)mult1 * x[2];
        const uint32_t y[4] = {
            (uint32_t)(prod1 >> 32) ^ x[1] ^ k0,
            (uint32_t)prod1,
            (uint32_t)(prod0 >> 32) ^ x[3] ^ k1,
            (uint32_t)prod0,
        };
        for (int w = 0; w < 4; ++w)
            x[w] = y[w];
    }
    for (int w = 0; w < 4; ++w)
        out[w] = x[w];
}

/* Exported for the known-answer tests of the generator. */
void attn_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    philox4x32_10(ctr, key, out);
}

struct dropout_cfg {
    int on;
    uint32_t thr;        /* keep when the 16-bit draw is >= thr */
    uint32_t key[2];
    uint32_t offset;
    uint32_t bh;         /* flat (sequence, head) index */
    double keep_scale;   /* 1 / (1 - p) */
};

/* z_ij of the dropout reading above. */
static int kept(const struct dropout_cfg *dc, long long i, long long j)
{
    const uint32_t ctr[4] = {(uint32_t)(j / 8), (uint32_t)i, dc->bh, dc->offset};
    uint32_t r[4];
    philox4x32_10(ctr, dc->key, r);
    const int t = (int)(j % 8);
    const uint32_t draw = (r[t / 2] >> (16 * (t % 2))) & 0xFFFFu;
    return draw >= dc->thr;
}

/* The admissible keys of query i, J_i = { lo .. hi }: 0 <= j < S and
 * i - wl <= j <= i + wr, a negative wl or wr leaving that side unbounded. */
static void key_range(long long S, long long i, long long wl, long long wr,
                      long long *lo, long long *hi)
{
    *lo = 0;
    if (wl >= 0 && i - wl > 0)
        *lo = i - wl;
    *hi = S - 1;
    if (wr >= 0 && i + wr < S - 1)
        *hi = i + wr;
}

/* One query row over keys lo..hi: writes D outputs and the log-sum-exp. `s`
 * and `p` are caller-provided scratch arrays of at least hi-lo+1 doubles. */
static void attend_row(const double *qi, const double *k, const double *v,
                       long long D, long long i, long long lo, long long hi,
                       double scale, const struct dropout_cfg *dc,
                       double *s, double *p, double *o_row, double *lse_out)
{
    const long long n_keys = hi - lo + 1;   /* s[t], p[t] belong to key j = lo + t */

    /* scores */
    for (long long t = 0; t < n_keys; ++t) {
        const double *kj = k + (lo + t) * D;
        double dot = 0.0;
        for (long long d = 0; d < D; ++d)
            dot += qi[d] * kj[d];
        s[t] = scale * dot;
    }

    /* row max */
    double M = s[0];
    for (long long t = 1; t < n_keys; ++t)
        if (s[t] > M)
            M = s[t];

    /* normaliser */
    double l = 0.0;
    for (long long t = 0; t < n_keys; ++t)
        l += exp(s[t] - M);

    /* probabilities */
    for (long long t = 0; t < n_keys; ++t)
        p[t] = exp(s[t] - M) / l;

    /* dropout on P (the normaliser above is unaffected) */
    if (dc && dc->on)
        for (long long t = 0; t < n_keys; ++t)
            p[t] = kept(dc, i, lo + t) ? p[t] * dc->keep_scale : 0.0;

    /* output row: O_i = sum_j P_ij v_j */
    for (long long d = 0; d < D; ++d) {
        double acc = 0.0;
        for (long long t = 0; t < n_keys; ++t)
            acc += p[t] * v[(lo + t) * D + d];
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
            long long head = r / S, i = r % S, lo, hi;
            const long long base = head * (long long)S * D;
            key_range(S, i, -1, causal ? 0 : -1, &lo, &hi);
            attend_row(q + base + i * D, k + base, v + base, D, i, lo, hi, scale, NULL,
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
            long long head = r / S, i = r % S, lo, hi;
            const long long base = head * (long long)S * D;
            key_range(S, i, -1, causal ? 0 : -1, &lo, &hi);
            attend_row(q + base + i * D, k + base, v + base, D, i, lo, hi, scale, NULL,
                       s, p, O + (long long)n * D, LSE + n);
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* One problem: the S query rows q [S, D] of one (sequence, head) against the
 * S keys and values k, v [S, D] of its K/V head, with a local window (wl, wr)
 * and optional dropout (drop != 0: threshold thr, Philox key (key0, key1),
 * counter words bh and offset, kept weights scaled by keep_scale). With
 * rows == NULL every row is computed and O is [S, D], LSE [S]; otherwise only
 * rows[0..nrows-1] (indices into 0..S-1) and O is [nrows, D], LSE [nrows]. */
int attn_oracle_head_f64(const double *q, const double *k, const double *v,
                         int S, int D, int wl, int wr, double scale,
                         int drop, uint32_t thr, uint32_t key0, uint32_t key1,
                         uint32_t bh, uint32_t offset, double keep_scale,
                         const long long *rows, int nrows,
                         double *O, double *LSE, int nthreads)
{
    if (!q || !k || !v || !O || !LSE || S < 1 || D < 1 || wl < -1 || wr < -1)
        return -1;
    if (rows) {
        if (nrows < 0)
            return -1;
        for (int n = 0; n < nrows; ++n)
            if (rows[n] < 0 || rows[n] >= S)
                return -1;
    } else {
        nrows = S;
    }
    struct dropout_cfg dc = {drop != 0, thr, {key0, key1}, offset, bh, keep_scale};
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
#pragma omp for schedule(dynamic, 4)
        for (int n = 0; n < nrows; ++n) {
            if (!s || !p)
                continue;
            const long long i = rows ? rows[n] : n;
            long long lo, hi;
            key_range(S, i, wl, wr, &lo, &hi);
            attend_row(q + i * D, k, v, D, i, lo, hi, scale, &dc,
                       s, p, O + (long long)n * D, LSE + n);
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* Number of threads a parallel region of this library uses by default. */
int attn_oracle_max_threads(void) { return omp_get_max_threads(); }
