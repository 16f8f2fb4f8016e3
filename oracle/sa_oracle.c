/*
 * sa_oracle.c -- plain fp64 CPU reference for causal factorized sparse
 * self-attention (strided and fixed patterns).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library; its pattern definitions below are written out on their
 * own.
 *
 * What it computes (sources):
 *   - "OpenAI Sparse Transformer" (agentlenshq.com), section "Sparse Attention
 *     and Algorithmic Complexity": every output position computes weights
 *     only over a subset of the input positions.
 *   - same page, section "Factorized Attention Patterns", and
 *     "Генеративное моделирование с разреженными трансформерами"
 *     (pcnews.ru), section "Разреженное внимание": the strided pattern
 *     (a position attends its row and its column) and the fixed pattern
 *     (a fixed column plus the elements after the latest column element).
 *     Formalised as: strided A  0 <= i-j < l;  strided B  (i-j) mod l == 0;
 *     fixed A  floor(j/l) == floor(i/l);  fixed B  j mod l >= l-c;
 *     every pattern causal (j <= i).  A fifth, "dense causal" (j <= i only),
 *     is the full attention the pages compare against.
 *   - "희소 어텐션 (Sparse Attention)" (molayo1419.me): scores are query-key
 *     dot products, followed by a softmax so that the weights sum to one.
 *   - "[논문 리뷰] Generating Long Sequences with Sparse Transformers"
 *     (nubint.ai), ABSTRACT item (b) and "제안 방법": the backward pass
 *     recomputes the attention matrix instead of storing it.  The gradients
 *     here are the exact analytic gradients of L = sum(dO * O).
 *
 * Readings where the pages are silent:
 *   - the score is scale * (q_i . k_j) with an explicit scale argument;
 *   - a row with no allowed key (fixed B, rows i with i < l-c) has O = 0,
 *     lse = -inf and contributes no gradient;
 *   - lse is the natural log-sum-exp of the scaled scores.
 *
 * Everything is fp64, one (batch, head) slice at a time, OpenMP over rows or
 * over key columns.  Allowed pairs are found by testing the predicate for
 * every j <= i; nothing is derived from a block layout.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_STRIDED_A 0
#define ORC_STRIDED_B 1
#define ORC_FIXED_A 2
#define ORC_FIXED_B 3
#define ORC_DENSE 4

/* The pattern predicates, one line each, straight from their definitions. */
int oracle_allowed(int pattern, int64_t i, int64_t j, int64_t l, int64_t c)
{
    if (j < 0 || j > i) return 0; /* causal */
    switch (pattern) {
    case ORC_STRIDED_A: return (i - j) < l;
    case ORC_STRIDED_B: return ((i - j) % l) == 0;
    case ORC_FIXED_A: return (j / l) == (i / l);
    case ORC_FIXED_B: return (j % l) >= (l - c);
    case ORC_DENSE: return 1;
    default: return 0;
    }
}

static double dot(const double* a, const double* b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/* Row i of the forward pass.  js/ss are scratch of length >= i+1.
 * Writes o_i (d values) and returns lse_i. */
static double fwd_row(int pattern, int64_t l, int64_t c, int64_t i, int d, double scale,
                      const double* q, const double* k, const double* v, double* o_i,
                      int64_t* js, double* ss)
{
    int64_t cnt = 0;
    for (int64_t j = 0; j <= i; ++j) {
        if (!oracle_allowed(pattern, i, j, l, c)) continue;
        js[cnt] = j;
        ss[cnt] = scale * dot(q + i * d, k + j * d, d);
        ++cnt;
    }
    for (int t = 0; t < d; ++t) o_i[t] = 0.0;
    if (cnt == 0) return -INFINITY;
    double m = ss[0];
    for (int64_t a = 1; a < cnt; ++a) if (ss[a] > m) m = ss[a];
    double sum = 0.0;
    for (int64_t a = 0; a < cnt; ++a) sum += exp(ss[a] - m);
    double lse = m + log(sum);
    for (int64_t a = 0; a < cnt; ++a) {
        double p = exp(ss[a] - lse);
        const double* vj = v + js[a] * d;
        for (int t = 0; t < d; ++t) o_i[t] += p * vj[t];
    }
    return lse;
}

/* Forward for one head over the listed rows (rows == NULL: all n rows).
 * q,k,v: [n][d] row-major; o: [n][d]; lse: [n].  Only listed rows are written. */
void oracle_head_fwd(int pattern, int64_t l, int64_t c, int64_t n, int d, double scale,
                     const double* q, const double* k, const double* v,
                     const int64_t* rows, int64_t nrows, double* o, double* lse)
{
    int64_t count = rows ? nrows : n;
#pragma omp parallel
    {
        int64_t* js = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* ss = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(dynamic, 16)
        for (int64_t a = 0; a < count; ++a) {
            int64_t i = rows ? rows[a] : a;
            lse[i] = fwd_row(pattern, l, c, i, d, scale, q, k, v, o + i * d, js, ss);
        }
        free(js);
        free(ss);
    }
}

/* Backward for one head.
 *   Given q, k, v, dout (all [n][d]) it recomputes O and lse in fp64, then
 *     D_i   = sum_t dO_it O_it
 *     P_ij  = exp(s_ij - lse_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_{j in S_i} dS_ij k_j
 *     dK_j  = scale * sum_{i : j in S_i} dS_ij q_i
 *     dV_j  = sum_{i : j in S_i} P_ij dO_i
 *   qrows/kcols select which dQ rows and which dK/dV rows are produced
 *   (NULL: all).  o_out and lse_out (may be NULL) receive the recomputed
 *   forward for every row that was needed. */
void oracle_head_bwd(int pattern, int64_t l, int64_t c, int64_t n, int d, double scale,
                     const double* q, const double* k, const double* v, const double* dout,
                     const int64_t* qrows, int64_t nq, const int64_t* kcols, int64_t nk,
                     double* dq, double* dk, double* dv, double* o_out, double* lse_out)
{
    int64_t cq = qrows ? nq : n;
    int64_t ck = kcols ? nk : n;
    /* Which rows need lse_i and D_i. */
    unsigned char* need = (unsigned char*)calloc((size_t)n, 1);
    for (int64_t a = 0; a < cq; ++a) need[qrows ? qrows[a] : a] = 1;
    for (int64_t a = 0; a < ck; ++a) {
        int64_t j = kcols ? kcols[a] : a;
        for (int64_t i = j; i < n; ++i)
            if (oracle_allowed(pattern, i, j, l, c)) need[i] = 1;
    }
    double* o = (double*)calloc((size_t)(n * d), sizeof(double));
    double* lse = (double*)malloc(sizeof(double) * (size_t)n);
    double* D = (double*)malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) { lse[i] = -INFINITY; D[i] = 0.0; }

#pragma omp parallel
    {
        int64_t* js = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* ss = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            if (!need[i]) continue;
            lse[i] = fwd_row(pattern, l, c, i, d, scale, q, k, v, o + i * d, js, ss);
            D[i] = dot(dout + i * d, o + i * d, d);
        }
        free(js);
        free(ss);
    }

    /* dQ, one row at a time. */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t a = 0; a < cq; ++a) {
        int64_t i = qrows ? qrows[a] : a;
        double* g = dq + i * d;
        for (int t = 0; t < d; ++t) g[t] = 0.0;
        if (isinf(lse[i])) continue; /* empty row */
        for (int64_t j = 0; j <= i; ++j) {
            if (!oracle_allowed(pattern, i, j, l, c)) continue;
            double p = exp(scale * dot(q + i * d, k + j * d, d) - lse[i]);
            double dp = dot(dout + i * d, v + j * d, d);
            double ds = p * (dp - D[i]);
            for (int t = 0; t < d; ++t) g[t] += scale * ds * k[j * d + t];
        }
    }

    /* dK and dV, one key column at a time. */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t a = 0; a < ck; ++a) {
        int64_t j = kcols ? kcols[a] : a;
        double* gk = dk + j * d;
        double* gv = dv + j * d;
        for (int t = 0; t < d; ++t) { gk[t] = 0.0; gv[t] = 0.0; }
        for (int64_t i = j; i < n; ++i) {
            if (!oracle_allowed(pattern, i, j, l, c)) continue;
            double p = exp(scale * dot(q + i * d, k + j * d, d) - lse[i]);
            double dp = dot(dout + i * d, v + j * d, d);
            double ds = p * (dp - D[i]);
            for (int t = 0; t < d; ++t) {
                gv[t] += p * dout[i * d + t];
                gk[t] += scale * ds * q[i * d + t];
            }
        }
    }

    if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)(n * d));
    if (lse_out) memcpy(lse_out, lse, sizeof(double) * (size_t)n);
    free(need);
    free(o);
    free(lse);
    free(D);
}

/* Dense boolean mask of the pattern, mask[i*n + j] in {0,1}, for small n. */
void oracle_mask_dense(int pattern, int64_t l, int64_t c, int64_t n, unsigned char* mask)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) mask[i * n + j] = (unsigned char)oracle_allowed(pattern, i, j, l, c);
}

/* Number of allowed keys of every row, cnt[i] = |S_i|. */
void oracle_row_counts(int pattern, int64_t l, int64_t c, int64_t n, int64_t* cnt)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i) {
        int64_t s = 0;
        for (int64_t j = 0; j <= i; ++j) s += oracle_allowed(pattern, i, j, l, c);
        cnt[i] = s;
    }
}

/* Block view of the pattern for block size T (n % T == 0), straight from the
 * predicate: for query block qb (rows qb*T..qb*T+T-1) and every key block kb
 * it tests all T*T elements.  Output, for query block qb:
 *   nblk[qb]                       number of key blocks with any allowed element
 *   kbs[qb*nkb + a], a < nblk[qb]  those key blocks, ascending
 *   bits[(qb*nkb + a)*T*T + r*T + s] the element mask of that block (0/1)
 * Callers size kbs as nqb*nkb and bits as nqb*nkb*T*T; only suitable for
 * moderate n. */
void oracle_block_layout(int pattern, int64_t l, int64_t c, int64_t n, int64_t T,
                         int64_t* nblk, int64_t* kbs, unsigned char* bits)
{
    int64_t nb = n / T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t qb = 0; qb < nb; ++qb) {
        int64_t cnt = 0;
        for (int64_t kb = 0; kb < nb; ++kb) {
            unsigned char* tile = bits + (qb * nb + cnt) * T * T;
            int any = 0;
            for (int64_t r = 0; r < T; ++r)
                for (int64_t s = 0; s < T; ++s) {
                    int a = oracle_allowed(pattern, qb * T + r, kb * T + s, l, c);
                    tile[r * T + s] = (unsigned char)a;
                    any |= a;
                }
            if (any) kbs[qb * nb + cnt++] = kb;
        }
        nblk[qb] = cnt;
    }
}

/* Sparse block view for large n: the same definition as oracle_block_layout,
 * but it only reports, per query block, the allowed key blocks and the number
 * of allowed elements in each, and the 64-bit words of each block's mask in
 * row-major bit order (bit (r*T+s) mod 64 of word (r*T+s)/64).
 *   Pass 1 (words == NULL): fills nblk[qb] only.
 *   Pass 2: kbs/pop/words sized from the prefix sum of nblk, with
 *   off[qb] the first slot of query block qb. */
void oracle_block_layout_sparse(int pattern, int64_t l, int64_t c, int64_t n, int64_t T,
                                int64_t* nblk, const int64_t* off, int64_t* kbs, int64_t* pop,
                                uint64_t* words)
{
    int64_t nb = n / T;
    int64_t nw = (T * T + 63) / 64;
#pragma omp parallel
    {
        uint64_t* tile = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)nw);
#pragma omp for schedule(dynamic, 1)
        for (int64_t qb = 0; qb < nb; ++qb) {
            int64_t cnt = 0;
            for (int64_t kb = 0; kb <= qb; ++kb) {
                int64_t np = 0;
                memset(tile, 0, sizeof(uint64_t) * (size_t)nw);
                for (int64_t r = 0; r < T; ++r)
                    for (int64_t s = 0; s < T; ++s)
                        if (oracle_allowed(pattern, qb * T + r, kb * T + s, l, c)) {
                            int64_t e = r * T + s;
                            tile[e / 64] |= (uint64_t)1 << (e % 64);
                            ++np;
                        }
                if (np == 0) continue;
                if (words) {
                    int64_t slot = off[qb] + cnt;
                    kbs[slot] = kb;
                    pop[slot] = np;
                    memcpy(words + slot * nw, tile, sizeof(uint64_t) * (size_t)nw);
                }
                ++cnt;
            }
            nblk[qb] = cnt;
        }
        free(tile);
    }
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of OpenMP threads a parallel region here will use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
