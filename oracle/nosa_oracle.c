/*
 * NOSA decode-step oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU path neither links
 * nor calls it, and it shares no code with the GPU path.
 *
 * Plain, single-threaded fp64 loops. Inputs arrive as float32 arrays whose
 * values are the exact input values (bfloat16 inputs are bfloat16-exact
 * float32); every arithmetic step below is done in double and nothing is
 * rounded back. It follows "NOSA: Native and Offloadable Sparse Attention"
 * (technical summary pages, section Methodology, subsection "1. Algorithm:
 * NOSA"), step by step, for one row = one (batch, KV head) pair:
 *
 *   pooling      two-stage pooling: mean inside each sub-block, then max over
 *                the block's sub-blocks (bullet "Block-Wise Implementation");
 *   Gamma_e      query-agnostic selection of k_e blocks by their pooled,
 *                pre-exponential eviction scores (bullets "Dual-Selection
 *                Mechanism" and "ED-DMA"); with static per-token scores and
 *                a candidate set that only grows, the k_e greatest candidates
 *                are exactly what a never-readmit eviction policy keeps, so
 *                the oracle uses that stateless definition;
 *   Gamma_q      the k_q greatest of the remaining candidates by the
 *                query-aware pooled score (same bullet, "Query-Aware
 *                Selection");
 *   attention    plain softmax over the tokens of the selected blocks plus the
 *                newest (partial) block, with the eviction score added to the
 *                logit so that its exponential happens only in the softmax
 *                (bullet "ED-DMA").
 *
 * Readings of points the pages leave open (the group of G query heads sums
 * its per-head block scores; per-head max over sub-blocks comes before that
 * sum; scores are scaled by `scale` with no softmax; the newest block is
 * always attended and is not a candidate; equal scores rank the lower block
 * index first; pooled keys and pooled queries are the exact means) are
 * listed in the repository's design notes. Nothing is rounded by default.
 * One variant is offered for a stack that stores its pooled keys in the
 * model's dtype: with `pooled_bf16` set, each pooled mean (key, and the
 * pooled query of a prefill query block) is the exact mean rounded to the
 * nearest bfloat16, ties to even; that is a quantisation of the stored
 * pooled values, not an arithmetic shortcut, and the score is still
 * computed in double from the quantised means.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* x rounded to the nearest bfloat16 value, ties to the even one. bfloat16
   has 8 significant bits and float32's exponent range: in the binade
   [2^(e-1), 2^e) its values are the multiples of 2^(e-8), and below the
   smallest normal (2^-126) the multiples of 2^-133. Rounding is to the
   nearest such multiple (rint: ties to even under the default rounding
   mode). Results beyond the largest finite bfloat16 do not occur for means
   of bfloat16 inputs. */
double oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    int e;
    frexp(x, &e);
    int q = e - 8;
    if (q < -133)
        q = -133;
    double ulp = ldexp(1.0, q);
    return rint(x / ulp) * ulp;
}

/* Sub-block mean of keys: kbar[i*D + d] = mean over the `sub` tokens of
   sub-block i of block j of K[token][d]; K is [tokens][D] with row stride D.
   pooled_bf16: the mean is then rounded to the nearest bfloat16. */
void oracle_pool_keys(const float *K, int D, int block, int sub, int j, int pooled_bf16,
                      double *kbar)
{
    int m = block / sub;
    for (int i = 0; i < m; ++i) {
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int u = 0; u < sub; ++u)
                s += (double)K[(int64_t)(j * block + i * sub + u) * D + d];
            double mean = s / (double)sub;
            kbar[i * D + d] = pooled_bf16 ? oracle_round_bf16(mean) : mean;
        }
    }
}

/* Eviction head of one KV head for one token (Methodology, "Dual-Selection
   Mechanism": a head that scores tokens independently of the query; "ED-DMA":
   the score stays pre-exponential). Reading taken, the pages giving no form:
   a linear head on the token's hidden state, e = x . w + bias, one logit per
   KV head. Summed in double. */
double oracle_evict_logit(const float *x, const float *w, int hidden, double bias)
{
    double s = 0.0;
    for (int i = 0; i < hidden; ++i)
        s += (double)x[i] * (double)w[i];
    return s + bias;
}

/* Pooled eviction score of block j: max over its sub-blocks of the mean of
   the per-token (pre-exponential) eviction scores. */
double oracle_block_evict(const float *e, int block, int sub, int j)
{
    int m = block / sub;
    double best = -INFINITY;
    for (int i = 0; i < m; ++i) {
        double s = 0.0;
        for (int u = 0; u < sub; ++u)
            s += (double)e[j * block + i * sub + u];
        double mean = s / (double)sub;
        if (mean > best)
            best = mean;
    }
    return best;
}

/* Query-aware pooled score of block j for a group of G query heads q[h][D]
   (double): sum over heads of (max over sub-blocks of scale * q_h . kbar_i). */
double oracle_block_score(const double *q, int G, int D, const float *K, int block, int sub,
                          int j, double scale, int pooled_bf16)
{
    int m = block / sub;
    double *kbar = (double *)malloc(sizeof(double) * (size_t)m * (size_t)D);
    oracle_pool_keys(K, D, block, sub, j, pooled_bf16, kbar);
    double total = 0.0;
    for (int h = 0; h < G; ++h) {
        double best = -INFINITY;
        for (int i = 0; i < m; ++i) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += q[h * D + d] * kbar[i * D + d];
            double a = scale * dot;
            if (a > best)
                best = a;
        }
        total += best;
    }
    free(kbar);
    return total;
}

/* a ranks above b: greater score, or equal score and lower index. */
static int ranks_above(const double *x, int a, int b)
{
    return x[a] > x[b] || (x[a] == x[b] && a < b);
}

/* The k greatest of the allowed indices 0..n-1 under the order above, by
   repeated selection of the best remaining one. Writes them to out[] in
   ascending index order and returns how many there are (min(k, #allowed)).
   allowed == NULL allows every index. */
int oracle_topk(const double *x, const unsigned char *allowed, int n, int k, int *out)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)(n > 0 ? n : 1), 1);
    int cnt = 0;
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int j = 0; j < n; ++j) {
            if ((allowed && !allowed[j]) || taken[j])
                continue;
            if (best < 0 || ranks_above(x, j, best))
                best = j;
        }
        if (best < 0)
            break;
        taken[best] = 1;
        ++cnt;
    }
    int w = 0;
    for (int j = 0; j < n; ++j)
        if (taken[j])
            out[w++] = j;
    free(taken);
    return cnt;
}

/* Softmax attention of G query heads over an explicit token list.
   z_i = scale * q_h . K[tok_i] + e[tok_i]; out[h] = sum_i softmax(z)_i V[tok_i].
   The eviction score enters as an additive logit, so its exponential is taken
   only inside the softmax. Tokens are visited in the order given. */
void oracle_attend_tokens(const float *q, int G, int D, const float *K, const float *V,
                          const float *e, const int *tok, int n_tok, double scale, double *out)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
    for (int h = 0; h < G; ++h) {
        double mx = -INFINITY;
        for (int i = 0; i < n_tok; ++i) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += (double)q[h * D + d] * (double)K[(int64_t)tok[i] * D + d];
            z[i] = scale * dot + (e ? (double)e[tok[i]] : 0.0);
            if (z[i] > mx)
                mx = z[i];
        }
        double den = 0.0;
        for (int i = 0; i < n_tok; ++i) {
            z[i] = exp(z[i] - mx);
            den += z[i];
        }
        for (int d = 0; d < D; ++d) {
            double num = 0.0;
            for (int i = 0; i < n_tok; ++i)
                num += z[i] * (double)V[(int64_t)tok[i] * D + d];
            out[h * D + d] = num / den;
        }
    }
    free(z);
}

/* One decode step for one row.
 *
 * n_tokens tokens exist (the newest one was appended this step). Candidate
 * blocks are 0..c-1 with c = (n_tokens - 1) / block; block c holds tokens
 * [c*block, n_tokens) and is always attended.
 *
 * Inputs: q [G][D], K and V [>= n_tokens][D], e [>= n_tokens].
 * Outputs: ge[] (Gamma_e, ascending, returns its size in *n_ge), gq[]
 * (Gamma_q, ascending, *n_gq), out [G][D]; E[c] and S[c] receive every
 * candidate's pooled eviction and query-aware scores when not NULL.
 * Returns c. */
int oracle_step_row(int n_tokens, int G, int D, int block, int sub, int k_e, int k_q,
                    double scale, int pooled_bf16, const float *q, const float *K,
                    const float *V, const float *e, int *ge, int *n_ge, int *gq, int *n_gq,
                    double *out, double *E, double *S)
{
    int c = (n_tokens - 1) / block;
    int cc = c > 0 ? c : 1;
    double *Eb = (double *)malloc(sizeof(double) * (size_t)cc);
    double *Sb = (double *)malloc(sizeof(double) * (size_t)cc);
    unsigned char *rest = (unsigned char *)malloc((size_t)cc);

    double *qd = (double *)malloc(sizeof(double) * (size_t)G * (size_t)D);
    for (int i = 0; i < G * D; ++i)
        qd[i] = (double)q[i];
    for (int j = 0; j < c; ++j) {
        Eb[j] = oracle_block_evict(e, block, sub, j);
        Sb[j] = oracle_block_score(qd, G, D, K, block, sub, j, scale, pooled_bf16);
    }
    free(qd);

    /* Gamma_e: the k_e greatest candidates by pooled eviction score. */
    *n_ge = oracle_topk(Eb, NULL, c, k_e, ge);

    /* Gamma_q: the k_q greatest of the candidates outside Gamma_e. */
    for (int j = 0; j < c; ++j)
        rest[j] = 1;
    for (int i = 0; i < *n_ge; ++i)
        rest[ge[i]] = 0;
    *n_gq = oracle_topk(Sb, rest, c, k_q, gq);

    /* Tokens attended: every token of every selected block, ascending, then
       the newest block's tokens. */
    unsigned char *pick = (unsigned char *)calloc((size_t)cc, 1);
    for (int i = 0; i < *n_ge; ++i)
        pick[ge[i]] = 1;
    for (int i = 0; i < *n_gq; ++i)
        pick[gq[i]] = 1;
    int *tok = (int *)malloc(sizeof(int) * (size_t)((*n_ge + *n_gq) * block + block));
    int nt = 0;
    for (int j = 0; j < c; ++j)
        if (pick[j])
            for (int u = 0; u < block; ++u)
                tok[nt++] = j * block + u;
    for (int u = c * block; u < n_tokens; ++u)
        tok[nt++] = u;
    oracle_attend_tokens(q, G, D, K, V, e, tok, nt, scale, out);

    if (E)
        memcpy(E, Eb, sizeof(double) * (size_t)c);
    if (S)
        memcpy(S, Sb, sizeof(double) * (size_t)c);
    free(tok);
    free(pick);
    free(rest);
    free(Sb);
    free(Eb);
    return c;
}

/* ------------------------------------------------------------------------
 * Prefill (training-time forward) with the same selection per query block.
 * Readings taken, the pages describing the trainable mechanism but not its
 * forward over a whole sequence: queries come in blocks of `block` tokens;
 * query block i selects among the complete blocks before it (0..i-1) exactly
 * as a decode step with those candidates does (Gamma_e: the k_e greatest
 * pooled eviction scores; Gamma_q: the k_q greatest of the rest by the
 * query-aware score), the query-aware score being that of the block's pooled
 * query (the exact mean of its tokens' queries per head; rounded to the
 * nearest bfloat16 with `pooled_bf16`, as the pooled keys are); every query
 * token of the block attends the tokens of the selected blocks and, causally,
 * the tokens of its own block up to itself.
 * ------------------------------------------------------------------------ */

/* Pooled query of n tokens q[u][h][d] (u < n): per (h, d) the mean over u
   (rounded to the nearest bfloat16 with pooled_bf16). */
void oracle_pool_queries(const float *q, int n, int G, int D, int pooled_bf16, double *out)
{
    for (int h = 0; h < G; ++h)
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int u = 0; u < n; ++u)
                s += (double)q[((int64_t)u * G + h) * D + d];
            double mean = s / (double)n;
            out[h * D + d] = pooled_bf16 ? oracle_round_bf16(mean) : mean;
        }
}

/* Query block i of a row's prefill (N tokens, q [N][G][D], K and V [N][D],
   e [N]): its tokens lo = i*block .. hi-1 select among the blocks before it,
   Gamma_e by pooled eviction score and Gamma_q by the score of the block's
   pooled query, and attend the selected blocks' tokens plus, causally, their
   own block up to themselves. Writes out [hi - lo][G][D] and the ascending
   selection sel[0 .. k_e + k_q - 1] (-1 padded). */
void oracle_prefill_qblock(int N, int G, int D, int block, int sub, int k_e, int k_q,
                           double scale, int pooled_bf16, const float *q, const float *K,
                           const float *V, const float *e, int i, double *out, int *sel)
{
    int k = k_e + k_q;
    int c = i;  /* candidates: blocks 0..i-1 */
    int lo = i * block, hi = lo + block < N ? lo + block : N;
    int cmax = c > 0 ? c : 1;
    double *Eb = (double *)malloc(sizeof(double) * (size_t)cmax);
    double *Sb = (double *)malloc(sizeof(double) * (size_t)cmax);
    unsigned char *rest = (unsigned char *)malloc((size_t)cmax);
    unsigned char *pick = (unsigned char *)malloc((size_t)cmax);
    int *ge = (int *)malloc(sizeof(int) * (size_t)(k_e > 0 ? k_e : 1));
    int *gq = (int *)malloc(sizeof(int) * (size_t)(k_q > 0 ? k_q : 1));
    int *tok = (int *)malloc(sizeof(int) * (size_t)(k * block + block));
    double *qbar = (double *)malloc(sizeof(double) * (size_t)G * (size_t)D);
    for (int j = 0; j < c; ++j)
        Eb[j] = oracle_block_evict(e, block, sub, j);
    oracle_pool_queries(q + (int64_t)lo * G * D, hi - lo, G, D, pooled_bf16, qbar);
    for (int j = 0; j < c; ++j)
        Sb[j] = oracle_block_score(qbar, G, D, K, block, sub, j, scale, pooled_bf16);
    int n_ge = oracle_topk(Eb, NULL, c, k_e, ge);
    for (int j = 0; j < c; ++j)
        rest[j] = 1;
    for (int t = 0; t < n_ge; ++t)
        rest[ge[t]] = 0;
    int n_gq = oracle_topk(Sb, rest, c, k_q, gq);
    for (int j = 0; j < c; ++j)
        pick[j] = 0;
    for (int t = 0; t < n_ge; ++t)
        pick[ge[t]] = 1;
    for (int t = 0; t < n_gq; ++t)
        pick[gq[t]] = 1;
    int ns = 0, nt = 0;
    for (int j = 0; j < c; ++j)
        if (pick[j]) {
            sel[ns++] = j;
            for (int u = 0; u < block; ++u)
                tok[nt++] = j * block + u;
        }
    for (int t = ns; t < k; ++t)
        sel[t] = -1;
    for (int p = lo; p < hi; ++p) {
        int m = nt;
        for (int u = lo; u <= p; ++u)
            tok[m++] = u;
        oracle_attend_tokens(q + (int64_t)p * G * D, G, D, K, V, e, tok, m, scale,
                             out + (int64_t)(p - lo) * G * D);
    }
    free(qbar);
    free(tok);
    free(gq);
    free(ge);
    free(pick);
    free(rest);
    free(Sb);
    free(Eb);
}

/* Prefill of one row: every query block in turn. Writes out [N][G][D] and
   sel [n_qb][k_e + k_q]. Returns the number of query blocks. */
int oracle_prefill_row(int N, int G, int D, int block, int sub, int k_e, int k_q, double scale,
                       int pooled_bf16, const float *q, const float *K, const float *V,
                       const float *e, double *out, int *sel)
{
    int nqb = (N + block - 1) / block;
    int k = k_e + k_q;
    for (int i = 0; i < nqb; ++i)
        oracle_prefill_qblock(N, G, D, block, sub, k_e, k_q, scale, pooled_bf16, q, K, V, e, i,
                              out + (int64_t)i * block * G * D, sel + i * k);
    return nqb;
}
