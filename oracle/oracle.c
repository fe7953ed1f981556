/*
 * CPU oracle for dynamic block-sparse video attention -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously correct fp64 loops.  Only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg use this file; the product path
 * never links or calls it, and it shares no code with the HIP library.
 *
 * What it computes follows the NABLA summary page ("NABLA: Neighborhood
 * Adaptive Block-Level Attention", section "Methodologie : NABLA"):
 *   - Sous-echantillonnage: Q and K are mean-pooled per block of tokens;
 *   - Attention Reduite: a full attention map (softmax over every key block)
 *     is computed on the pooled vectors;
 *   - Seuil CDF: per row of that map, blocks are kept by the cumulative
 *     distribution against the threshold thr;
 *   - Expansion: the block mask says which 64x64 token tiles are computed;
 *   - Integration Hybride avec STA: the final mask is the union of the
 *     content mask and a static sliding-tile window (M = M_nabla OR M_STA);
 * followed by exact softmax attention of every query token over the tokens of
 * its kept key blocks.
 *
 * Readings taken where the page is silent (each restated in the design notes):
 *   - pooled scores use the same scale as the attention, 1/sqrt(d) by default;
 *   - the softmax of the reduced map runs over all key blocks, no causal mask;
 *   - CDF rule: blocks are ordered by probability descending, ties broken by
 *     the lower block index; with E(j) the mass of the blocks strictly before
 *     j, block j is kept iff E(j) < thr.  This is the page's "cumulative
 *     probability above 1 - thr" counted from the small end, and it keeps the
 *     block that makes the mass reach thr;
 *   - thr >= 1 keeps every block (the literal rule could drop blocks whose
 *     probability underflows, which would not be dense attention);
 *   - the window is a box of radius (wt, wh, ww) in block coordinates,
 *     clipped at the grid edges, without wrap or shift;
 *   - a query row with no kept block gives O = 0 and LSE = -inf.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Sous-echantillonnage: xbar[b][c] = mean over the tokens of block b of x[token][c].
 * valid (optional, [nB * tpb], the same for every head): the tokens of a partial
 * tile that lie beyond the grid are padding; only the valid ones are averaged.  With
 * valid == NULL every token counts (mean over tpb).
 */
void oracle_pool(const float *x, int64_t nblocks, int64_t tpb, int64_t d, const uint8_t *valid, int64_t nB,
                 double *xbar)
{
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *vb = valid ? valid + (b % nB) * tpb : NULL;
        int64_t n = 0;
        for (int64_t t = 0; t < tpb; ++t) n += vb ? (vb[t] != 0) : 1;
        for (int64_t c = 0; c < d; ++c) {
            double s = 0.0;
            for (int64_t t = 0; t < tpb; ++t)
                if (!vb || vb[t]) s += (double)x[(b * tpb + t) * d + c];
            xbar[b * d + c] = s / (double)n;
        }
    }
}

typedef struct {
    double p;
    int64_t j;
} prob_idx;

/* Order for the CDF: larger probability first, then lower block index. */
static int by_prob_desc(const void *a, const void *b)
{
    const prob_idx *x = (const prob_idx *)a, *y = (const prob_idx *)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

/*
 * Attention Reduite + Seuil CDF + union with the window, for a list of rows.
 *
 * qbar: pooled query blocks [BH][nB][d], kbar: pooled key blocks [BH][nK][d] (fp64;
 * nK == nB for NABLA's square map, nK = 16 nB for AB-Attention's 4-token key blocks,
 * "Les trois techniques d'AB-Attention", third technique).  A row index
 * r = bh * nB + i names query block i of batch-head bh; its head is bh % H.  The
 * window applies to the square map only.
 * keep[k][j] (k-th listed row) receives bit 0 when the CDF rule keeps j and
 * bit 1 when the window contains j.  p_out / E_out (optional, [nrows][nB])
 * receive the row's probabilities and the exclusive mass E(j) in CDF order.
 */
void oracle_select_rows(const double *qbar, const double *kbar, int64_t H, int64_t nB, int64_t nK, int64_t d,
                        const int64_t *rows, int64_t nrows, double scale, const double *thr_head,
                        int64_t nT, int64_t nTy, int64_t nTx, int64_t wt, int64_t wh, int64_t ww,
                        uint8_t *keep, double *p_out, double *E_out)
{
    (void)nT;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)nK);
        prob_idx *ord = (prob_idx *)malloc(sizeof(prob_idx) * (size_t)nK);
#pragma omp for schedule(dynamic, 4)
        for (int64_t k = 0; k < nrows; ++k) {
            const int64_t r = rows[k];
            const int64_t bh = r / nB, i = r % nB;
            const double thr = thr_head[bh % H];
            const double *qi = qbar + (bh * nB + i) * d;
            uint8_t *kr = keep + k * nK;

            /* reduced attention map row: scaled dot products, then a softmax over all key blocks */
            double mx = -INFINITY;
            for (int64_t j = 0; j < nK; ++j) {
                const double *kj = kbar + (bh * nK + j) * d;
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += qi[c] * kj[c];
                s[j] = acc * scale;
                if (s[j] > mx) mx = s[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < nK; ++j) {
                s[j] = exp(s[j] - mx);
                z += s[j];
            }
            for (int64_t j = 0; j < nK; ++j) s[j] /= z;

            /* CDF: walk the blocks from the most probable; keep while the mass before is below thr */
            for (int64_t j = 0; j < nK; ++j) {
                ord[j].p = s[j];
                ord[j].j = j;
            }
            qsort(ord, (size_t)nK, sizeof(prob_idx), by_prob_desc);
            double before = 0.0;
            for (int64_t n = 0; n < nK; ++n) {
                const int64_t j = ord[n].j;
                kr[j] = (thr >= 1.0 || before < thr) ? 1 : 0;
                if (E_out) E_out[k * nK + j] = before;
                before += ord[n].p;
            }
            if (p_out)
                for (int64_t j = 0; j < nK; ++j) p_out[k * nK + j] = s[j];

            /* static window around the query block, in block coordinates (t, y, x) */
            if (wt >= 0 && wh >= 0 && ww >= 0 && nK == nB) {
                const int64_t ti = i / (nTy * nTx), yi = (i / nTx) % nTy, xi = i % nTx;
                for (int64_t j = 0; j < nB; ++j) {
                    const int64_t tj = j / (nTy * nTx), yj = (j / nTx) % nTy, xj = j % nTx;
                    if (llabs(tj - ti) <= wt && llabs(yj - yi) <= wh && llabs(xj - xi) <= ww)
                        kr[j] |= 2;
                }
            }
        }
        free(s);
        free(ord);
    }
}

/*
 * Exact attention over the kept tiles (Expansion): for every token n of query
 * block i, softmax over all tokens of the key blocks listed in the CSR row of
 * (bh, i), then the weighted sum of V.  Query blocks hold tpb tokens, key blocks
 * tk (tk == tpb for NABLA's tiles; tk = 4 for AB-Attention's 4-token key blocks,
 * whose kept blocks the kernel gathers into full tiles).
 *
 * q, k, v: [BH][nB*tpb][d] float32 (the exact values the GPU sees).
 * row_ptr/col_idx: CSR over rows r = bh * nB + i.  For each listed row, out
 * receives [tpb][d] fp64 and lse [tpb] the natural-log normaliser
 * log(sum_m exp(scale * q_n . k_m)).  An empty row yields O = 0, LSE = -inf.
 * w_sum (optional, [nrows][tpb]) receives the sum of the row's softmax weights.
 * col_bias (optional, one value per CSR entry) is added to the logits of every
 * key of that entry's block: the logit offset by which AB-Attention's sampling
 * ("SIP", section "Les trois techniques d'AB-Attention" of the AB-Attention
 * page) weighs a kept block by the inverse of its inclusion probability.
 * valid (optional, [nB * tpb], the same for every head): padding tokens of partial
 * tiles take no part as keys, and a padding query token gets O = 0, LSE = -inf.
 */
void oracle_attention_rows(const float *q, const float *k, const float *v, int64_t nB, int64_t tpb, int64_t tk,
                           int64_t d, const int64_t *row_ptr, const int32_t *col_idx,
                           const double *col_bias, const uint8_t *valid, const int64_t *rows, int64_t nrows,
                           double scale, double *out, double *lse, double *w_sum)
{
    const int64_t N = nB * tpb;
#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)N);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t kr = 0; kr < nrows; ++kr) {
            for (int64_t t = 0; t < tpb; ++t) {
                const int64_t r = rows[kr];
                const int64_t bh = r / nB, i = r % nB;
                const float *qn = q + (bh * N + i * tpb + t) * d;
                const int64_t beg = row_ptr[r], end = row_ptr[r + 1];
                double *o = out + (kr * tpb + t) * d;
                const int64_t m_count = (end - beg) * tk;
                if (m_count == 0 || (valid && !valid[i * tpb + t])) {
                    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                    lse[kr * tpb + t] = -INFINITY;
                    if (w_sum) w_sum[kr * tpb + t] = 0.0;
                    continue;
                }
                double mx = -INFINITY;
                int64_t m = 0;
                for (int64_t e = beg; e < end; ++e) {
                    const int64_t j = col_idx[e];
                    for (int64_t u = 0; u < tk; ++u, ++m) {
                        if (valid && !valid[j * tk + u]) {          /* padding key: no weight */
                            logit[m] = -INFINITY;
                            continue;
                        }
                        const float *km = k + (bh * N + j * tk + u) * d;
                        double a = 0.0;
                        for (int64_t c = 0; c < d; ++c) a += (double)qn[c] * (double)km[c];
                        logit[m] = a * scale + (col_bias ? col_bias[e] : 0.0);
                        if (logit[m] > mx) mx = logit[m];
                    }
                }
                double z = 0.0;
                for (int64_t mm = 0; mm < m_count; ++mm) {
                    logit[mm] = exp(logit[mm] - mx);
                    z += logit[mm];
                }
                for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
                double wsum = 0.0;
                m = 0;
                for (int64_t e = beg; e < end; ++e) {
                    const int64_t j = col_idx[e];
                    for (int64_t u = 0; u < tk; ++u, ++m) {
                        const float *vm = v + (bh * N + j * tk + u) * d;
                        const double w = logit[m] / z;
                        wsum += w;
                        for (int64_t c = 0; c < d; ++c) acc[c] += w * (double)vm[c];
                    }
                }
                for (int64_t c = 0; c < d; ++c) o[c] = acc[c];
                lse[kr * tpb + t] = mx + log(z);
                if (w_sum) w_sum[kr * tpb + t] = wsum;
            }
        }
        free(logit);
        free(acc);
    }
}

/*
 * Gradients of the block-sparse attention (the backward of the computation
 * above, for NABLA's training use: "Methodologie : NABLA" and the training
 * results of the NABLA summary page).  With P the softmax weights of query
 * token n over the tokens of its kept blocks and O_n = sum_m P_nm v_m, for an
 * upstream gradient dO:
 *   dV_m = sum_n P_nm dO_n
 *   dP_nm = dO_n . v_m,  D_n = dO_n . O_n,  dS_nm = P_nm (dP_nm - D_n)
 *   dQ_n = scale sum_m dS_nm k_m,  dK_m = scale sum_n dS_nm q_n.
 * D_n is the product of dO_n with the forward output.  A caller that holds that
 * output, rounded as it was stored, passes it as `out` [BH][N][d] and D_n uses it;
 * with out == NULL, O_n is recomputed here in fp64.
 * Partial tiles (`valid` [N], NULL when every slot is a token): the sums over n
 * and m above run over token slots only, so padding slots get zero gradients
 * and take no part in any other token's.
 * One head at a time (heads in parallel); within a head the rows are visited in
 * order, so the sums over n are in a fixed order.  Outputs are fp64 [BH][N][d].
 */
void oracle_attention_backward(const float *q, const float *k, const float *v, const float *dout,
                               const float *out, int64_t BH, int64_t nB, int64_t tpb, int64_t d,
                               const int64_t *row_ptr, const int32_t *col_idx, const uint8_t *valid,
                               double scale, double *dq, double *dk, double *dv)
{
    const int64_t N = nB * tpb;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)N);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < BH; ++bh) {
            const float *qh = q + bh * N * d, *kh = k + bh * N * d, *vh = v + bh * N * d, *gh = dout + bh * N * d;
            double *dqh = dq + bh * N * d, *dkh = dk + bh * N * d, *dvh = dv + bh * N * d;
            for (int64_t x = 0; x < N * d; ++x) dqh[x] = dkh[x] = dvh[x] = 0.0;
            for (int64_t i = 0; i < nB; ++i) {
                const int64_t r = bh * nB + i, beg = row_ptr[r], end = row_ptr[r + 1];
                const int64_t mc = (end - beg) * tpb;
                if (mc == 0) continue;
                for (int64_t t = 0; t < tpb; ++t) {
                    const int64_t n = i * tpb + t;
                    if (valid && !valid[n]) continue;               /* padding query: no gradient */
                    const float *qn = qh + n * d, *gn = gh + n * d;
                    /* weights P_nm over the kept tokens, in kept order (padding keys: none) */
                    double mx = -INFINITY;
                    int64_t m = 0;
                    for (int64_t e = beg; e < end; ++e)
                        for (int64_t u = 0; u < tpb; ++u, ++m) {
                            const int64_t mt = col_idx[e] * tpb + u;
                            if (valid && !valid[mt]) {
                                w[m] = 0.0;
                                continue;
                            }
                            const float *km = kh + mt * d;
                            double a = 0.0;
                            for (int64_t c = 0; c < d; ++c) a += (double)qn[c] * (double)km[c];
                            w[m] = a * scale;
                            if (w[m] > mx) mx = w[m];
                        }
                    double z = 0.0;
                    m = 0;
                    for (int64_t e = beg; e < end; ++e)
                        for (int64_t u = 0; u < tpb; ++u, ++m) {
                            if (valid && !valid[col_idx[e] * tpb + u]) continue;
                            w[m] = exp(w[m] - mx);
                            z += w[m];
                        }
                    for (int64_t mm = 0; mm < mc; ++mm) w[mm] /= z;
                    /* O_n and D_n */
                    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                    m = 0;
                    for (int64_t e = beg; e < end; ++e)
                        for (int64_t u = 0; u < tpb; ++u, ++m) {
                            if (valid && !valid[col_idx[e] * tpb + u]) continue;
                            const float *vm = vh + (col_idx[e] * tpb + u) * d;
                            for (int64_t c = 0; c < d; ++c) o[c] += w[m] * (double)vm[c];
                        }
                    if (out)
                        for (int64_t c = 0; c < d; ++c) o[c] = (double)out[(bh * N + n) * d + c];
                    double Dn = 0.0;
                    for (int64_t c = 0; c < d; ++c) Dn += (double)gn[c] * o[c];
                    /* dV, dP, dS, dQ, dK */
                    m = 0;
                    for (int64_t e = beg; e < end; ++e)
                        for (int64_t u = 0; u < tpb; ++u, ++m) {
                            const int64_t mt = col_idx[e] * tpb + u;
                            if (valid && !valid[mt]) continue;
                            const float *vm = vh + mt * d, *km = kh + mt * d;
                            double dp = 0.0;
                            for (int64_t c = 0; c < d; ++c) dp += (double)gn[c] * (double)vm[c];
                            const double ds = w[m] * (dp - Dn);
                            for (int64_t c = 0; c < d; ++c) {
                                dvh[mt * d + c] += w[m] * (double)gn[c];
                                dqh[n * d + c] += scale * ds * (double)km[c];
                                dkh[mt * d + c] += scale * ds * (double)qn[c];
                            }
                        }
                }
            }
        }
        free(w);
        free(o);
    }
}
