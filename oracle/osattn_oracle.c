/*
 * osattn_oracle.c -- plain, slow, obviously-correct CPU oracle for exact
 * scaled-dot-product attention and its gradient, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library: it includes only the C standard library and OpenMP.
 *
 * What it computes (the definitions, written out with no blocking, fusion or
 * online recurrence):
 *
 *   Forward -- TIGA-lang "Attention and dense relations" (注意力与稠密关系),
 *   equations of the sections on full attention (全量注意力，无掩码), the causal
 *   dense relation (因果稠密关系) and varlen causal attention
 *   (用图组合表达 varlen 因果注意力):
 *       s_hij  = <k_hj, q_hi> * scale                 (scale given; the pages
 *                                                      use D^-1/2)
 *       out_hi = sum_{j in A(i)} softmax_j(s_hi.) v_hj
 *   with the admitted key set A(i):
 *       dense          : all j < n_k
 *       causal         : j <= i                (n_q == n_k)
 *       varlen         : cu_b <= j < cu_{b+1}, where cu_b <= i < cu_{b+1}
 *       varlen causal  : the varlen set intersected with j <= i
 *   The softmax is the two-pass textbook form: pass 1 takes the row maximum
 *   m_i, pass 2 forms p_ij = exp(s_ij - m_i) / l_i with
 *   l_i = sum_j exp(s_ij - m_i), and the output is sum_j p_ij v_j.
 *   The row statistics (m_i, l_i) are returned because the method persists
 *   exactly this O(N) state for the backward (OCANNL "Module
 *   Ir.Online_softmax", fourth rewrite bullet; TIGA-lang GAT section, the
 *   training remark).  m is in natural-log units of the scaled score.
 *
 *   Backward -- OCANNL "Module Ir.Online_softmax", third rewrite bullet
 *   (the composed backward).  Written in its chain-rule (Jacobian) form, NOT
 *   with the per-row shortcut D = sum(dO * O), so that tests can check that
 *   shortcut against this definition:
 *       P_ij    = exp(s_ij - m_i) / l_i  on A(i), 0 elsewhere
 *       dV_j    = sum_i P_ij dO_i
 *       dP_ij   = <dO_i, v_j>
 *       delta_i = sum_j P_ij dP_ij
 *       dS_ij   = P_ij (dP_ij - delta_i)
 *       dQ_i    = scale * sum_j dS_ij k_j
 *       dK_j    = scale * sum_i dS_ij q_i
 *
 *   Tile-pruned forward (an approximation, defined on query blocks and key
 *   tiles) -- see oracle_attn_fwd_pruned below.
 *
 *   CSR segment softmax with given edge scores -- see oracle_csr_softmax.
 *
 * Layout: every array is (H, N, D) row-major and contiguous, in double.
 * Parallelism: OpenMP over independent (head, row) pairs only; every output
 * element is produced by one thread with a fixed serial summation order, so
 * results do not depend on the thread count.
 *
 * Return value of every entry point: 0 on success, -1 on an invalid
 * argument (null pointer, non-positive size, malformed cu_seqlens, causal
 * with n_q != n_k), -2 if a work buffer cannot be allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Admitted key interval [lo, hi) of query row i (A(i) above). */
static void admitted_keys(int64_t i, int64_t n_k, int causal,
                          const int32_t *cu_seqlens, int num_seqs,
                          int64_t *lo, int64_t *hi)
{
    int64_t a = 0, b = n_k;
    if (cu_seqlens) {
        for (int s = 0; s < num_seqs; ++s) {
            if (cu_seqlens[s] <= i && i < cu_seqlens[s + 1]) {
                a = cu_seqlens[s];
                b = cu_seqlens[s + 1];
                break;
            }
        }
    }
    if (causal && b > i + 1) b = i + 1;
    *lo = a;
    *hi = b;
}

static int check_args(int H, int64_t n_q, int64_t n_k, int D, int causal,
                      const int32_t *cu_seqlens, int num_seqs)
{
    if (H <= 0 || n_q <= 0 || n_k <= 0 || D <= 0) return -1;
    if (causal && n_q != n_k) return -1;
    if (cu_seqlens) {
        if (num_seqs <= 0 || n_q != n_k) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != n_q) return -1;
        for (int s = 0; s < num_seqs; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    }
    return 0;
}

static double dot(const double *a, const double *b, int D)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += a[d] * b[d];
    return acc;
}

/*
 * Forward for a list of (head, row) pairs.  rows[r] = h * n_q + i; when rows
 * is NULL all H * n_q pairs are computed in order.  Outputs are indexed by
 * position in the list: o[r * D + d], m[r], l[r].
 */
int oracle_attn_fwd_rows(int H, int64_t n_q, int64_t n_k, int D,
                         const double *q, const double *k, const double *v,
                         double scale, int causal,
                         const int32_t *cu_seqlens, int num_seqs,
                         const int64_t *rows, int64_t n_rows,
                         double *o, double *m, double *l)
{
    if (!q || !k || !v || !o || !m || !l) return -1;
    if (check_args(H, n_q, n_k, D, causal, cu_seqlens, num_seqs)) return -1;
    if (!rows) n_rows = (int64_t)H * n_q;
    int status = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)n_k);
        if (!s) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            int64_t flat = rows ? rows[r] : r;
            int64_t h = flat / n_q, i = flat % n_q;
            const double *qi = q + (h * n_q + i) * D;
            const double *kh = k + h * n_k * D;
            const double *vh = v + h * n_k * D;
            double *oi = o + r * D;
            int64_t lo, hi;
            admitted_keys(i, n_k, causal, cu_seqlens, num_seqs, &lo, &hi);

            /* scores, then pass 1: the row maximum */
            double mx = -INFINITY;
            for (int64_t j = lo; j < hi; ++j) {
                s[j] = dot(kh + j * D, qi, D) * scale;
                if (s[j] > mx) mx = s[j];
            }
            /* pass 2: normaliser, then normalised weights against v */
            double sum = 0.0;
            for (int64_t j = lo; j < hi; ++j) sum += exp(s[j] - mx);
            for (int d = 0; d < D; ++d) oi[d] = 0.0;
            for (int64_t j = lo; j < hi; ++j) {
                double p = exp(s[j] - mx) / sum;
                for (int d = 0; d < D; ++d) oi[d] += p * vh[j * D + d];
            }
            m[r] = mx;
            l[r] = sum;
        }
        free(s);
    }
    return status;
}

int oracle_attn_fwd(int H, int64_t n_q, int64_t n_k, int D,
                    const double *q, const double *k, const double *v,
                    double scale, int causal,
                    const int32_t *cu_seqlens, int num_seqs,
                    double *o, double *m, double *l)
{
    return oracle_attn_fwd_rows(H, n_q, n_k, D, q, k, v, scale, causal,
                                cu_seqlens, num_seqs, NULL, 0, o, m, l);
}

/*
 * Backward in the chain-rule form above.  For each head it materialises the
 * probability matrix P and the score gradient dS as (n_q, n_k) arrays
 * (that is what the composed form does; it is the oracle, not the method).
 * Optional outputs m_out, l_out, delta_out (H, n_q) may be NULL.
 */
int oracle_attn_bwd(int H, int64_t n_q, int64_t n_k, int D,
                    const double *q, const double *k, const double *v,
                    const double *dout, double scale, int causal,
                    const int32_t *cu_seqlens, int num_seqs,
                    double *dq, double *dk, double *dv,
                    double *m_out, double *l_out, double *delta_out)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (check_args(H, n_q, n_k, D, causal, cu_seqlens, num_seqs)) return -1;

    double *P = (double *)malloc(sizeof(double) * (size_t)(n_q * n_k));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(n_q * n_k));
    if (!P || !dS) {
        free(P);
        free(dS);
        return -2;
    }

    for (int h = 0; h < H; ++h) {
        const double *qh = q + (int64_t)h * n_q * D;
        const double *kh = k + (int64_t)h * n_k * D;
        const double *vh = v + (int64_t)h * n_k * D;
        const double *doh = dout + (int64_t)h * n_q * D;
        double *dqh = dq + (int64_t)h * n_q * D;
        double *dkh = dk + (int64_t)h * n_k * D;
        double *dvh = dv + (int64_t)h * n_k * D;

        /* Row-wise: P, dP, delta, dS, dQ. */
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_q; ++i) {
            double *Pi = P + i * n_k, *dSi = dS + i * n_k;
            const double *qi = qh + i * D, *doi = doh + i * D;
            int64_t lo, hi;
            admitted_keys(i, n_k, causal, cu_seqlens, num_seqs, &lo, &hi);
            for (int64_t j = 0; j < n_k; ++j) Pi[j] = dSi[j] = 0.0;

            double mx = -INFINITY;
            for (int64_t j = lo; j < hi; ++j) {
                Pi[j] = dot(kh + j * D, qi, D) * scale; /* s_ij for now */
                if (Pi[j] > mx) mx = Pi[j];
            }
            double sum = 0.0;
            for (int64_t j = lo; j < hi; ++j) sum += exp(Pi[j] - mx);
            for (int64_t j = lo; j < hi; ++j) Pi[j] = exp(Pi[j] - mx) / sum;

            double delta = 0.0;
            for (int64_t j = lo; j < hi; ++j) {
                dSi[j] = dot(doi, vh + j * D, D); /* dP_ij for now */
                delta += Pi[j] * dSi[j];
            }
            for (int64_t j = lo; j < hi; ++j) dSi[j] = Pi[j] * (dSi[j] - delta);

            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t j = lo; j < hi; ++j) acc += dSi[j] * kh[j * D + d];
                dqh[i * D + d] = scale * acc;
            }
            if (m_out) m_out[(int64_t)h * n_q + i] = mx;
            if (l_out) l_out[(int64_t)h * n_q + i] = sum;
            if (delta_out) delta_out[(int64_t)h * n_q + i] = delta;
        }

        /* Column-wise: dV and dK (P and dS are zero outside A(i)); each
         * element sums over i in increasing order. */
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t j = 0; j < n_k; ++j) {
            double *dvj = dvh + j * D, *dkj = dkh + j * D;
            for (int d = 0; d < D; ++d) dvj[d] = dkj[d] = 0.0;
            for (int64_t i = 0; i < n_q; ++i) {
                double p = P[i * n_k + j], ds = dS[i * n_k + j];
                for (int d = 0; d < D; ++d) {
                    dvj[d] += p * doh[i * D + d];
                    dkj[d] += ds * qh[i * D + d];
                }
            }
            for (int d = 0; d < D; ++d) dkj[d] *= scale;
        }
    }
    free(P);
    free(dS);
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
/*
 * Tile-pruned dense forward -- TIGA-lang "基于 tile 剪枝的稀疏注意力"
 * (tile-pruned sparse attention), section "具体规则与边界" (rules and
 * boundaries) and its admission inequality.  An approximation of the dense
 * attention above, defined on tiles: query block b = rows [b br, (b+1) br),
 * key tile t = keys [t bc, (t+1) bc) (both cut at the tensor ends).  For each
 * (head, query block) the key tiles are visited in increasing key order,
 * with a block-level running maximum m_run that starts at -inf:
 *     m_tile = max over rows i of the block and keys j of the tile of s_ij
 *     the tile is admitted  iff  m_tile >= m_run + ln(rho)      (0 < rho <= 1)
 *     if admitted: m_run = max(m_run, m_tile)
 * A pruned tile contributes nothing: each row's output is the exact two-pass
 * softmax attention over the keys of its block's admitted tiles, and m, l are
 * that softmax's row maximum and normaliser.  (rho -> 0 admits every tile:
 * the exact dense result.)
 * Extra outputs, each optional (NULL): admit[(h * nqb + b) * nkt + t] = 1 or 0
 * with nqb = ceil(n_q / br), nkt = ceil(n_k / bc); *min_margin = the smallest
 * |m_tile - (m_run + ln rho)| over the decisions taken against a finite
 * m_run (+inf if there are none), so a caller can tell whether rounding of
 * the scores could flip a decision.
 */
int oracle_attn_fwd_pruned(int H, int64_t n_q, int64_t n_k, int D,
                           const double *q, const double *k, const double *v,
                           double scale, double rho, int br, int bc,
                           double *o, double *m, double *l,
                           unsigned char *admit, double *min_margin)
{
    if (!q || !k || !v || !o || !m || !l) return -1;
    if (check_args(H, n_q, n_k, D, 0, NULL, 0)) return -1;
    if (!(rho > 0.0 && rho <= 1.0) || br <= 0 || bc <= 0) return -1;
    const int64_t nqb = (n_q + br - 1) / br, nkt = (n_k + bc - 1) / bc;
    const double log_rho = log(rho);
    int status = 0;
    double margin = INFINITY;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)br * (size_t)n_k);
        unsigned char *adm = (unsigned char *)malloc((size_t)nkt);
        double my_margin = INFINITY;
        if (!s || !adm) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t hb = 0; hb < (int64_t)H * nqb; ++hb) {
            if (!s || !adm) continue;
            const int64_t h = hb / nqb, b = hb % nqb;
            const int64_t i0 = b * br, i1 = (i0 + br < n_q) ? i0 + br : n_q;
            const double *kh = k + h * n_k * D;
            const double *vh = v + h * n_k * D;
            /* every score of the block */
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = 0; j < n_k; ++j)
                    s[(i - i0) * n_k + j] = dot(kh + j * D, q + (h * n_q + i) * D, D) * scale;
            /* the admission scan over the key tiles */
            double m_run = -INFINITY;
            for (int64_t t = 0; t < nkt; ++t) {
                const int64_t j0 = t * bc, j1 = (j0 + bc < n_k) ? j0 + bc : n_k;
                double m_tile = -INFINITY;
                for (int64_t i = i0; i < i1; ++i)
                    for (int64_t j = j0; j < j1; ++j)
                        if (s[(i - i0) * n_k + j] > m_tile) m_tile = s[(i - i0) * n_k + j];
                const double thr = m_run + log_rho;
                adm[t] = (unsigned char)(m_tile >= thr);
                if (isfinite(m_run) && fabs(m_tile - thr) < my_margin) my_margin = fabs(m_tile - thr);
                if (adm[t] && m_tile > m_run) m_run = m_tile;
                if (admit) admit[hb * nkt + t] = adm[t];
            }
            /* each row: two-pass softmax over the admitted tiles' keys */
            for (int64_t i = i0; i < i1; ++i) {
                const double *si = s + (i - i0) * n_k;
                double *oi = o + (h * n_q + i) * D;
                double mx = -INFINITY;
                for (int64_t j = 0; j < n_k; ++j)
                    if (adm[j / bc] && si[j] > mx) mx = si[j];
                double sum = 0.0;
                for (int64_t j = 0; j < n_k; ++j)
                    if (adm[j / bc]) sum += exp(si[j] - mx);
                for (int d = 0; d < D; ++d) oi[d] = 0.0;
                for (int64_t j = 0; j < n_k; ++j) {
                    if (!adm[j / bc]) continue;
                    const double p = exp(si[j] - mx) / sum;
                    for (int d = 0; d < D; ++d) oi[d] += p * vh[j * D + d];
                }
                m[h * n_q + i] = mx;
                l[h * n_q + i] = sum;
            }
        }
#pragma omp critical
        {
            if (my_margin < margin) margin = my_margin;
        }
        free(s);
        free(adm);
    }
    if (min_margin) *min_margin = margin;
    return status;
}

/*
 * CSR segment softmax with field scores -- TIGA-lang "用图组合表达 varlen 因果注意力"
 * (varlen causal attention by graph composition), its remark that compiled
 * streaming covers CSR segment softmax over field scores, and the relation
 * view of "Attention and dense relations": a relation is a set of edges
 * (j -> i), and each destination row i takes the softmax of its edges'
 * scores against the source values.  Here the scores are given per edge (a
 * field), not computed from q and k:
 *     edges of row i:  e = row_ptr[i] .. row_ptr[i+1]-1, source col_idx[e]
 *     m_hi = max_e s_he,   l_hi = sum_e exp(s_he - m_hi)
 *     out_hi = sum_e exp(s_he - m_hi) / l_hi * v_h,col_idx[e]
 * A row with no edges has out = 0, m = -inf, l = 0 (an empty relation row).
 * scores is (H, nnz) with nnz = row_ptr[n_dst]; v is (H, n_src, D); o is
 * (H, n_dst, D); m, l are (H, n_dst).  Returns -1 on malformed CSR
 * (row_ptr not starting at 0 or decreasing, a column outside [0, n_src)).
 */
int oracle_csr_softmax(int H, int64_t n_dst, int64_t n_src, int D,
                       const int32_t *row_ptr, const int32_t *col_idx,
                       const double *scores, const double *v,
                       double *o, double *m, double *l)
{
    if (!row_ptr || !scores || !v || !o || !m || !l) return -1;
    if (H <= 0 || n_dst <= 0 || n_src <= 0 || D <= 0 || row_ptr[0] != 0) return -1;
    for (int64_t i = 0; i < n_dst; ++i)
        if (row_ptr[i + 1] < row_ptr[i]) return -1;
    const int64_t nnz = row_ptr[n_dst];
    if (nnz > 0 && !col_idx) return -1;
    for (int64_t e = 0; e < nnz; ++e)
        if (col_idx[e] < 0 || col_idx[e] >= n_src) return -1;

#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < (int64_t)H * n_dst; ++r) {
        const int64_t h = r / n_dst, i = r % n_dst;
        const double *sh = scores + h * nnz;
        const double *vh = v + h * n_src * D;
        double *oi = o + r * D;
        double mx = -INFINITY;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
            if (sh[e] > mx) mx = sh[e];
        double sum = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) sum += exp(sh[e] - mx);
        for (int d = 0; d < D; ++d) oi[d] = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const double p = exp(sh[e] - mx) / sum;
            for (int d = 0; d < D; ++d) oi[d] += p * vh[(int64_t)col_idx[e] * D + d];
        }
        m[r] = mx;
        l[r] = sum;
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
