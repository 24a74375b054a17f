/*
 * Plain fp64 CPU reference of scaled dot-product attention -- TEST
 * INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; it shares no code with the HIP
 * library (built by gcc from the oracle's own sources).
 *
 * The pages name attention only as a second workload of the same
 * matrix-core path: its score, probability and output tiles (S, P, O) and
 * their reuse ("B200 TMEM Lifecycle Planner", section A2 trigger 2 and
 * section E step 1).  They give no formula; the reading taken is the
 * standard one, for every batch b, head h and query row i:
 *     s_j    = scale * sum_d q(i,d) k(j,d)             over visible keys j
 *     m      = max_j s_j
 *     w_j    = exp(s_j - m),   l = sum_j w_j
 *     o(i,d) = sum_j w_j v(j,d) / l
 * with every element decoded exactly from bf16 to fp64, dot products summed
 * over d in order and the sums over j in order.  A key j is visible to query
 * i when j < seq_k and, with the causal mask, j <= i + seq_k - seq_q (the
 * last query row sees every key).  A row with no visible key has o = 0.
 *
 * Beside o it returns, for the acceptance bound:
 *     pv(i,d) = sum_j (w_j / l) |v(j,d)|               (the scale of the output error)
 *     smax(i) = scale * max_j sum_d |q(i,d) k(j,d)|    (the scale of the score error)
 *
 * Layout: Q is batch x heads x seq_q x dim bf16, row-major with dim
 * contiguous; K and V batch x heads x seq_k x dim; outputs are indexed by the
 * flattened query row r = (b * heads + h) * seq_q + i.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t bits);

int oracle_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t dim,
                     const uint16_t *Q, const uint16_t *K, const uint16_t *V, float scale,
                     int causal, int64_t row_begin, int64_t row_end, double *O, double *PV,
                     double *SMAX)
{
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || dim < 1)
        return 1;
    const int64_t rows = batch * heads * seq_q;
    if (row_begin < 0 || row_end > rows || row_begin > row_end)
        return 1;
    if (row_end > row_begin && (!Q || !O || !PV || !SMAX))
        return 1;
    if (seq_k > 0 && row_end > row_begin && (!K || !V))
        return 1;
    const double sc = (double)scale;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t bh = r / seq_q, i = r % seq_q;
        double *o = O + (r - row_begin) * dim;
        double *pv = PV + (r - row_begin) * dim;
        double *s = malloc(sizeof(double) * (size_t)(seq_k > 0 ? seq_k : 1));
        double *q = malloc(sizeof(double) * (size_t)dim);
        if (!s || !q) {
            bad = 1;
            free(s);
            free(q);
            continue;
        }
        for (int64_t d = 0; d < dim; ++d) {
            o[d] = 0.0;
            pv[d] = 0.0;
            q[d] = oracle_bf16_to_f64(Q[r * dim + d]);
        }
        // visible keys: j < nvis
        int64_t nvis = seq_k;
        if (causal) {
            nvis = i + seq_k - seq_q + 1;
            if (nvis > seq_k)
                nvis = seq_k;
            if (nvis < 0)
                nvis = 0;
        }
        double m = -INFINITY, smax = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
            const uint16_t *kj = K + (bh * seq_k + j) * dim;
            double dot = 0.0, mag = 0.0;
            for (int64_t d = 0; d < dim; ++d) {
                const double p = q[d] * oracle_bf16_to_f64(kj[d]);
                dot += p;
                mag += fabs(p);
            }
            s[j] = sc * dot;
            if (s[j] > m)
                m = s[j];
            if (fabs(sc) * mag > smax)
                smax = fabs(sc) * mag;
        }
        SMAX[r - row_begin] = smax;
        if (nvis > 0) {
            double l = 0.0;
            for (int64_t j = 0; j < nvis; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            for (int64_t j = 0; j < nvis; ++j) {
                const uint16_t *vj = V + (bh * seq_k + j) * dim;
                for (int64_t d = 0; d < dim; ++d) {
                    const double v = oracle_bf16_to_f64(vj[d]);
                    o[d] += s[j] * v;
                    pv[d] += s[j] * fabs(v);
                }
            }
            for (int64_t d = 0; d < dim; ++d) {
                o[d] /= l;
                pv[d] /= l;
            }
        }
        free(s);
        free(q);
    }
    return bad;
}
