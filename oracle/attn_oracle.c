/*
 * attn_oracle.c -- fp64 CPU oracle for exact (ring) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes is the plain definition that ring attention reaches
 * exactly (up to rounding order):
 *
 *   Lesson 8 "Context Parallelism (CP)" (hpc.payai.win), section 1: the
 *   attention of one token is softmax(q K^T / sqrt(d)) V over the keys it may
 *   see; section 3 (online softmax): folding key blocks one at a time gives the
 *   same O as the unblocked computation; section 4: under a causal mask the
 *   query at global position i sees the keys at positions j <= i.
 *   "Paralelismo de sequencia e atencao de anel" (aiunderstanding.org), deep
 *   dive: after one full loop every query has seen every key, so the result is
 *   full attention, not an approximation.
 *
 * There is no blocking and no online rescaling here: for each (query row,
 * head) the score vector over all visible keys is materialised in fp64, its
 * maximum taken, then the exponentials, their sum and the weighted V sum.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *  - softmax scale 1/sqrt(d_head), computed in fp64;
 *  - grouped-query attention: query head h reads key/value head
 *    floor(h / (Hq/Hkv)) (contiguous groups; the Helix article states that
 *    several query heads share one KV head but not which ones);
 *  - LSE (not on the pages) is the natural log of the softmax denominator of
 *    the scaled scores: m + ln(sum_j exp(s_j - m));
 *  - a row that sees no key at all gives O = 0 and LSE = -inf.
 *
 * Element types of the inputs: 0 = fp32, 1 = bf16 bit patterns (uint16, the
 * exact bits a GPU run uploads), 2 = fp64.  Every input element is widened
 * exactly to fp64 before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen(const void* p, int elem, int64_t i) {
    if (elem == 0) return (double)((const float*)p)[i];
    if (elem == 1) {
        uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)p)[i];
}

/*
 * Attention for a list of query rows, all query heads.
 *   Q   [B, Sq,  Hq,  d]   natural sequence order
 *   K,V [B, Skv, Hkv, d]   natural sequence order
 *   rows: n_rows pairs (row_b[n], row_i[n]) naming query (batch, position)
 *   O_out   [n_rows, Hq, d]  fp64
 *   lse_out [n_rows, Hq]     fp64
 * causal != 0 requires Sq == Skv and lets position i see keys j <= i.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attention_rows(const void* Q, const void* K, const void* V, int elem,
                          int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                          int64_t d, int causal, int64_t n_rows, const int64_t* row_b,
                          const int64_t* row_i, double* O_out, double* lse_out) {
    if (B <= 0 || Sq <= 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0)
        return -1;
    if (causal && Sq != Skv) return -1;
    if (elem < 0 || elem > 2) return -1;
    for (int64_t n = 0; n < n_rows; ++n)
        if (row_b[n] < 0 || row_b[n] >= B || row_i[n] < 0 || row_i[n] >= Sq) return -1;

    const int64_t group = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t work = n_rows * Hq;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        double* q = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < work; ++w) {
            const int64_t n = w / Hq, h = w % Hq;
            const int64_t b = row_b[n], i = row_i[n];
            const int64_t kvh = h / group;
            const int64_t visible = causal ? (i + 1) : Skv;
            double* o = O_out + (n * Hq + h) * d;

            for (int64_t e = 0; e < d; ++e)
                q[e] = widen(Q, elem, ((b * Sq + i) * Hq + h) * d + e);

            /* scores of every visible key */
            for (int64_t j = 0; j < visible; ++j) {
                const int64_t kbase = ((b * Skv + j) * Hkv + kvh) * d;
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e) dot += q[e] * widen(K, elem, kbase + e);
                s[j] = dot * scale;
            }
            if (visible == 0) {
                for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
                lse_out[n * Hq + h] = -INFINITY;
                continue;
            }
            /* softmax: maximum, exponentials, denominator */
            double m = s[0];
            for (int64_t j = 1; j < visible; ++j)
                if (s[j] > m) m = s[j];
            double l = 0.0;
            for (int64_t j = 0; j < visible; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            /* weighted sum of the value rows */
            for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
            for (int64_t j = 0; j < visible; ++j) {
                const int64_t vbase = ((b * Skv + j) * Hkv + kvh) * d;
                const double p = s[j];
                for (int64_t e = 0; e < d; ++e) o[e] += p * widen(V, elem, vbase + e);
            }
            for (int64_t e = 0; e < d; ++e) o[e] /= l;
            lse_out[n * Hq + h] = m + log(l);
        }
        free(q);
        free(s);
    }
    return 0;
}

/*
 * Merge of (O, lse) partials computed over disjoint key sets of the same
 * query rows.  The combination is the online-softmax fold of lesson 8,
 * section 3, applied to whole shards (the Helix article, phase 1, shards the
 * KV cache over the sequence and combines the per-shard results in one
 * exchange): with M = max_p lse_p and w_p = exp(lse_p - M),
 *   lse = M + ln(sum_p w_p),   O = sum_p w_p O_p / sum_p w_p.
 * A partial with lse = -inf (a shard that saw no key) has weight 0; if every
 * partial of a row has lse = -inf the row gives O = 0, lse = -inf.
 *   O_parts [n_parts, rows, d], lse_parts [n_parts, rows]  fp64
 *   O_out   [rows, d], lse_out [rows]                       fp64
 */
int oracle_merge(const double* O_parts, const double* lse_parts, int64_t n_parts,
                 int64_t rows, int64_t d, double* O_out, double* lse_out) {
    if (n_parts <= 0 || rows < 0 || d <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int64_t p = 0; p < n_parts; ++p)
            if (lse_parts[p * rows + r] > M) M = lse_parts[p * rows + r];
        double* o = O_out + r * d;
        for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
        if (M == -INFINITY) {
            lse_out[r] = -INFINITY;
            continue;
        }
        double W = 0.0;
        for (int64_t p = 0; p < n_parts; ++p) {
            const double lp = lse_parts[p * rows + r];
            if (lp == -INFINITY) continue;
            const double w = exp(lp - M);
            W += w;
            const double* op = O_parts + (p * rows + r) * d;
            for (int64_t e = 0; e < d; ++e) o[e] += w * op[e];
        }
        for (int64_t e = 0; e < d; ++e) o[e] /= W;
        lse_out[r] = M + log(W);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later parallel regions use (n >= 1). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
