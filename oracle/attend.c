/*
 * attend.c - restricted softmax attention over explicit key ranges, in
 * double precision.  Part of the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call it (through
 * oracle/minf_oracle.py); the product path never does, and this file shares
 * no code with it.
 *
 * What it computes (PaperTrace 2.1.2 "MInference", section 1.1, Eq. 2
 * restricted to the candidate set N_h(i); an empty set gives o = 0 and
 * LSE = -inf): for each listed row r, with N(r) the union of the key ranges
 * [lo[t], hi[t]] for t in [rptr[r], rptr[r+1]) (disjoint, inclusive),
 *   s_j  = scale * q_r . k_j                      (j in N(r)),
 *   m    = max_j s_j,
 *   o_r  = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),
 *   lse_r = m + log(sum_j exp(s_j - m)).
 * Inputs are float32 values (bf16 inputs widen to float32 exactly); every
 * product and sum is formed in double.  Plain loops: two passes per row
 * (scores and their maximum, then weights and sums).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_attend_ranges(int64_t R, int64_t dh, const float* q, const float* k, const float* v,
                         const int64_t* rptr, const int64_t* lo, const int64_t* hi, double scale,
                         double* o, double* lse) {
  int64_t most = 0;
  for (int64_t r = 0; r < R; ++r) {
    int64_t c = 0;
    for (int64_t t = rptr[r]; t < rptr[r + 1]; ++t)
      if (hi[t] >= lo[t]) c += hi[t] - lo[t] + 1;
    if (c > most) most = c;
  }
  double* s = (double*)malloc((size_t)(most > 0 ? most : 1) * sizeof(double));
  double* qd = (double*)malloc((size_t)dh * sizeof(double));
  double* acc = (double*)malloc((size_t)dh * sizeof(double));
  if (!s || !qd || !acc) {
    free(s);
    free(qd);
    free(acc);
    return -1;
  }
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t d = 0; d < dh; ++d) qd[d] = (double)q[r * dh + d];
    /* pass 1: the scores of the kept keys and their maximum */
    int64_t c = 0;
    double m = -INFINITY;
    for (int64_t t = rptr[r]; t < rptr[r + 1]; ++t) {
      for (int64_t j = lo[t]; j <= hi[t]; ++j) {
        const float* kj = k + j * dh;
        double dot = 0.0;
        for (int64_t d = 0; d < dh; ++d) dot += qd[d] * (double)kj[d];
        s[c] = scale * dot;
        if (s[c] > m) m = s[c];
        ++c;
      }
    }
    if (c == 0) {
      for (int64_t d = 0; d < dh; ++d) o[r * dh + d] = 0.0;
      lse[r] = -INFINITY;
      continue;
    }
    /* pass 2: the weights exp(s_j - m), their sum and the weighted values */
    for (int64_t d = 0; d < dh; ++d) acc[d] = 0.0;
    double l = 0.0;
    c = 0;
    for (int64_t t = rptr[r]; t < rptr[r + 1]; ++t) {
      for (int64_t j = lo[t]; j <= hi[t]; ++j) {
        const double p = exp(s[c++] - m);
        const float* vj = v + j * dh;
        l += p;
        for (int64_t d = 0; d < dh; ++d) acc[d] += p * (double)vj[d];
      }
    }
    for (int64_t d = 0; d < dh; ++d) o[r * dh + d] = acc[d] / l;
    lse[r] = m + log(l);
  }
  free(s);
  free(qd);
  free(acc);
  return 0;
}
