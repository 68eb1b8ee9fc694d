/*
 * Plain fp64 loops for the CPU oracle (test infrastructure only: nothing in
 * the library links or calls this file).
 *
 * The oracle's rotations (y = Pi u, q' = Pi q, x_hat = Pi^T c), sketches
 * (z = S r, q_s = S q'), scores (<q', c[idx]> and <q_s, sign>) and its
 * quantizer (idx = number of boundaries <= y, ties to the upper cell;
 * TurboQuant paper review, "Method") are written out here as the textbook
 * loops: one dot product per output, summed in index order, no blocking or
 * reordering.  Rows are independent, so the outer loop is split over threads.
 */
#include <stdint.h>

/* c[i][j] = sum_t a[i][t] * b[j][t]   (a: n x k, b: m x k, c: n x m, row-major) */
void tq_oracle_matmul_nt(const double* a, const double* b, double* c, int64_t n, int64_t m, int64_t k) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double* ai = a + i * k;
    for (int64_t j = 0; j < m; ++j) {
      const double* bj = b + j * k;
      double s = 0.0;
      for (int64_t t = 0; t < k; ++t) s += ai[t] * bj[t];
      c[i * m + j] = s;
    }
  }
}

/* idx[i] = #{ k < nt : t[k] <= y[i] }   (t ascending or not: every boundary is counted) */
void tq_oracle_count_le(const double* t, int64_t nt, const double* y, int64_t n, int64_t stride_y,
                        int64_t* idx, int64_t stride_idx) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double v = y[i * stride_y];
    int64_t c = 0;
    for (int64_t k = 0; k < nt; ++k) c += t[k] <= v ? 1 : 0;
    idx[i * stride_idx] = c;
  }
}
