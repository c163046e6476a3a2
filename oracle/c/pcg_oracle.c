/*
 * Plain C fp64 oracle of the H-matrix-preconditioned CG solve.
 *
 * TEST INFRASTRUCTURE ONLY: the same definitions as the numpy oracle in this
 * directory's package, written as straightforward loops so that the oracle
 * can be timed on host cores as a CPU baseline.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it; it shares no
 * code with the HIP library.  Everything is fp64; the fp32 inputs (matrix,
 * factors, gate, right-hand side) are promoted exactly.
 *
 * Definitions followed:
 *  - SpMV: y_i = sum over the stored entries of row i of A_ij x_j, in storage
 *    order ("Hierarchical Transformer Preconditioning for Interactive Physics
 *    Simulation", section 5, stage (iii)).
 *  - M r: the diagonal stage y_k = U_k (U_k^T r_k) per leaf (section 5, stage
 *    (i)), then per tile (l, j) with row leaves [2jS, 2jS+S) and column leaves
 *    [2jS+S, 2jS+2S), S = 2^l (Supplementary section 2, K - 1 tiles):
 *    a = U^T r_R, c = V^T r_C, y_R += U c, y_C += V a, where U stacks the row
 *    leaves' level-l slabs W_l[k] and V the column leaves' (section 5, stage
 *    (ii), eqs. (2)-(5) with the coupling core equal to the identity), then
 *    y += g r.
 *  - PCG: the textbook loop (Saad, preconditioned CG), x_0 = 0, stop when
 *    ||r|| <= tol ||b|| on the recursively updated r (Supplementary section 1,
 *    "Convergence criterion"); the count is the number of products A p done
 *    when the test first passes; a non-positive or non-finite p.Ap or r.z is a
 *    breakdown.
 *
 * Threads (OpenMP) split rows, leaves and the tiles of one level, which write
 * disjoint rows; every sum keeps one fixed order, so the result does not
 * depend on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void orc_set_threads(int t) {
#ifdef _OPENMP
  if (t > 0) omp_set_num_threads(t);
#else
  (void)t;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_spmv(int n, const int* row_ptr, const int* col, const float* val, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    double s = 0.0;
    for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e) s += (double)val[e] * x[col[e]];
    y[i] = s;
  }
}

/* y = M r for one system.  U [K][L][L] row-major (row = node in leaf),
 * W [levels][K][L][R], g [K L]. */
void orc_apply_M(int K, int L, int R, int levels, const float* U, const float* W, const float* g, const double* r,
                 double* y) {
  const int n = K * L;
  /* (i) diagonal stage: t = U_k^T r_k, y_k = U_k t */
#pragma omp parallel for schedule(static)
  for (int k = 0; k < K; ++k) {
    const float* Uk = U + (size_t)k * L * L;
    const double* rk = r + (size_t)k * L;
    double* t = (double*)malloc(sizeof(double) * L);
    for (int c = 0; c < L; ++c) {
      double s = 0.0;
      for (int i = 0; i < L; ++i) s += (double)Uk[(size_t)i * L + c] * rk[i];
      t[c] = s;
    }
    for (int i = 0; i < L; ++i) {
      double s = 0.0;
      for (int c = 0; c < L; ++c) s += (double)Uk[(size_t)i * L + c] * t[c];
      y[(size_t)k * L + i] = s;
    }
    free(t);
  }
  /* (ii) off-diagonal tiles, level by level; the tiles of a level cover
   * disjoint rows */
  for (int l = 0; l < levels; ++l) {
    const int S = 1 << l, ntiles = K / (2 * S);
#pragma omp parallel for schedule(static)
    for (int j = 0; j < ntiles; ++j) {
      const int kr = 2 * j * S, kc = 2 * j * S + S;   /* first row leaf, first column leaf */
      const float* Ut = W + ((size_t)l * K + kr) * L * R;   /* S L x R, row-major */
      const float* Vt = W + ((size_t)l * K + kc) * L * R;
      const double* rR = r + (size_t)kr * L;
      const double* rC = r + (size_t)kc * L;
      double* a = (double*)calloc((size_t)R, sizeof(double));
      double* c = (double*)calloc((size_t)R, sizeof(double));
      for (int q = 0; q < R; ++q) {
        double sa = 0.0, sc = 0.0;
        for (int i = 0; i < S * L; ++i) {
          sa += (double)Ut[(size_t)i * R + q] * rR[i];
          sc += (double)Vt[(size_t)i * R + q] * rC[i];
        }
        a[q] = sa;
        c[q] = sc;
      }
      for (int i = 0; i < S * L; ++i) {
        double su = 0.0, sv = 0.0;
        for (int q = 0; q < R; ++q) {
          su += (double)Ut[(size_t)i * R + q] * c[q];
          sv += (double)Vt[(size_t)i * R + q] * a[q];
        }
        y[(size_t)kr * L + i] += su;
        y[(size_t)kc * L + i] += sv;
      }
      free(a);
      free(c);
    }
  }
  /* gate */
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) y[i] += (double)g[i] * r[i];
}

static double dot(int n, const double* a, const double* b) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/* One system: returns 0 converged, 1 not converged, 2 breakdown; *iters and
 * *relres (recursive ||r|| / ||b||) as the library reports them. */
int orc_pcg(int n, const int* row_ptr, const int* col, const float* val, int L, int R, int levels,
            const float* U, const float* W, const float* g, const float* b32, double tol, int maxit, double* x,
            int* iters, double* relres) {
  const int K = n / L;
  double* b = (double*)malloc(sizeof(double) * n);
  double* r = (double*)malloc(sizeof(double) * n);
  double* z = (double*)malloc(sizeof(double) * n);
  double* p = (double*)malloc(sizeof(double) * n);
  double* q = (double*)malloc(sizeof(double) * n);
  int status = 1;
  for (int i = 0; i < n; ++i) {
    b[i] = (double)b32[i];
    r[i] = b[i];
    x[i] = 0.0;
  }
  const double bnorm = sqrt(dot(n, b, b));
  *iters = 0;
  *relres = 0.0;
  if (bnorm == 0.0) {
    status = 0;
    goto done;
  }
  *relres = 1.0;
  orc_apply_M(K, L, R, levels, U, W, g, r, z);
  memcpy(p, z, sizeof(double) * n);
  double rz = dot(n, r, z);
  if (!(rz > 0.0) || !isfinite(rz)) {
    status = 2;
    goto done;
  }
  for (int it = 1; it <= maxit; ++it) {
    orc_spmv(n, row_ptr, col, val, p, q);
    const double pq = dot(n, p, q);
    *iters = it;
    if (!(pq > 0.0) || !isfinite(pq)) {
      status = 2;
      goto done;
    }
    const double alpha = rz / pq;
    for (int i = 0; i < n; ++i) {
      x[i] += alpha * p[i];
      r[i] -= alpha * q[i];
    }
    const double rel = sqrt(dot(n, r, r)) / bnorm;
    *relres = rel;
    if (rel <= tol) {
      status = 0;
      goto done;
    }
    orc_apply_M(K, L, R, levels, U, W, g, r, z);
    const double rz_new = dot(n, r, z);
    if (!(rz_new > 0.0) || !isfinite(rz_new)) {
      status = 2;
      goto done;
    }
    const double beta = rz_new / rz;
    for (int i = 0; i < n; ++i) p[i] = z[i] + beta * p[i];
    rz = rz_new;
  }
  *iters = maxit;
done:
  free(b);
  free(r);
  free(z);
  free(p);
  free(q);
  return status;
}
