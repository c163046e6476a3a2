// Per-column state of the block PCG and the two steps of an iteration that
// turn dot products into step sizes ("Hierarchical Transformer Preconditioning
// for Interactive Physics Simulation", project page, Background: the
// preconditioned CG loop; alpha = r.z / p.Ap, beta = r'.z' / r.z).
//
// Each step runs inside the kernel that needs its result, in every workgroup
// that needs it: every workgroup adds the same partials in the same order, so
// all of them take bitwise the same alpha (or beta), and the workgroups of
// leaf 0 store the new state.  No kernel reads a field that the same kernel
// stores: the PQ step reads status and rz and stores status_pq, rz_prev, alpha
// and iters; the RRZ step reads status_pq, rz_prev, iters and bnorm and stores
// status, rz, beta and relres.
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

struct ColState {
  double bnorm;      // ||B_j||
  double rz;         // R_j . Z_j of the last completed iteration (RRZ step; setup)
  double rz_prev;    // rz as the PQ step found it: the RRZ step's beta denominator
  double alpha;      // this iteration's step (PQ step)
  double beta;
  double relres;     // ||R_j|| / ||B_j|| after the last update
  int status;        // ST_* after the RRZ step (and the setup): what the host reads
  int status_pq;     // ST_* after the PQ step
  int iters;
  int pad;
};

// The PQ step of a column from p.Ap: one more iteration for a running column,
// alpha = rz / p.Ap, or a breakdown when p.Ap is not positive and finite.
__device__ __forceinline__ void bs_step_pq(ColState& st, double pq) {
  int s = st.status;
  st.alpha = 0.0;
  st.rz_prev = st.rz;
  if (s == ST_RUNNING) {
    st.iters += 1;
    if (!(pq > 0.0) || !isfinite(pq)) s = ST_BREAKDOWN;
    else st.alpha = st.rz / pq;
  }
  st.status_pq = s;
}

// The RRZ step from the new r.r (the convergence test) and r.z (beta); a
// column that stops gets beta = 0.
__device__ __forceinline__ void bs_step_rrz(ColState& st, double rz, double rr, double tol, int maxit) {
  int s = st.status_pq;
  if (s == ST_RUNNING) {
    st.relres = sqrt(rr) / st.bnorm;
    if (st.relres <= tol) s = ST_CONVERGED;
    else if (st.iters >= maxit) s = ST_NOT_CONVERGED;
  }
  st.beta = 0.0;
  if (s == ST_RUNNING) {
    if (!(rz > 0.0) || !isfinite(rz)) {
      s = ST_BREAKDOWN;
    } else {
      st.beta = rz / st.rz_prev;
      st.rz = rz;
    }
  }
  st.status = s;
}

// Thread g of ng adds p[k * stride] for k = g, g + ng, ... < count in order,
// eight loads in flight at a time.
__device__ __forceinline__ double bs_strided_sum(const double* __restrict__ p, int count, int stride, int g,
                                                 int ng) {
  double a = 0.0;
  int k = g;
  for (; k + 7 * ng < count; k += 8 * ng) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(k + u * ng) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  for (; k < count; k += ng) a += p[(size_t)k * stride];
  return a;
}

}  // namespace hpcg
