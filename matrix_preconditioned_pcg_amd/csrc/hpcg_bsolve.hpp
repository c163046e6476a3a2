// Block PCG: one independent preconditioned CG per (system, column) of a
// node-major block of right-hand sides, run in lockstep so that every apply of
// M is a block apply on the matrix cores (hpcg_block.hpp) and every A product
// a block SpMV.  The columns share nothing but the launches: each has its own
// step sizes, its own convergence test and its own iteration count, exactly as
// if it were solved alone ("Hierarchical Transformer Preconditioning for
// Interactive Physics Simulation", project page, Background, the
// preconditioned CG the solve runs; the multi-vector apply of section 5,
// stages (i)-(ii)).
//
// Per iteration, for every running column j:
//   Q = A P;  pq_j = P_j . Q_j;  alpha_j = rz_j / pq_j;
//   X_j += alpha_j P_j;  R_j -= alpha_j Q_j;  Z = M R;  rz'_j = R_j . Z_j;
//   stop when ||R_j|| / ||B_j|| <= tol, else beta_j = rz'_j / rz_j;
//   P_j = Z_j + beta_j P_j.
// The test is taken with beta, after Z = M R: a column that has just
// converged costs one unused column of the block apply, and its count and x
// are those of the textbook loop, with one launch fewer per iteration.
// Six launches per iteration (eight with the block apply's three): the SpMV
// leaves the p.q partials; the apply's leaf stage takes R -= alpha Q and
// leaves the r.r partials, its prolongation the r.z partials; X += alpha P
// waits for the direction step, which reads P anyway.
// R, Z, P, Q are fp32 (the block apply's arithmetic), X and every scalar fp64.
// A finished column gets alpha = beta = 0 from then on, so its X and R stay
// as they were while the others continue.
//
// Dot products: every product is taken in fp64 and every partial is a sum in
// a fixed order: p.q per 32-row block (the SpMV's workgroups, which own 32 rows
// and 64 columns), r.r and r.z per leaf (the block apply's workgroups), and
// the setup's b.b and r.z per 32-row block (k_bs_init, k_bs_dot).  The
// partials of a system are added by one wave per (system, column) in a fixed
// order (lane-strided, then a fixed butterfly): every sum has one order, so a
// solve is bitwise reproducible.
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

constexpr int BS_ROWS = 32;     // rows per workgroup (n is a multiple of 128)
constexpr int BS_COLS = 64;     // columns per workgroup
constexpr int BS_NT = 256;      // threads per workgroup

struct ColState {
  double bnorm;    // ||B_j||
  double rz;       // R_j . Z_j of the last completed iteration
  double alpha;
  double beta;
  double relres;   // ||R_j|| / ||B_j|| after the last update
  int status;      // ST_*
  int iters;
  int pad[2];
};

enum : int { BS_INIT = 0, BS_RZ0 = 1, BS_PQ = 2, BS_RRZ = 3 };

// Workgroup (leaf rb, column tile) -> thread's column c, row group rg.
__device__ __forceinline__ double bs_rowgroup_reduce(double acc, double* red) {
  const int tid = threadIdx.x, c = tid & (BS_COLS - 1), rg = tid / BS_COLS;
  red[rg * BS_COLS + c] = acc;
  __syncthreads();
  double s = 0.0;
  if (rg == 0) s = ((red[c] + red[BS_COLS + c]) + red[2 * BS_COLS + c]) + red[3 * BS_COLS + c];
  return s;
}

// part[rb][c] = sum over the rows of leaf rb of X[row][c] * Y[row][c].
__global__ __launch_bounds__(BS_NT) void k_bs_dot(const float* __restrict__ X, const float* __restrict__ Y,
                                                  double* __restrict__ part, int nrhs) {
  __shared__ double red[BS_NT];
  const int tid = threadIdx.x, rg = tid / BS_COLS;
  const int c = blockIdx.y * BS_COLS + (tid & (BS_COLS - 1));
  const size_t rb = blockIdx.x;
  double acc = 0.0;
  if (c < nrhs) {
#pragma unroll
    for (int r = rg; r < BS_ROWS; r += BS_NT / BS_COLS) {
      const size_t i = (rb * BS_ROWS + r) * nrhs + c;
      acc = fma((double)X[i], (double)Y[i], acc);
    }
  }
  const double s = bs_rowgroup_reduce(acc, red);
  if (rg == 0 && c < nrhs) part[rb * nrhs + c] = s;
}

// R = B, X = 0, part = per-leaf partials of B . B.
__global__ __launch_bounds__(BS_NT) void k_bs_init(const float* __restrict__ Bm, float* __restrict__ R,
                                                   double* __restrict__ X, double* __restrict__ part, int nrhs) {
  __shared__ double red[BS_NT];
  const int tid = threadIdx.x, rg = tid / BS_COLS;
  const int c = blockIdx.y * BS_COLS + (tid & (BS_COLS - 1));
  const size_t rb = blockIdx.x;
  double acc = 0.0;
  if (c < nrhs) {
#pragma unroll
    for (int r = rg; r < BS_ROWS; r += BS_NT / BS_COLS) {
      const size_t i = (rb * BS_ROWS + r) * nrhs + c;
      const float b = Bm[i];
      R[i] = b;
      X[i] = 0.0;
      acc = fma((double)b, (double)b, acc);
    }
  }
  const double s = bs_rowgroup_reduce(acc, red);
  if (rg == 0 && c < nrhs) part[rb * nrhs + c] = s;
}

// Q = A P and the block's partials of P . Q (the layout of k_bs_dot).  A
// workgroup of 512 takes a 32-row block and a 64-column tile: thread (rr, g)
// row rr and columns 4g..4g+3, the row's entries four at a time, their indices
// and then their P rows all in flight together (two rows per thread, in 256,
// were slower).  A row's sum is taken in fp64 and rounded to fp32 once:
// R -= alpha Q moves R away from B - A X by alpha (A P - Q) every step, and a
// sum of the stencil's cancelling terms rounded at every step moved it by
// several times tol on long, stiff grids.  The partial of a column adds the
// rows' products (with the stored, rounded Q) over the four row groups of a
// wave (fixed butterfly) and then the eight waves in order.
constexpr int BS_SPMV_NT = 512;
__global__ __launch_bounds__(BS_SPMV_NT) void k_bs_spmv_dot(const int* __restrict__ row_ptr,
                                                            const int* __restrict__ col,
                                                            const float* __restrict__ val,
                                                            const float* __restrict__ P, float* __restrict__ Q,
                                                            double* __restrict__ part, int nrhs) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int NWV = BS_SPMV_NT / 64;
  __shared__ double red[NWV * BS_COLS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = tid & 15, rr = tid >> 4;
  const int c4 = blockIdx.y * BS_COLS + 4 * g;
  const size_t rb = blockIdx.x;
  double d[4] = {0.0, 0.0, 0.0, 0.0};
  if (c4 < nrhs) {
    const int row = (int)(rb * BS_ROWS) + rr;
    const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
    const f4 pv = *reinterpret_cast<const f4*>(P + (size_t)row * nrhs + c4);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int e = e0; e < e1; e += 4) {
      int c[4];
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = e + u < e1;
        c[u] = in ? col[e + u] : row;
        a[u] = in ? val[e + u] : 0.f;
      }
      f4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f4*>(P + (size_t)c[u] * nrhs + c4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (e + u < e1) {
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] = fma((double)a[u], (double)x[u][t], acc[t]);
        }
      }
    }
    const f4 qv = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
    *reinterpret_cast<f4*>(Q + (size_t)row * nrhs + c4) = qv;
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = (double)pv[t] * (double)qv[t];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    d[t] += __shfl_xor(d[t], 16);
    d[t] += __shfl_xor(d[t], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w * BS_COLS + 4 * lane + t] = d[t];
  }
  __syncthreads();
  const int c = blockIdx.y * BS_COLS + tid;
  if (tid < BS_COLS && c < nrhs) {
    double sum = red[tid];
#pragma unroll
    for (int k = 1; k < NWV; ++k) sum += red[k * BS_COLS + tid];
    part[rb * nrhs + c] = sum;
  }
}

// X += alpha P, then P = Z + beta P (alpha and beta per column of the row's
// system).  alpha = 0 (the setup, and every step of a finished column) leaves X
// as it is; beta = 0 (the first step, and every step of a finished column)
// takes P = Z without reading P, which holds no value before the first step.
__global__ __launch_bounds__(BS_NT) void k_bs_direction(const ColState* __restrict__ cs, const float* __restrict__ Z,
                                                        float* __restrict__ P, double* __restrict__ X, int nrhs,
                                                        int blocks_per_system) {
  const int tid = threadIdx.x, rg = tid / BS_COLS;
  const int c = blockIdx.y * BS_COLS + (tid & (BS_COLS - 1));
  const size_t rb = blockIdx.x;
  const int s = (int)(rb / blocks_per_system);
  if (c >= nrhs) return;
  const double alpha = cs[(size_t)s * nrhs + c].alpha;
  const double beta = cs[(size_t)s * nrhs + c].beta;
#pragma unroll
  for (int r = rg; r < BS_ROWS; r += BS_NT / BS_COLS) {
    const size_t i = (rb * BS_ROWS + r) * nrhs + c;
    if (alpha != 0.0) {
      const float p = P[i];
      X[i] = fma(alpha, (double)p, X[i]);
      P[i] = beta == 0.0 ? Z[i] : (float)((double)Z[i] + beta * (double)p);
    } else {
      P[i] = beta == 0.0 ? Z[i] : (float)((double)Z[i] + beta * (double)P[i]);
    }
  }
}

// One wave per (system, column): lane l adds the system's per-block partials
// l, l + 64, ... and the lanes are combined by the fixed butterfly of
// wave_sum (one order, every call); lane 0 takes the step the mode names.
constexpr int BS_SC_COLS = 4;   // columns (waves) per workgroup
// RRZ takes the convergence test on part2 (r.r) and then beta on part (r.z).
// part holds blocks_per_system partials per (system, column), part2 (RRZ only)
// blocks2 of them.
template <int MODE>
__global__ __launch_bounds__(64 * BS_SC_COLS) void k_bs_scalars(ColState* __restrict__ cs,
                                                                const double* __restrict__ part, int systems,
                                                                int nrhs, int blocks_per_system, double tol,
                                                                int maxit, const double* __restrict__ part2,
                                                                int blocks2) {
  const int idx = blockIdx.x * BS_SC_COLS + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (idx >= systems * nrhs) return;     // whole waves leave together
  const int s = idx / nrhs, c = idx - s * nrhs;
  double v = 0.0, v2 = 0.0;
  for (int k = lane; k < blocks_per_system; k += 64) v += part[((size_t)s * blocks_per_system + k) * nrhs + c];
  if constexpr (MODE == BS_RRZ) {
    for (int k = lane; k < blocks2; k += 64) v2 += part2[((size_t)s * blocks2 + k) * nrhs + c];
  }
  const double sum = wave_sum(v);
  double sum2 = 0.0;
  if constexpr (MODE == BS_RRZ) sum2 = wave_sum(v2);
  if (lane != 0) return;
  ColState st = cs[idx];
  if constexpr (MODE == BS_INIT) {
    st.bnorm = sqrt(sum);
    st.rz = st.alpha = st.beta = 0.0;
    st.iters = 0;
    st.status = sum == 0.0 ? ST_CONVERGED : ST_RUNNING;
    st.relres = sum == 0.0 ? 0.0 : 1.0;
  } else if constexpr (MODE == BS_RZ0) {
    st.beta = 0.0;
    if (st.status == ST_RUNNING) {
      if (!(sum > 0.0) || !isfinite(sum)) st.status = ST_BREAKDOWN;
      else st.rz = sum;
    }
  } else if constexpr (MODE == BS_PQ) {
    st.alpha = 0.0;
    if (st.status == ST_RUNNING) {
      st.iters += 1;
      if (!(sum > 0.0) || !isfinite(sum)) st.status = ST_BREAKDOWN;
      else st.alpha = st.rz / sum;
    }
  } else {   // BS_RRZ
    if (st.status == ST_RUNNING) {
      st.relres = sqrt(sum2) / st.bnorm;
      if (st.relres <= tol) st.status = ST_CONVERGED;
      else if (st.iters >= maxit) st.status = ST_NOT_CONVERGED;
    }
    st.beta = 0.0;
    if (st.status == ST_RUNNING) {
      if (!(sum > 0.0) || !isfinite(sum)) {
        st.status = ST_BREAKDOWN;
      } else {
        st.beta = sum / st.rz;
        st.rz = sum;
      }
    }
  }
  cs[idx] = st;
}

// Progress word for the host: bit 0 = no column is running, bits 1.. = replays
// completed (counted in *ctr on the device).
__global__ __launch_bounds__(256) void k_bs_progress(const ColState* __restrict__ cs, int total, int* ctr,
                                                     int* host_flag) {
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  int mine = 0;
  for (int i = threadIdx.x; i < total; i += blockDim.x) mine |= (cs[i].status == ST_RUNNING);
  if (mine) any = 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int r = *ctr + 1;
    *ctr = r;
    __hip_atomic_store(host_flag, (r << 1) | (any ? 0 : 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ void k_bs_reset(int* ctr, int* host_flag) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    *ctr = 0;
    __hip_atomic_store(host_flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace hpcg
