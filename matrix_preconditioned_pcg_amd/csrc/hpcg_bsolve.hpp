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
// Five launches per iteration: the SpMV leaves the p.q partials; the apply's
// leaf stage takes the PQ step (alpha) and R -= alpha Q and leaves the r.r
// partials; the halfsums; the prolongation leaves the r.z partials; the
// direction step takes the RRZ step (the test and beta), X += alpha P (it
// reads P anyway) and P = Z + beta P.  The steps sit in the kernels that use
// their results (hpcg_colstate.hpp), so no launch is spent on a few scalars.
// R, Z, P, Q are fp32 (the block apply's arithmetic), X and every scalar fp64.
// A finished column gets alpha = beta = 0 from then on, so its X and R stay
// as they were while the others continue.
//
// Dot products: every product is taken in fp64 and every partial is a sum in
// a fixed order: p.q, r.r and r.z per leaf (the SpMV's and the block apply's
// workgroups), and the setup's b.b and r.z per 32-row block (k_bs_init,
// k_bs_dot).  The partials of a system are added in a fixed order (interleaved
// groups, each in order, then the groups in order): every sum has one order,
// so a solve is bitwise reproducible.
#pragma once
#include "hpcg_colstate.hpp"

namespace hpcg {

constexpr int BS_ROWS = 32;     // rows per workgroup (n is a multiple of 128)
constexpr int BS_COLS = 64;     // columns per workgroup
constexpr int BS_NT = 256;      // threads per workgroup

enum : int { BS_INIT = 0, BS_RZ0 = 1 };

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

// Q = A P and the leaf's partials of P . Q, part[s][k][c].  A workgroup of
// 1024 takes a leaf (128 rows) and a 32-column tile: thread (rr, g) row rr and
// columns 4g..4g+3 (a row's 32 columns are one 128-byte line), the row's
// entries four at a time, their indices and then their P rows all in flight
// together.  A row's sum is taken in fp64 and rounded to fp32 once: R -= alpha
// Q moves R away from B - A X by alpha (A P - Q) every step, and a sum of the
// stencil's cancelling terms rounded at every step moved it by several times
// tol on long, stiff grids.  The partial of a column adds the rows' products
// (with the stored, rounded Q) over the eight rows of a wave (fixed butterfly)
// and then the sixteen waves in order.
constexpr int BS_SPMV_NT = 1024;
constexpr int BS_SPMV_COLS = 32;
__global__ __launch_bounds__(BS_SPMV_NT) void k_bs_spmv_dot(const int* __restrict__ row_ptr,
                                                            const int* __restrict__ col,
                                                            const float* __restrict__ val,
                                                            const float* __restrict__ P, float* __restrict__ Q,
                                                            double* __restrict__ part, int nrhs) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int NWV = BS_SPMV_NT / 64;
  constexpr int CG = BS_SPMV_COLS / 4;       // column groups of a row (8)
  __shared__ double red[NWV * BS_SPMV_COLS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = tid % CG, rr = tid / CG;
  const int c4 = blockIdx.y * BS_SPMV_COLS + 4 * g;
  const size_t leaf = blockIdx.x;            // over the B K leaves of the batch
  double d[4] = {0.0, 0.0, 0.0, 0.0};
  if (c4 < nrhs) {
    const int row = (int)(leaf * LEAF) + rr;
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
#pragma unroll
    for (int o = CG; o < 64; o <<= 1) d[t] += __shfl_xor(d[t], o);
  }
  if (lane < CG) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w * BS_SPMV_COLS + 4 * lane + t] = d[t];
  }
  __syncthreads();
  const int c = blockIdx.y * BS_SPMV_COLS + tid;
  if (tid < BS_SPMV_COLS && c < nrhs) {
    double sum = red[tid];
#pragma unroll
    for (int k = 1; k < NWV; ++k) sum += red[k * BS_SPMV_COLS + tid];
    part[leaf * nrhs + c] = sum;
  }
}

// X += alpha P, then P = Z + beta P (alpha and beta per column of the row's
// system).  alpha = 0 (the setup, and every step of a finished column) leaves X
// as it is; beta = 0 (the first step, and every step of a finished column)
// takes P = Z without using P, which holds no value before the first step.
// A workgroup of 512 takes a leaf (128 rows) and a 64-column tile: thread
// (rg, c) rows rg, rg + 8, ... of column c.  RRZ: the workgroup first takes the
// RRZ step of its columns (hpcg_colstate.hpp) from the r.z and r.r partials,
// thread (rg, c) adding every eighth partial in order and then the eight
// groups in order, its rows' P, Z (and X) loads already in flight and its X
// stores (which need alpha only) issued; the workgroups of leaf 0 store the
// state.  Without RRZ (the setup) beta is the stored one.
struct BsRrz {
  const double* rz;   // [B][rz_blocks][nrhs] partials of R . Z
  int rz_blocks;
  const double* rr;   // [B][rr_blocks][nrhs] partials of R . R
  int rr_blocks;
  double tol;
  int maxit;
};
constexpr int BS_DIR_NT = 512;
constexpr int BS_DIR_COLS = 64;
template <bool RRZ>
__global__ __launch_bounds__(BS_DIR_NT) void k_bs_direction(ColState* __restrict__ cs, const float* __restrict__ Z,
                                                            float* __restrict__ P, double* __restrict__ X, int nrhs,
                                                            int K, BsRrz st) {
  constexpr int NG = BS_DIR_NT / BS_DIR_COLS;   // row groups (8)
  constexpr int RPT = LEAF / NG;                // rows per thread (16)
  __shared__ double red[2 * NG * BS_DIR_COLS];
  __shared__ double beta_s[BS_DIR_COLS];
  const int tid = threadIdx.x, cl = tid % BS_DIR_COLS, rg = tid / BS_DIR_COLS;
  const int c = blockIdx.y * BS_DIR_COLS + cl;
  const size_t leaf = blockIdx.x;            // over the B K leaves of the batch
  const int s = (int)(leaf / K);
  const bool live = c < nrhs;
  const size_t idx = (size_t)s * nrhs + (live ? c : 0);
  const double alpha = live ? cs[idx].alpha : 0.0;
  float pv[RPT], zv[RPT];
  double xv[RPT];
  if (live) {
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const size_t i = (leaf * LEAF + rg + NG * u) * nrhs + c;
      pv[u] = P[i];
      zv[u] = Z[i];
      xv[u] = alpha != 0.0 ? X[i] : 0.0;
    }
    if (alpha != 0.0) {
#pragma unroll
      for (int u = 0; u < RPT; ++u) X[(leaf * LEAF + rg + NG * u) * nrhs + c] = fma(alpha, (double)pv[u], xv[u]);
    }
  }
  double beta;
  if constexpr (RRZ) {
    red[tid] = live ? bs_strided_sum(st.rz + (size_t)s * st.rz_blocks * nrhs + c, st.rz_blocks, nrhs, rg, NG) : 0.0;
    red[NG * BS_DIR_COLS + tid] =
        live ? bs_strided_sum(st.rr + (size_t)s * st.rr_blocks * nrhs + c, st.rr_blocks, nrhs, rg, NG) : 0.0;
    __syncthreads();
    if (rg == 0 && live) {
      double rz = red[cl], rr = red[NG * BS_DIR_COLS + cl];
#pragma unroll
      for (int k = 1; k < NG; ++k) {
        rz += red[k * BS_DIR_COLS + cl];
        rr += red[(NG + k) * BS_DIR_COLS + cl];
      }
      ColState cst = cs[idx];
      bs_step_rrz(cst, rz, rr, st.tol, st.maxit);
      beta_s[cl] = cst.beta;
      if (leaf % K == 0) {
        cs[idx].status = cst.status;
        cs[idx].rz = cst.rz;
        cs[idx].beta = cst.beta;
        cs[idx].relres = cst.relres;
      }
    }
    __syncthreads();
    beta = live ? beta_s[cl] : 0.0;
  } else {
    beta = live ? cs[idx].beta : 0.0;
  }
  if (!live) return;
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const size_t i = (leaf * LEAF + rg + NG * u) * nrhs + c;
    P[i] = beta == 0.0 ? zv[u] : (float)((double)zv[u] + beta * (double)pv[u]);
  }
}

// The setup's steps (INIT: ||B_j|| and the state; RZ0: the first r.z) from
// per-block partials.  A workgroup per (system, 16-column tile): thread (g, c)
// adds the partials g, g + 16, ... of its column in order (the 16 columns of a
// partial row are one 128-byte line), then thread (0, c) adds the 16 group
// sums in order.  Grid: systems * nrhs / 16 workgroups (nrhs a multiple of 16).
constexpr int BS_SC_C = 16;     // columns per workgroup
constexpr int BS_SC_G = 16;     // partial groups per column
template <int MODE>
__global__ __launch_bounds__(BS_SC_C * BS_SC_G) void k_bs_scalars(ColState* __restrict__ cs,
                                                                  const double* __restrict__ part, int systems,
                                                                  int nrhs, int blocks_per_system) {
  __shared__ double red[BS_SC_G * BS_SC_C];
  const int tid = threadIdx.x, cl = tid % BS_SC_C, g = tid / BS_SC_C;
  const int tiles = nrhs / BS_SC_C;
  const int s = (int)blockIdx.x / tiles, c = ((int)blockIdx.x - s * tiles) * BS_SC_C + cl;
  if (s >= systems) return;        // whole workgroups leave together
  red[tid] = bs_strided_sum(part + (size_t)s * blocks_per_system * nrhs + c, blocks_per_system, nrhs, g, BS_SC_G);
  __syncthreads();
  if (g != 0) return;
  double sum = red[cl];
#pragma unroll
  for (int k = 1; k < BS_SC_G; ++k) sum += red[k * BS_SC_C + cl];
  const size_t idx = (size_t)s * nrhs + c;
  ColState st = cs[idx];
  if constexpr (MODE == BS_INIT) {
    st.bnorm = sqrt(sum);
    st.rz = st.rz_prev = st.alpha = st.beta = 0.0;
    st.iters = 0;
    st.status = st.status_pq = sum == 0.0 ? ST_CONVERGED : ST_RUNNING;
    st.relres = sum == 0.0 ? 0.0 : 1.0;
  } else {   // BS_RZ0
    st.beta = 0.0;
    if (st.status == ST_RUNNING) {
      if (!(sum > 0.0) || !isfinite(sum)) st.status = ST_BREAKDOWN;
      else st.rz = sum;
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
