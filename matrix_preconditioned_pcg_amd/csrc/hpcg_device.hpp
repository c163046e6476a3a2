// Device-side building blocks of the H-matrix-preconditioned CG solve on gfx950.
//
// Work decomposition.  Every system's n rows are cut into leaves of LEAF = 128
// rows, and every leaf into `bpl` row blocks of RB = LEAF / bpl rows.  One
// workgroup of NT = 256 threads (four wave64 wavefronts) owns one row block in
// every phase, so the same rows, the same rows of U_k and the same rows of the
// level slabs W_l[k] stay with the same workgroup through the whole iteration.
//
// One PCG iteration is three phases with a device-wide dependency between them
// ("Hierarchical Transformer Preconditioning for Interactive Physics
// Simulation", section 5: apply, SpMV, SAXPYs and dot reductions form the whole
// inner loop):
//   A  beta = (r.z)/(r.z)_old;  p = z + beta p;  q = A p;  partial p.q
//   B  alpha = (r.z)/(p.q);  x += alpha p;  r -= alpha q;  partial r.r;
//      restriction of the new r: t_k partial = U_k^T r_k over the block's rows,
//      and per level the slab partial W_l[k]^T r_k          (eq. (2))
//   C  convergence test on sum r.r;  z = M r from the restriction sums:
//      z_k = U_k t_k + sum_l W_l[k] P_l[partner half] + g r_k  (eqs. (3)-(5),
//      coupling core = identity);  partial r.z
// Scalars are accumulated in fp64, vectors are fp32, x is fp64.  Every sum of
// partials is evaluated by every workgroup that needs it in one fixed order, so
// all workgroups agree bit for bit and a solve is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hpcg {

constexpr int LEAF = 128;
constexpr int RANK = 32;
constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr int MAX_LEVELS = 12;

enum : int { ST_RUNNING = 0, ST_CONVERGED = 1, ST_NOT_CONVERGED = 2, ST_BREAKDOWN = 3 };

// `status` changes only in phase C (and at init): a breakdown found in phase A
// or B is parked in `brk`/`brk_it` and turned into a status by the next phase C.
// Every status a workgroup reads after a phase-C barrier is therefore final for
// that iteration, and all workgroups take the same loop-exit decision.
struct SysState {
  double rz[2];     // (r.z) after phase C of iteration j lives in rz[j & 1]
  double bnorm;     // ||b||_2
  double relres;    // latest ||r|| / ||b||
  int status;
  int iters;
  int brk;          // breakdown seen in phase A or B of the current iteration
  int brk_it;       // iteration to report for it
};

struct Geom {
  int n;         // rows per system
  int K;         // leaves per system
  int levels;    // tile levels
  int B;         // systems
  int bpl;       // row blocks per leaf
  int RB;        // rows per block (LEAF / bpl)
  int nblk_sys;  // K * bpl
  int nblk;      // B * nblk_sys
};

struct Bufs {
  const int* row_ptr;
  const int* col;
  const float* val;
  const float* U;      // [B][K][LEAF][LEAF]
  const float* W;      // [B][levels][K][LEAF][RANK]
  const float* g;      // [B*n]
  const float* b;      // [B*n]
  float* r;
  float* z;
  float* q;
  float* p0;
  float* p1;
  double* x;
  float* tpart;        // [B][K][bpl][LEAF]
  float* ppart;        // [B][levels][K][bpl][RANK]
  double* pq_part;     // [nblk]
  double* rr_part;
  double* rz_part;
  SysState* st;        // [B]
  unsigned* barrier;   // device-wide barrier arrival counter
  int* abort_flag;     // set when a barrier wait exceeds its bound
  int* itbase;         // graph engine: absolute iteration of the replay's first step
  int* replays;        // graph engine: replays finished
  double tol;
  int maxit;
};

struct alignas(16) Smem {
  float r[LEAF];                       // the block's rows of r
  float t[LEAF];                       // t_k = U_k^T r_k (whole leaf)
  float P[MAX_LEVELS * RANK];          // partner-half sums per level
  union {
    float redA[8][LEAF];               // restriction: U partials per row group
    float redP[8][MAX_LEVELS * RANK];  // prolongation: partner-sum partials
  };
  float redB[NWAVE][MAX_LEVELS * RANK];  // restriction: slab partials per wave
  float redU[LEAF][33];                // prolongation: per-row, per-column-slot dots
  float yoff[LEAF];
  float y[LEAF];
  double dred[NWAVE];
  int flag;
};

struct Blk {
  int s;      // system
  int lb;     // block within system
  int k;      // leaf
  int sub;    // row block within leaf
  int grow0;  // first global row
};

__device__ __forceinline__ Blk decode(const Geom& G, int b) {
  Blk o;
  o.s = b / G.nblk_sys;
  o.lb = b - o.s * G.nblk_sys;
  o.k = o.lb / G.bpl;
  o.sub = o.lb - o.k * G.bpl;
  o.grow0 = o.s * G.n + o.k * LEAF + o.sub * G.RB;
  return o;
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

// Sum over the whole workgroup in a fixed tree order (deterministic).
__device__ __forceinline__ double wg_sum(double v, Smem& sm) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) sm.dred[tid >> 6] = v;
  __syncthreads();
  double s = sm.dred[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) s += sm.dred[w];
  __syncthreads();
  return s;
}

// Sum of one system's per-block partials, identical in every workgroup.
__device__ __forceinline__ double sys_sum(const double* part, int s, int nblk_sys, Smem& sm) {
  double v = 0.0;
  for (int j = threadIdx.x; j < nblk_sys; j += NT) v += part[(size_t)s * nblk_sys + j];
  return wg_sum(v, sm);
}

// Broadcast a system's status through LDS so the whole workgroup branches alike.
// Returns ST_RUNNING, a final status, or -1 when a breakdown is pending.
__device__ __forceinline__ int read_status(const SysState* st, Smem& sm) {
  if (threadIdx.x == 0) {
    int v = __hip_atomic_load(&st->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v == ST_RUNNING && __hip_atomic_load(&st->brk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) v = -1;
    sm.flag = v;
  }
  __syncthreads();
  const int v = sm.flag;
  __syncthreads();
  return v;
}

__device__ __forceinline__ void park_breakdown(SysState* st, int it) {
  st->brk_it = it;
  __hip_atomic_store(&st->brk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_state(SysState* st, int status, int iters) {
  st->iters = iters;
  __hip_atomic_store(&st->status, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where a block's rows of U_k and of its level slabs are read from: global
// memory (row stride LEAF for U; slab level stride K*LEAF*RANK) or a resident
// copy in LDS (level stride RB*RANK).
struct FactorView {
  const float* Ub;   // first row of the block in U_k, rows LEAF floats apart
  const float* Wb;   // first row of the block in W_0[k], rows RANK floats apart
  size_t wstride;    // floats between consecutive levels
};

__device__ __forceinline__ FactorView global_view(const Geom& G, const Bufs& B, const Blk& bk) {
  FactorView v;
  v.Ub = B.U + ((size_t)bk.s * G.K + bk.k) * LEAF * LEAF + (size_t)bk.sub * G.RB * LEAF;
  v.Wb = B.W + ((size_t)bk.s * G.levels * G.K + bk.k) * LEAF * RANK + (size_t)bk.sub * G.RB * RANK;
  v.wstride = (size_t)G.K * LEAF * RANK;
  return v;
}

// ---------------------------------------------------------------------------
// Restriction (eq. (2) per leaf and level): from sm.r (block rows) write the
// block's partial t = U_blk^T r_blk and, for every level, W_l,blk^T r_blk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void restrict_block(const Geom& G, const Bufs& B, const Blk& bk,
                                               const FactorView& fv, Smem& sm) {
  const int tid = threadIdx.x;
  const int RB = G.RB;
  {
    const int cs = tid & 31, rg = tid >> 5;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = rg; i < RB; i += 8) {
      const float4 u = ld4(fv.Ub + (size_t)i * LEAF + 4 * cs);
      const float ri = sm.r[i];
      acc.x += u.x * ri; acc.y += u.y * ri; acc.z += u.z * ri; acc.w += u.w * ri;
    }
    *reinterpret_cast<float4*>(&sm.redA[rg][4 * cs]) = acc;
  }
  {
    const int cs = tid & 7, rg = tid >> 3, lane = tid & 63, wave = tid >> 6;
    for (int l = 0; l < G.levels; ++l) {
      const float* Wl = fv.Wb + (size_t)l * fv.wstride;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = rg; i < RB; i += 32) {
        const float4 w = ld4(Wl + (size_t)i * RANK + 4 * cs);
        const float ri = sm.r[i];
        acc.x += w.x * ri; acc.y += w.y * ri; acc.z += w.z * ri; acc.w += w.w * ri;
      }
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o); acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o); acc.w += __shfl_xor(acc.w, o);
      }
      if (lane < 8) *reinterpret_cast<float4*>(&sm.redB[wave][l * RANK + 4 * cs]) = acc;
    }
  }
  __syncthreads();
  if (tid < LEAF) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) s += sm.redA[g][tid];
    B.tpart[(((size_t)bk.s * G.K + bk.k) * G.bpl + bk.sub) * LEAF + tid] = s;
  }
  for (int e = tid; e < G.levels * RANK; e += NT) {
    float s = sm.redB[0][e];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) s += sm.redB[w][e];
    const int l = e / RANK, c = e - l * RANK;
    B.ppart[((((size_t)bk.s * G.levels + l) * G.K + bk.k) * G.bpl + bk.sub) * RANK + c] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Prolongation and assembly of y = M r on the block's rows (eqs. (3)-(5) and
// the diagonal stage), reading the restriction partials of every block of the
// system.  Needs sm.r; leaves y in sm.y[0..RB).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void prolong_block(const Geom& G, const Bufs& B, const Blk& bk,
                                              const FactorView& fv, Smem& sm) {
  const int tid = threadIdx.x;
  const int RB = G.RB;
  // t_k: sum of the leaf's block partials
  if (tid < LEAF) {
    const float* tp = B.tpart + ((size_t)bk.s * G.K + bk.k) * G.bpl * LEAF + tid;
    float s = 0.f;
    for (int j = 0; j < G.bpl; ++j) s += tp[(size_t)j * LEAF];
    sm.t[tid] = s;
  }
  // strip aggregation: partner-half sums per level (eq. (3))
  {
    const int c = tid & 31, j0 = tid >> 5;
    for (int l = 0; l < G.levels; ++l) {
      const int kp0 = ((bk.k >> l) ^ 1) << l;
      const int cnt = (1 << l) * G.bpl;
      const float* base = B.ppart + (((size_t)bk.s * G.levels + l) * G.K + kp0) * G.bpl * RANK + c;
      float acc = 0.f;
      for (int v = j0; v < cnt; v += 8) acc += base[(size_t)v * RANK];
      sm.redP[j0][l * RANK + c] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < G.levels * RANK; e += NT) {
    float s = sm.redP[0][e];
#pragma unroll
    for (int j = 1; j < 8; ++j) s += sm.redP[j][e];
    sm.P[e] = s;
  }
  __syncthreads();
  // diagonal stage: per row, dot of U row and t, split over 32 column slots
  {
    const int cs = tid & 31, rg = tid >> 5;
    const float4 t4 = *reinterpret_cast<const float4*>(&sm.t[4 * cs]);
    for (int i = rg; i < RB; i += 8) sm.redU[i][cs] = dot4(ld4(fv.Ub + (size_t)i * LEAF + 4 * cs), t4);
  }
  // prolongation (eq. (5)): per row, sum over levels of slab row . P_l
  {
    const int cs = tid & 7, rg = tid >> 3;
    for (int i = rg; i < RB; i += 32) {
      float acc = 0.f;
      for (int l = 0; l < G.levels; ++l) {
        const float4 w = ld4(fv.Wb + (size_t)l * fv.wstride + (size_t)i * RANK + 4 * cs);
        const float4 p4 = *reinterpret_cast<const float4*>(&sm.P[l * RANK + 4 * cs]);
        acc += dot4(w, p4);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if (cs == 0) sm.yoff[i] = acc;
    }
  }
  __syncthreads();
  if (tid < RB) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) s += sm.redU[tid][c];
    const int grow = bk.grow0 + tid;
    sm.y[tid] = s + sm.yoff[tid] + B.g[grow] * sm.r[tid];
  }
  __syncthreads();
}

// p_new = z + beta p_old, evaluated identically wherever it is needed so that
// the stored p and the p the SpMV multiplies are the same numbers.
__device__ __forceinline__ float pdir(float z, float pold, double beta) {
  return (float)((double)z + beta * (double)pold);
}

// ---------------------------------------------------------------------------
// Phases.  b = global block index; it = iteration (1-based; 0 = initial apply).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void phase_init(const Geom& G, const Bufs& B, int b, const FactorView& fv, Smem& sm) {
  const Blk bk = decode(G, b);
  const int tid = threadIdx.x;
  double loc = 0.0;
  if (tid < G.RB) {
    const int grow = bk.grow0 + tid;
    const float bv = B.b[grow];
    B.r[grow] = bv;
    B.x[grow] = 0.0;
    sm.r[tid] = bv;
    loc = (double)bv * (double)bv;
  }
  __syncthreads();
  restrict_block(G, B, bk, fv, sm);
  const double rr = wg_sum(loc, sm);
  if (tid == 0) {
    B.rr_part[b] = rr;
    if (bk.lb == 0) {
      SysState* st = B.st + bk.s;
      st->relres = 1.0;
      st->brk = 0;
      st->brk_it = 0;
      set_state(st, ST_RUNNING, 0);
    }
  }
}

__device__ __forceinline__ void phase_A(const Geom& G, const Bufs& B, int b, int it, Smem& sm) {
  const Blk bk = decode(G, b);
  SysState* st = B.st + bk.s;
  if (read_status(st, sm) != ST_RUNNING) return;
  const int tid = threadIdx.x;
  const double rz = sys_sum(B.rz_part, bk.s, G.nblk_sys, sm);
  if (!(rz > 0.0) || !isfinite(rz)) {
    if (tid == 0 && bk.lb == 0) park_breakdown(st, it - 1);
    return;
  }
  double beta = 0.0;
  if (it > 1) beta = rz / st->rz[(it - 2) & 1];
  if (tid == 0 && bk.lb == 0) st->rz[(it - 1) & 1] = rz;
  const float* pold = (it & 1) ? B.p0 : B.p1;
  float* pnew = (it & 1) ? B.p1 : B.p0;
  const bool first = (it == 1);
  // SpMV on the fly of p_new: TPR threads per row
  const int TPR = NT / G.RB;
  const int i = tid / TPR, lr = tid - i * TPR;
  const int grow = bk.grow0 + i;
  const int e0 = B.row_ptr[grow], e1 = B.row_ptr[grow + 1];
  float acc = 0.f;
  for (int e = e0 + lr; e < e1; e += TPR) {
    const int c = B.col[e];
    const float v = first ? B.z[c] : pdir(B.z[c], pold[c], beta);
    acc = fmaf(B.val[e], v, acc);
  }
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
  double loc = 0.0;
  if (lr == 0) {
    const float pn = first ? B.z[grow] : pdir(B.z[grow], pold[grow], beta);
    pnew[grow] = pn;
    B.q[grow] = acc;
    loc = (double)pn * (double)acc;
  }
  const double pq = wg_sum(loc, sm);
  if (tid == 0) B.pq_part[b] = pq;
}

__device__ __forceinline__ void phase_B(const Geom& G, const Bufs& B, int b, int it, const FactorView& fv, Smem& sm) {
  const Blk bk = decode(G, b);
  SysState* st = B.st + bk.s;
  if (read_status(st, sm) != ST_RUNNING) return;
  const int tid = threadIdx.x;
  const double pq = sys_sum(B.pq_part, bk.s, G.nblk_sys, sm);
  if (!(pq > 0.0) || !isfinite(pq)) {
    if (tid == 0 && bk.lb == 0) park_breakdown(st, it);
    return;
  }
  const double alpha = st->rz[(it - 1) & 1] / pq;
  const float* pnew = (it & 1) ? B.p1 : B.p0;
  double loc = 0.0;
  if (tid < G.RB) {
    const int grow = bk.grow0 + tid;
    const float rn = (float)((double)B.r[grow] - alpha * (double)B.q[grow]);
    B.r[grow] = rn;
    B.x[grow] += alpha * (double)pnew[grow];
    sm.r[tid] = rn;
    loc = (double)rn * (double)rn;
  }
  __syncthreads();
  restrict_block(G, B, bk, fv, sm);
  const double rr = wg_sum(loc, sm);
  if (tid == 0) B.rr_part[b] = rr;
}

__device__ __forceinline__ void phase_C(const Geom& G, const Bufs& B, int b, int it, const FactorView& fv, Smem& sm) {
  const Blk bk = decode(G, b);
  SysState* st = B.st + bk.s;
  const int tid = threadIdx.x;
  const bool lead = (tid == 0 && bk.lb == 0);
  const int cur = read_status(st, sm);
  if (cur == -1) {
    if (lead) set_state(st, ST_BREAKDOWN, st->brk_it);
    return;
  }
  if (cur != ST_RUNNING) return;
  const double rr = sys_sum(B.rr_part, bk.s, G.nblk_sys, sm);
  if (it == 0) {
    if (lead) st->bnorm = sqrt(rr);
    if (rr == 0.0) {
      if (lead) { st->relres = 0.0; set_state(st, ST_CONVERGED, 0); }
      return;
    }
  } else {
    const double rel = sqrt(rr) / st->bnorm;
    if (lead) st->relres = rel;
    if (rel <= B.tol) {
      if (lead) set_state(st, ST_CONVERGED, it);
      return;
    }
    if (it >= B.maxit) {
      if (lead) set_state(st, ST_NOT_CONVERGED, B.maxit);
      return;
    }
  }
  if (tid < G.RB) sm.r[tid] = B.r[bk.grow0 + tid];
  __syncthreads();
  prolong_block(G, B, bk, fv, sm);
  double loc = 0.0;
  if (tid < G.RB) {
    const float zv = sm.y[tid];
    B.z[bk.grow0 + tid] = zv;
    loc = (double)sm.r[tid] * (double)zv;
  }
  const double rz = wg_sum(loc, sm);
  if (tid == 0) B.rz_part[b] = rz;
}

}  // namespace hpcg
