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
//
// Precision.  Factors and matrix values are always fp32 (they are the bytes
// that bound the apply).  The vector type T of the solve is a template
// parameter: T = float is the pages' split (fp32 vectors and apply arithmetic,
// fp64 scalars; Supplementary section 7), T = double carries r, z, p, q, the
// restriction partials and all accumulations in fp64.  Scalars and x are fp64
// in both.  Every sum of partials is evaluated by every workgroup that needs it
// in one fixed order, so all workgroups agree bit for bit and a solve is
// deterministic.
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

// Device buffers.  Vector buffers are sized for double; with T = float only the
// first half of each is used.
struct Bufs {
  const int* row_ptr;
  const int* col;
  const float* val;
  const float* U;      // [B][K][LEAF][LEAF]
  const float* W;      // [B][levels][K][LEAF][RANK]
  const float* g;      // [B*n]
  const float* b;      // [B*n]
  void* r;
  void* z;
  void* q;
  void* p0;
  void* p1;
  double* x;
  void* tpart;         // [B][K][bpl][LEAF]
  void* ppart;         // [B][levels][K][bpl][RANK]
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

template <typename T>
struct alignas(16) Smem {
  T r[LEAF];                         // the block's rows of r
  T t[LEAF];                         // t_k = U_k^T r_k (whole leaf)
  T P[MAX_LEVELS * RANK];            // partner-half sums per level
  union {
    struct {
      T redA[NWAVE][LEAF];           // restriction: U partials per wave
      T redB[NWAVE][MAX_LEVELS * RANK];  // restriction: slab partials per wave
    };
    T redP[NWAVE][MAX_LEVELS * RANK];    // prolongation: partner-sum partials per wave
  };
  T yleaf[LEAF];
  T yoff[LEAF];
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

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

template <typename T>
struct Vec4 { T x, y, z, w; };

template <typename T>
__device__ __forceinline__ Vec4<T> lds4(const T* p) {
  Vec4<T> v;
  v.x = p[0]; v.y = p[1]; v.z = p[2]; v.w = p[3];
  return v;
}

template <typename T>
__device__ __forceinline__ T dot4(float4 a, const Vec4<T>& b) {
  T s = (T)a.x * b.x;
  s = fma((T)a.y, b.y, s);
  s = fma((T)a.z, b.z, s);
  return fma((T)a.w, b.w, s);
}

template <typename T>
__device__ __forceinline__ void axpy4(Vec4<T>& acc, float4 u, T s) {
  acc.x = fma((T)u.x, s, acc.x);
  acc.y = fma((T)u.y, s, acc.y);
  acc.z = fma((T)u.z, s, acc.z);
  acc.w = fma((T)u.w, s, acc.w);
}

// Sum over the whole workgroup in a fixed tree order (deterministic).
template <typename T>
__device__ __forceinline__ double wg_sum(double v, Smem<T>& sm) {
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
template <typename T>
__device__ __forceinline__ double sys_sum(const double* part, int s, int nblk_sys, Smem<T>& sm) {
  double v = 0.0;
  for (int j = threadIdx.x; j < nblk_sys; j += NT) v += part[(size_t)s * nblk_sys + j];
  return wg_sum(v, sm);
}

// Broadcast a system's status through LDS so the whole workgroup branches alike.
// Returns ST_RUNNING, a final status, or -1 when a breakdown is pending.
template <typename T>
__device__ __forceinline__ int read_status(const SysState* st, Smem<T>& sm) {
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
// U: lane = 4-column slot (32 per row), 8 row groups; W: 8 slots per row, 32
// row groups.  Row groups are summed across lanes, then across waves in LDS.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void restrict_block(const Geom& G, const Bufs& B, const Blk& bk,
                                               const FactorView& fv, Smem<T>& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int RB = G.RB;
  T* tpart = reinterpret_cast<T*>(B.tpart);
  T* ppart = reinterpret_cast<T*>(B.ppart);
  {
    const int cs = tid & 31, rg = tid >> 5;
    Vec4<T> acc{0, 0, 0, 0};
    for (int i = rg; i < RB; i += 8) axpy4(acc, ld4(fv.Ub + (size_t)i * LEAF + 4 * cs), sm.r[i]);
    acc.x += __shfl_xor(acc.x, 32); acc.y += __shfl_xor(acc.y, 32);
    acc.z += __shfl_xor(acc.z, 32); acc.w += __shfl_xor(acc.w, 32);
    if (lane < 32) {
      T* d = &sm.redA[wave][4 * cs];
      d[0] = acc.x; d[1] = acc.y; d[2] = acc.z; d[3] = acc.w;
    }
  }
  {
    const int cs = tid & 7, rg = tid >> 3;
    for (int l = 0; l < G.levels; ++l) {
      const float* Wl = fv.Wb + (size_t)l * fv.wstride;
      Vec4<T> acc{0, 0, 0, 0};
      for (int i = rg; i < RB; i += 32) axpy4(acc, ld4(Wl + (size_t)i * RANK + 4 * cs), sm.r[i]);
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o); acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o); acc.w += __shfl_xor(acc.w, o);
      }
      if (lane < 8) {
        T* d = &sm.redB[wave][l * RANK + 4 * cs];
        d[0] = acc.x; d[1] = acc.y; d[2] = acc.z; d[3] = acc.w;
      }
    }
  }
  __syncthreads();
  if (tid < LEAF) {
    T s = sm.redA[0][tid];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) s += sm.redA[w][tid];
    tpart[(((size_t)bk.s * G.K + bk.k) * G.bpl + bk.sub) * LEAF + tid] = s;
  }
  for (int e = tid; e < G.levels * RANK; e += NT) {
    T s = sm.redB[0][e];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) s += sm.redB[w][e];
    const int l = e / RANK, c = e - l * RANK;
    ppart[((((size_t)bk.s * G.levels + l) * G.K + bk.k) * G.bpl + bk.sub) * RANK + c] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Prolongation and assembly of y = M r on the block's rows (eqs. (3)-(5) and
// the diagonal stage), reading the restriction partials of every block of the
// system.  Needs sm.r; returns y for row tid (tid < RB).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T prolong_block(const Geom& G, const Bufs& B, const Blk& bk,
                                           const FactorView& fv, Smem<T>& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int RB = G.RB;
  const T* tpart = reinterpret_cast<const T*>(B.tpart);
  const T* ppart = reinterpret_cast<const T*>(B.ppart);
  // t_k: sum of the leaf's block partials
  if (tid < LEAF) {
    const T* tp = tpart + ((size_t)bk.s * G.K + bk.k) * G.bpl * LEAF + tid;
    T s = tp[0];
    for (int j = 1; j < G.bpl; ++j) s += tp[(size_t)j * LEAF];
    sm.t[tid] = s;
  }
  // strip aggregation: partner-half sums per level (eq. (3))
  {
    const int c = tid & 31, j0 = tid >> 5;
    for (int l = 0; l < G.levels; ++l) {
      const int kp0 = ((bk.k >> l) ^ 1) << l;
      const int cnt = (1 << l) * G.bpl;
      const T* base = ppart + (((size_t)bk.s * G.levels + l) * G.K + kp0) * G.bpl * RANK + c;
      T acc = 0;
      for (int v = j0; v < cnt; v += 8) acc += base[(size_t)v * RANK];
      acc += __shfl_xor(acc, 32);
      if (lane < 32) sm.redP[wave][l * RANK + c] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < G.levels * RANK; e += NT) {
    T s = sm.redP[0][e];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) s += sm.redP[w][e];
    sm.P[e] = s;
  }
  __syncthreads();
  // diagonal stage: row i's dot with t is split over 32 lanes (4 columns each);
  // two rows at a time are folded with a transpose-reduce (5 shuffles per pair)
  {
    const int cs = tid & 31, rg = tid >> 5;
    const Vec4<T> t4 = lds4(&sm.t[4 * cs]);
    const bool hi = (cs & 16) != 0;
    for (int i0 = rg; i0 < RB; i0 += 16) {
      const int i1 = i0 + 8;
      const T v0 = dot4(ld4(fv.Ub + (size_t)i0 * LEAF + 4 * cs), t4);
      const T v1 = (i1 < RB) ? dot4(ld4(fv.Ub + (size_t)i1 * LEAF + 4 * cs), t4) : T(0);
      T keep = hi ? v1 : v0;
      const T send = hi ? v0 : v1;
      keep += __shfl_xor(send, 16);
      keep += __shfl_xor(keep, 8);
      keep += __shfl_xor(keep, 4);
      keep += __shfl_xor(keep, 2);
      keep += __shfl_xor(keep, 1);
      if (cs == 0) sm.yleaf[i0] = keep;
      if (cs == 16 && i1 < RB) sm.yleaf[i1] = keep;
    }
  }
  // prolongation (eq. (5)): per row, sum over levels of slab row . P_l
  {
    const int cs = tid & 7, rg = tid >> 3;
    for (int i = rg; i < RB; i += 32) {
      T acc = 0;
      for (int l = 0; l < G.levels; ++l)
        acc += dot4(ld4(fv.Wb + (size_t)l * fv.wstride + (size_t)i * RANK + 4 * cs), lds4(&sm.P[l * RANK + 4 * cs]));
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if (cs == 0) sm.yoff[i] = acc;
    }
  }
  __syncthreads();
  T y = 0;
  if (tid < RB) y = sm.yleaf[tid] + sm.yoff[tid] + (T)B.g[bk.grow0 + tid] * sm.r[tid];
  return y;
}

// p_new = z + beta p_old, evaluated identically wherever it is needed so that
// the stored p and the p the SpMV multiplies are the same numbers.
template <typename T>
__device__ __forceinline__ T pdir(T z, T pold, double beta) {
  return (T)((double)z + beta * (double)pold);
}

// ---------------------------------------------------------------------------
// Phases.  b = global block index; it = iteration (1-based; 0 = initial apply).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void phase_init(const Geom& G, const Bufs& B, int b, const FactorView& fv, Smem<T>& sm) {
  const Blk bk = decode(G, b);
  const int tid = threadIdx.x;
  T* r = reinterpret_cast<T*>(B.r);
  double loc = 0.0;
  if (tid < G.RB) {
    const int grow = bk.grow0 + tid;
    const T bv = (T)B.b[grow];
    r[grow] = bv;
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

template <typename T>
__device__ __forceinline__ void phase_A(const Geom& G, const Bufs& B, int b, int it, Smem<T>& sm) {
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
  const T* z = reinterpret_cast<const T*>(B.z);
  const T* pold = reinterpret_cast<const T*>((it & 1) ? B.p0 : B.p1);
  T* pnew = reinterpret_cast<T*>((it & 1) ? B.p1 : B.p0);
  T* q = reinterpret_cast<T*>(B.q);
  const bool first = (it == 1);
  // SpMV on the fly of p_new: TPR threads per row
  const int TPR = NT / G.RB;
  const int i = tid / TPR, lr = tid - i * TPR;
  const int grow = bk.grow0 + i;
  const int e0 = B.row_ptr[grow], e1 = B.row_ptr[grow + 1];
  T acc = 0;
  for (int e = e0 + lr; e < e1; e += TPR) {
    const int c = B.col[e];
    const T v = first ? z[c] : pdir<T>(z[c], pold[c], beta);
    acc = fma((T)B.val[e], v, acc);
  }
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
  double loc = 0.0;
  if (lr == 0) {
    const T pn = first ? z[grow] : pdir<T>(z[grow], pold[grow], beta);
    pnew[grow] = pn;
    q[grow] = acc;
    loc = (double)pn * (double)acc;
  }
  const double pq = wg_sum(loc, sm);
  if (tid == 0) B.pq_part[b] = pq;
}

template <typename T>
__device__ __forceinline__ void phase_B(const Geom& G, const Bufs& B, int b, int it, const FactorView& fv, Smem<T>& sm) {
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
  const T* pnew = reinterpret_cast<const T*>((it & 1) ? B.p1 : B.p0);
  const T* q = reinterpret_cast<const T*>(B.q);
  T* r = reinterpret_cast<T*>(B.r);
  double loc = 0.0;
  if (tid < G.RB) {
    const int grow = bk.grow0 + tid;
    const T rn = (T)((double)r[grow] - alpha * (double)q[grow]);
    r[grow] = rn;
    B.x[grow] += alpha * (double)pnew[grow];
    sm.r[tid] = rn;
    loc = (double)rn * (double)rn;
  }
  __syncthreads();
  restrict_block(G, B, bk, fv, sm);
  const double rr = wg_sum(loc, sm);
  if (tid == 0) B.rr_part[b] = rr;
}

template <typename T>
__device__ __forceinline__ void phase_C(const Geom& G, const Bufs& B, int b, int it, const FactorView& fv, Smem<T>& sm) {
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
  const T* r = reinterpret_cast<const T*>(B.r);
  T* z = reinterpret_cast<T*>(B.z);
  if (tid < G.RB) sm.r[tid] = r[bk.grow0 + tid];
  __syncthreads();
  const T zv = prolong_block(G, B, bk, fv, sm);
  double loc = 0.0;
  if (tid < G.RB) {
    z[bk.grow0 + tid] = zv;
    loc = (double)sm.r[tid] * (double)zv;
  }
  const double rz = wg_sum(loc, sm);
  if (tid == 0) B.rz_part[b] = rz;
}

}  // namespace hpcg
