// Kernels of the H-matrix-preconditioned CG solve for gfx950 (wave64, 256 CUs).
//
// Two solve engines share the phase functions of hpcg_device.hpp:
//  * graph engine: one kernel per phase, G unrolled iterations captured in a
//    hipGraph and replayed; the host reads a pinned flag between replays.
//  * persistent engine: a single launch runs the whole solve; phases are
//    separated by a device-wide barrier.  The grid never exceeds what the
//    occupancy query says can be resident at once, and every wait is bounded.
// Standalone kernels serve the two-launch hpcg_apply_M (restriction, then
// prolongation).
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

// ---------------------------------------------------------------------------
// device-wide barrier (persistent engine)
// ---------------------------------------------------------------------------
// Every workgroup arrives once per barrier on a monotonically increasing
// counter; barrier number m completes when the counter reaches m * gridDim.x.
// Arrival is an agent-scope release, the wait an agent-scope acquire, so the
// data written before the barrier is visible after it on every XCD.  The wait
// is bounded: after ~2^26 polls the workgroup raises the abort flag and
// leaves, so a broken co-residency assumption ends the kernel with an error
// instead of hanging the device.
__device__ __forceinline__ bool grid_barrier(unsigned* ctr, int* abort_flag, unsigned& target) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int aborted;
  if (threadIdx.x == 0) {
    target += gridDim.x;
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    unsigned polls = 0;
    int ab = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (((++polls) & 1023u) == 0) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ab = 1; break; }
        if (polls > (1u << 26)) {
          __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    aborted = ab;
  }
  __syncthreads();
  return aborted != 0;
}

// Split form of the same barrier: arrive once this workgroup's writes for the
// other workgroups are done, do work nobody waits for, then wait.
__device__ __forceinline__ void grid_arrive(unsigned* ctr, unsigned& target) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    target += gridDim.x;
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ bool grid_wait(unsigned* ctr, int* abort_flag, unsigned target) {
  __shared__ int aborted_w;
  if (threadIdx.x == 0) {
    unsigned polls = 0;
    int ab = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (((++polls) & 1023u) == 0) {
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ab = 1; break; }
        if (polls > (1u << 26)) {
          __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    aborted_w = ab;
  }
  __syncthreads();
  return aborted_w != 0;
}

// ---------------------------------------------------------------------------
// graph-engine kernels (one workgroup per (leaf, slot))
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void k_phase_A(Geom G, Bufs B, int off) {
  __shared__ Smem<T> sm;
  phase_A(G, B, blockIdx.x, *B.itbase + off, sm);
}

// absolute >= 0 selects a fixed iteration (0 = initial restriction of b).
template <typename T>
__global__ __launch_bounds__(NT) void k_phase_B(Geom G, Bufs B, int off, int absolute, int stage) {
  __shared__ Smem<T> sm;
  extern __shared__ float4 dyn4[];
  const int it = absolute >= 0 ? absolute : *B.itbase + off;
  phase_B(G, B, blockIdx.x, it, sm, reinterpret_cast<float*>(dyn4), stage);
}

template <typename T>
__global__ __launch_bounds__(NT) void k_phase_C(Geom G, Bufs B, int off, int absolute, int stage) {
  __shared__ Smem<T> sm;
  extern __shared__ float4 dyn4[];
  const int it = absolute >= 0 ? absolute : *B.itbase + off;
  phase_C(G, B, blockIdx.x, it, sm, reinterpret_cast<float*>(dyn4), stage);
}

// End of a replay: advance the iteration base and publish (replay count, all
// systems finished) to pinned host memory with a system-scope store.
__global__ void k_advance(Geom G, Bufs B, int unroll, int* host_flag) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  *B.itbase += unroll;
  const int rep = *B.replays + 1;
  *B.replays = rep;
  int done = 1;
  for (int s = 0; s < G.B; ++s) done &= (B.st[s].status != ST_RUNNING) ? 1 : 0;
  if (__hip_atomic_load(B.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) done = 1;
  __hip_atomic_store(host_flag, (rep << 1) | done, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Reset the control words and the nflags per-workgroup barrier lines before a
// solve (a kernel, not a memset, so that it can also sit inside captured work).
constexpr int kFlagStride = 32;   // unsigned words per barrier line (128 bytes)
__global__ void k_reset(Bufs B, int itbase, int* host_flag, int nflags) {
  for (int i = threadIdx.x; i < nflags; i += blockDim.x) B.wgflag[(size_t)i * kFlagStride] = 0u;
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  *B.barrier = 0u;
  *B.abort_flag = 0;
  *B.itbase = itbase;
  *B.replays = 0;
  if (host_flag) __hip_atomic_store(host_flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// persistent engine: workgroups loop over (leaf, slot) items, device-wide
// barriers separate the phases
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void k_persistent(Geom G, Bufs B) {
  __shared__ Smem<T> sm;
  extern __shared__ float4 dyn4[];
  float* dyn = reinterpret_cast<float*>(dyn4);
  unsigned target = 0;
  for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) { phase_B(G, B, b, 0, sm, dyn); __syncthreads(); }
  if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) { phase_C(G, B, b, 0, sm, dyn); __syncthreads(); }
  if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  for (int it = 1; it <= B.maxit; ++it) {
    // Statuses change only in phase C, before the barrier just passed, so every
    // workgroup reads the same values here and leaves the loop together.
    int running = 0;
    for (int s = threadIdx.x; s < G.B; s += NT)
      running |= (__hip_atomic_load(&B.st[s].status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ST_RUNNING);
    if (!__syncthreads_or(running)) break;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) { phase_A(G, B, b, it, sm); __syncthreads(); }
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) { phase_B(G, B, b, it, sm, dyn); __syncthreads(); }
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) { phase_C(G, B, b, it, sm, dyn); __syncthreads(); }
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  }
}

// ---------------------------------------------------------------------------
// standalone apply (fp32 in and out) and SpMV
// ---------------------------------------------------------------------------
// Restriction of r: per leaf slot, the t_k slice and the owned levels' W^T r_k.
__global__ __launch_bounds__(NT) void k_apply_restrict(Geom G, Bufs B, const float* __restrict__ rin) {
  __shared__ Smem<float> sm;
  extern __shared__ float4 dyn4[];
  float* dyn = reinterpret_cast<float*>(dyn4);
  const Blk bk = decode(G, blockIdx.x);
  issue_restrict_dma<float>(G, B, bk, dyn);
  if (threadIdx.x < LEAF) sm.r[threadIdx.x] = rin[bk.leaf0 + threadIdx.x];
  lds_dma_wait();
  restrict_leaf(G, B, bk, dyn, sm);
}

// Prolongation and assembly of y on the workgroup's rows.
__global__ __launch_bounds__(NT) void k_apply_prolong(Geom G, Bufs B, const float* __restrict__ rin,
                                                       float* __restrict__ yout) {
  __shared__ Smem<float> sm;
  extern __shared__ float4 dyn4[];
  float* dyn = reinterpret_cast<float*>(dyn4);
  const Blk bk = decode(G, blockIdx.x);
  issue_prolong_dma<float>(G, B, bk, dyn, sm);
  if (threadIdx.x < G.RB) sm.r[threadIdx.x] = rin[bk.grow0 + threadIdx.x];
  lds_dma_wait();
  const float y = prolong_rows(G, B, bk, dyn, sm);
  if (threadIdx.x < G.RB) yout[bk.grow0 + threadIdx.x] = y;
}


// Bridge format -> per-level slabs: for tile m of level l, a row-half leaf k
// gets W_l[k] = U~_k B_m and a column-half leaf gets W_l[k] = V~_k, which gives
// the same M with the identity core ("Hierarchical Transformer Preconditioning
// for Interactive Physics Simulation", section 5, eqs. (2)-(5): the row strip
// is prolonged through U~ B, the column strip restricted through V~).  One
// workgroup per (system, level, leaf); fp32 products.
__global__ __launch_bounds__(NT) void k_expand_bridge(Geom G, const float* __restrict__ Ub,
                                                      const float* __restrict__ Vb, const float* __restrict__ Bc,
                                                      float* __restrict__ W) {
  __shared__ float Bs[RANK * RANK];
  const int b = blockIdx.x;
  const int k = b % G.K, l = (b / G.K) % G.levels, s = b / (G.K * G.levels);
  const size_t slab = (size_t)LEAF * RANK;
  float* out = W + (((size_t)s * G.levels + l) * G.K + k) * slab;
  const size_t leaf_off = ((size_t)s * G.K + k) * slab;
  if (((k >> l) & 1) != 0) {                     // column half: V~_k
    for (int e = threadIdx.x; e < LEAF * RANK; e += NT) out[e] = Vb[leaf_off + e];
    return;
  }
  int m = 0;                                     // tile index: level-major, j ascending
  for (int ll = 0; ll < l; ++ll) m += G.K >> (ll + 1);
  m += k >> (l + 1);
  const int cores = [&] { int c = 0; for (int ll = 0; ll < G.levels; ++ll) c += G.K >> (ll + 1); return c; }();
  const float* B = Bc + ((size_t)s * cores + m) * RANK * RANK;
  for (int e = threadIdx.x; e < RANK * RANK; e += NT) Bs[e] = B[e];
  __syncthreads();
  const float* Uk = Ub + leaf_off;
  for (int e = threadIdx.x; e < LEAF * RANK; e += NT) {
    const int i = e / RANK, c = e - i * RANK;
    float a = 0.f;
#pragma unroll 8
    for (int t = 0; t < RANK; ++t) a = fmaf(Uk[i * RANK + t], Bs[t * RANK + c], a);
    out[e] = a;
  }
}

// ---------------------------------------------------------------------------
// outer refinement (fp64 residual of the fp32 matrix, per-system scaling)
// ---------------------------------------------------------------------------
// r = b - A x in fp64 (thread per row).
__global__ void k_residual64(const int* __restrict__ row_ptr, const int* __restrict__ col,
                             const float* __restrict__ val, const float* __restrict__ b,
                             const double* __restrict__ x, double* __restrict__ r, int nrows) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows) return;
  double acc = 0.0;
  for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e) acc = fma((double)val[e], x[col[e]], acc);
  r[i] = (double)b[i] - acc;
}

// Per-system sum of squares of v (one workgroup per system, fixed order).
__global__ __launch_bounds__(NT) void k_sys_sumsq(const double* __restrict__ v, int n, double* __restrict__ out) {
  __shared__ double red[NWAVE];
  const double* p = v + (size_t)blockIdx.x * n;
  double a = 0.0;
  for (int i = threadIdx.x; i < n; i += NT) a = fma(p[i], p[i], a);
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = red[0];
    for (int w = 1; w < NWAVE; ++w) s += red[w];
    out[blockIdx.x] = s;
  }
}

// rhs = r * inv[s] rounded to fp32 (inv = 0 for a finished system).
__global__ void k_scale_rhs(const double* __restrict__ r, const double* __restrict__ inv, float* __restrict__ rhs,
                            int n, int N) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) rhs[i] = (float)(r[i] * inv[i / n]);
}

// x += scale[s] * d.
__global__ void k_add_scaled(double* __restrict__ x, const double* __restrict__ d, const double* __restrict__ scale,
                             int n, int N) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) x[i] = fma(scale[i / n], d[i], x[i]);
}

// dinv_i = 1 / A_ii (0 for a row without a stored diagonal).
__global__ void k_diag_inv(const int* __restrict__ row_ptr, const int* __restrict__ col,
                           const float* __restrict__ val, double* __restrict__ dinv, int nrows, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows) return;
  double d = 0.0;
  for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
    if (col[e] == i) d = (double)val[e];
  (void)n;
  dinv[i] = d != 0.0 ? 1.0 / d : 0.0;
}

// y = diag(A)^-1 r (fp32 in and out).
__global__ void k_jacobi_apply(const float* __restrict__ r, const double* __restrict__ dinv, float* __restrict__ y,
                               int nrows) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nrows) y[i] = (float)((double)r[i] * dinv[i]);
}

__global__ void k_copy_x(const double* __restrict__ src, double* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// Measurement aid: stream `n4` float4 from src as fast as one launch can
// (workgroup b reads the contiguous chunk b of gridDim.x, eight independent
// 16-byte loads in flight per thread), and write one sum per workgroup so the
// loads are not removed.  The read ceiling that the apply's bandwidth is set
// against.
constexpr int PROBE_NT = 256;
__global__ __launch_bounds__(PROBE_NT) void k_read_probe(const float4* __restrict__ src, size_t n4,
                                                        float* __restrict__ sink) {
  __shared__ float red[PROBE_NT / 64];
  const size_t chunk = (n4 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * chunk;
  const size_t end = beg + chunk < n4 ? beg + chunk : n4;
  float acc = 0.f;
  size_t i = beg + threadIdx.x;
  for (; i + 7 * PROBE_NT < end; i += 8 * PROBE_NT) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[i + j * PROBE_NT];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  }
  for (; i < end; i += PROBE_NT) {
    const float4 v = src[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace hpcg
