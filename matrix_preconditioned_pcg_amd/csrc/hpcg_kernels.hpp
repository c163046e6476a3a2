// Kernels of the H-matrix-preconditioned CG solve for gfx950 (wave64, 256 CUs).
//
// Two solve engines share the phase functions of hpcg_device.hpp:
//  * graph engine: one kernel per phase, G unrolled iterations captured in a
//    hipGraph and replayed; the host reads a pinned flag between replays.
//  * persistent engine: a single cooperative launch runs the whole solve; phases
//    are separated by a device-wide barrier, and each workgroup can keep its rows
//    of the factors resident in LDS for every iteration.
// Standalone kernels serve hpcg_apply_M and hpcg_spmv.
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

// ---------------------------------------------------------------------------
// device-wide barrier (persistent engine)
// ---------------------------------------------------------------------------
// Every workgroup arrives once per barrier on a monotonically increasing
// counter; barrier number m completes when the counter reaches m * gridDim.x.
// The wait is bounded: after ~2^26 polls (seconds) the workgroup raises the
// abort flag and leaves, so a broken co-residency assumption ends the kernel
// with an error instead of hanging the device.
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

// ---------------------------------------------------------------------------
// graph-engine kernels (one workgroup per row block)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void k_init(Geom G, Bufs B) {
  __shared__ Smem<T> sm;
  const int b = blockIdx.x;
  phase_init(G, B, b, global_view(G, B, decode(G, b)), sm);
}

template <typename T>
__global__ __launch_bounds__(NT) void k_phase_A(Geom G, Bufs B, int off) {
  __shared__ Smem<T> sm;
  phase_A(G, B, blockIdx.x, *B.itbase + off, sm);
}

template <typename T>
__global__ __launch_bounds__(NT) void k_phase_B(Geom G, Bufs B, int off) {
  __shared__ Smem<T> sm;
  const int b = blockIdx.x;
  phase_B(G, B, b, *B.itbase + off, global_view(G, B, decode(G, b)), sm);
}

template <typename T>
__global__ __launch_bounds__(NT) void k_phase_C(Geom G, Bufs B, int off, int absolute) {
  __shared__ Smem<T> sm;
  const int b = blockIdx.x;
  const int it = absolute >= 0 ? absolute : *B.itbase + off;
  phase_C(G, B, b, it, global_view(G, B, decode(G, b)), sm);
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

// Reset the control words before a solve (a kernel, not a memset, so that it
// can also sit inside captured work).
__global__ void k_reset(Bufs B, int itbase, int* host_flag) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  *B.barrier = 0u;
  *B.abort_flag = 0;
  *B.itbase = itbase;
  *B.replays = 0;
  if (host_flag) __hip_atomic_store(host_flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// persistent engine
// ---------------------------------------------------------------------------
// RES: each workgroup owns exactly one row block and copies its rows of U_k and
// of the level slabs into dynamic LDS once; every later apply reads them there.
template <typename T, bool RES>
__global__ __launch_bounds__(NT) void k_persistent(Geom G, Bufs B) {
  __shared__ Smem<T> sm;
  extern __shared__ float4 dyn4[];
  unsigned target = 0;
  FactorView fres{};
  if constexpr (RES) {
    const Blk bk = decode(G, blockIdx.x);
    const FactorView gv = global_view(G, B, bk);
    float* dyn = reinterpret_cast<float*>(dyn4);
    const int RB = G.RB;
    float4* du = reinterpret_cast<float4*>(dyn);
    for (int e = threadIdx.x; e < RB * LEAF / 4; e += NT) du[e] = ld4(gv.Ub + 4 * e);
    float* dw = dyn + RB * LEAF;
    for (int l = 0; l < G.levels; ++l) {
      float4* d = reinterpret_cast<float4*>(dw + (size_t)l * RB * RANK);
      const float* src = gv.Wb + (size_t)l * gv.wstride;
      for (int e = threadIdx.x; e < RB * RANK / 4; e += NT) d[e] = ld4(src + 4 * e);
    }
    fres.Ub = dyn;
    fres.Wb = dw;
    fres.wstride = (size_t)RB * RANK;
    __syncthreads();
  }
  auto view = [&](int b) -> FactorView {
    if constexpr (RES) return fres;
    else return global_view(G, B, decode(G, b));
  };
  for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) phase_init(G, B, b, view(b), sm);
  if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) phase_C(G, B, b, 0, view(b), sm);
  if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  for (int it = 1; it <= B.maxit; ++it) {
    // Statuses change only in phase C, before the barrier just passed, so every
    // workgroup reads the same values here and leaves the loop together.
    int running = 0;
    for (int s = threadIdx.x; s < G.B; s += NT)
      running |= (__hip_atomic_load(&B.st[s].status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ST_RUNNING);
    if (!__syncthreads_or(running)) break;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) phase_A(G, B, b, it, sm);
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) phase_B(G, B, b, it, view(b), sm);
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
    for (int b = blockIdx.x; b < G.nblk; b += gridDim.x) phase_C(G, B, b, it, view(b), sm);
    if (grid_barrier(B.barrier, B.abort_flag, target)) return;
  }
}

// ---------------------------------------------------------------------------
// standalone apply and SpMV
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void k_apply_restrict(Geom G, Bufs B, const float* __restrict__ rin) {
  __shared__ Smem<float> sm;
  const Blk bk = decode(G, blockIdx.x);
  if (threadIdx.x < G.RB) sm.r[threadIdx.x] = rin[bk.grow0 + threadIdx.x];
  __syncthreads();
  restrict_block(G, B, bk, global_view(G, B, bk), sm);
}

__global__ __launch_bounds__(NT) void k_apply_prolong(Geom G, Bufs B, const float* __restrict__ rin,
                                                       float* __restrict__ yout) {
  __shared__ Smem<float> sm;
  const Blk bk = decode(G, blockIdx.x);
  if (threadIdx.x < G.RB) sm.r[threadIdx.x] = rin[bk.grow0 + threadIdx.x];
  __syncthreads();
  const float y = prolong_block(G, B, bk, global_view(G, B, bk), sm);
  if (threadIdx.x < G.RB) yout[bk.grow0 + threadIdx.x] = y;
}

// y = A x; SPMV_TPR consecutive lanes share a row and stride over its entries.
constexpr int SPMV_TPR = 4;
constexpr int SPMV_ROWS = NT / SPMV_TPR;

__global__ __launch_bounds__(NT) void k_spmv(const int* __restrict__ row_ptr, const int* __restrict__ col,
                                             const float* __restrict__ val, const float* __restrict__ x,
                                             float* __restrict__ y, int nrows) {
  const int tid = threadIdx.x;
  const int row = blockIdx.x * SPMV_ROWS + tid / SPMV_TPR;
  const int lr = tid & (SPMV_TPR - 1);
  float acc = 0.f;
  if (row < nrows) {
    const int e1 = row_ptr[row + 1];
    for (int e = row_ptr[row] + lr; e < e1; e += SPMV_TPR) acc = fmaf(val[e], x[col[e]], acc);
  }
#pragma unroll
  for (int o = 1; o < SPMV_TPR; o <<= 1) acc += __shfl_xor(acc, o);
  if (row < nrows && lr == 0) y[row] = acc;
}

__global__ void k_copy_x(const double* __restrict__ src, double* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace hpcg
