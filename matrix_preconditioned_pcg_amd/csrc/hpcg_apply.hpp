// The two kernels of one apply + SpMV pair outside the solve engines: the
// single-pass H-matrix apply (every leaf on its own compute unit, factors read
// once, partners' restrictions exchanged as flagged words) and the CSR SpMV.
#pragma once
#include "hpcg_leaf.hpp"

namespace hpcg {

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
    // two of this thread's entries per round, both column indices and then
    // both x values in flight together; the sum keeps the entry order
    for (int e = row_ptr[row] + lr; e < e1; e += 2 * SPMV_TPR) {
      const int eb = e + SPMV_TPR;
      const bool hb = eb < e1;
      const int ca = col[e];
      const float va = val[e];
      int cb = ca;
      float vb = 0.f;
      if (hb) {
        cb = col[eb];
        vb = val[eb];
      }
      const float xa = x[ca], xb = x[cb];
      acc = fmaf(va, xa, acc);
      if (hb) acc = fmaf(vb, xb, acc);
    }
  }
#pragma unroll
  for (int o = 1; o < SPMV_TPR; o <<= 1) acc += __shfl_xor(acc, o);
  if (row < nrows && lr == 0) y[row] = acc;
}

// Single-launch apply y = M r (fp32 in and out) over whole systems whose leaves
// all get a compute unit (a larger batch runs as several launches, each over
// as many whole systems as fit, item0 being the first leaf of the launch,
// since a leaf waits only for leaves of its own system): the workgroup of
// leaf k loads U_k and its slabs into
// registers once, restricts (eq. (2)), gathers the partner halves'
// restrictions (eq. (3)), and prolongs (eqs. (4)-(5)) and adds the diagonal
// stage and the gate with the same registers, so every factor byte crosses HBM
// once per apply.
//
// No device-wide barrier: each restriction value travels with the number of
// the call that produced it, packed into one 8-byte word (value in the low
// half, epoch in the high half) that is stored and loaded as a whole with
// agent-scope atomics, so a reader that sees the epoch it expects also sees
// that call's value.  The epoch of a leaf counts the calls that leaf has
// completed (every call runs every leaf once, so all leaves agree at a call's
// start); the words hold the previous call's epoch until overwritten.  A
// reader therefore polls exactly the words it needs, and a workgroup waits for
// its partners only, for about one memory round trip after the last of them
// has written.  The polls are bounded: past the bound the abort flag is raised
// and the output is undefined (only if other work holds the device's compute
// units for about a second).
template <int LEV>
__device__ __forceinline__ void gather_partners_ll(const Geom& G, const Bufs& B, int s, int k, unsigned want,
                                                   float* stage) {
  if constexpr (LEV > 0) {
    // word w = row * RANK + c, row = 2^l - 1 + i: column c of the i-th leaf of
    // level l's partner half, staged at the same position
    constexpr int NWORDS = RANK * ((1 << LEV) - 1);
    constexpr int WPT = (NWORDS + NTR - 1) / NTR;
    const int tid = threadIdx.x;
    const unsigned long long* src[WPT];
    unsigned long long v[WPT];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int w = tid + j * NTR;
      src[j] = nullptr;
      if (w < NWORDS) {
        const int row = w / RANK, c = w - row * RANK;
        const int l = 31 - __clz(row + 1);
        const int kp = (((k >> l) ^ 1) << l) + (row + 1 - (1 << l));
        src[j] = B.llw + (((size_t)s * G.levels + l) * G.K + kp) * RANK + c;
        v[j] = ld_c(src[j]);
      }
    }
    // re-poll every word still short of its epoch together, so that a late
    // partner costs one round trip, not one per word
    unsigned pending = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if (src[j] && (unsigned)(v[j] >> 32) != want) pending |= 1u << j;
    unsigned polls = 0;
    while (pending) {
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < WPT; ++j)
        if (pending & (1u << j)) v[j] = ld_c(src[j]);
#pragma unroll
      for (int j = 0; j < WPT; ++j)
        if ((pending & (1u << j)) && (unsigned)(v[j] >> 32) == want) pending &= ~(1u << j);
      if (++polls > (1u << 20)) {
        st_c(B.abort_flag, 1);
        break;
      }
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if (src[j]) stage[tid + j * NTR] = __uint_as_float((unsigned)v[j]);
  }
}

template <int LEV>
__global__ __launch_bounds__(NTR) void k_apply_fused(Geom G, Bufs B, const float* __restrict__ rin,
                                                     float* __restrict__ yout, int item0) {
  __shared__ RSmem<float> sm;
  extern __shared__ int4 fdyn4[];
  float* stR = reinterpret_cast<float*>(fdyn4);
  const int tid = threadIdx.x;
  const int item = item0 + (int)blockIdx.x;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  // r, the gate and the epoch are issued before the factors: the loads
  // return in order, so storing r to LDS then waits for r alone
  float rv = 0.f, gate = 0.f;
  if (tid < LEAF) {
    rv = rin[leaf0 + tid];
    gate = B.g[leaf0 + tid];
  }
  const unsigned want = ld_c(B.lle + item) + 1u;
  Resident<float, LEV> F;
  load_factors(G, B, s, k, F);
  if (tid < LEAF) sm.r[tid] = rv;
  __syncthreads();
  // the slabs' restriction (what the partners need) first, then U_k^T r
  if constexpr (LEV > 0) {
    restrict_w_partials<float, LEV>(F, sm.r, sm);
    __syncthreads();
    if (tid < LEV * RANK) {
      float a = sm.redW[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
      const int l = tid / RANK, c = tid - l * RANK;
      st_c(B.llw + (((size_t)s * G.levels + l) * G.K + k) * RANK + c,
           ((unsigned long long)want << 32) | __float_as_uint(a));
    }
  }
  restrict_u_partials<float, LEV>(F, sm.r, sm);
  __syncthreads();
  if (tid < LEAF) {
    float a = sm.red[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
    sm.t[tid] = a;
  }
  __syncthreads();
  // the diagonal stage needs nothing from other leaves: it runs while the
  // partners' words are in flight
  prolong_diag<float, LEV>(F, sm);
  gather_partners_ll<LEV>(G, B, s, k, want, stR);
  __syncthreads();
  if constexpr (LEV > 0) prolong_strips<float, LEV>(sm, stR, (const float*)nullptr, 0.0);
  prolong_offdiag<float, LEV>(F, sm);
  __syncthreads();
  if (tid < LEAF) yout[leaf0 + tid] = sm.yleaf[tid] + sm.yoff[tid] + gate * sm.r[tid];
  if (tid == 0) st_c(B.lle + item, want);
}

// gather_partners_ll plus the leaf's own diagonal stage U_k U_k^T r published
// by its diagonal workgroup (LEAF words at B.lly[item]) into ydiag, in the
// same poll rounds.
template <int LEV>
__device__ __forceinline__ void gather_partners_diag_ll(const Geom& G, const Bufs& B, int s, int k, int item,
                                                        unsigned want, float* stage, float* ydiag) {
  constexpr int NP = RANK * ((1 << LEV) - 1);
  constexpr int NWORDS = NP + LEAF;
  constexpr int WPT = (NWORDS + NTR - 1) / NTR;
  static_assert(WPT <= 32, "poll mask");
  const int tid = threadIdx.x;
  const unsigned long long* src[WPT];
  unsigned long long v[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid + j * NTR;
    src[j] = nullptr;
    if (w < NP) {
      const int row = w / RANK, c = w - row * RANK;
      const int l = 31 - __clz(row + 1);
      const int kp = (((k >> l) ^ 1) << l) + (row + 1 - (1 << l));
      src[j] = B.llw + (((size_t)s * G.levels + l) * G.K + kp) * RANK + c;
    } else if (w < NWORDS) {
      src[j] = B.lly + (size_t)item * LEAF + (w - NP);
    }
    if (src[j]) v[j] = ld_c(src[j]);
  }
  unsigned pending = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j)
    if (src[j] && (unsigned)(v[j] >> 32) != want) pending |= 1u << j;
  unsigned polls = 0;
  while (pending) {
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if (pending & (1u << j)) v[j] = ld_c(src[j]);
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if ((pending & (1u << j)) && (unsigned)(v[j] >> 32) == want) pending &= ~(1u << j);
    if (++polls > (1u << 20)) {
      st_c(B.abort_flag, 1);
      break;
    }
  }
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid + j * NTR;
    if (w < NP) stage[w] = __uint_as_float((unsigned)v[j]);
    else if (w < NWORDS) ydiag[w - NP] = __uint_as_float((unsigned)v[j]);
  }
}

// Single-pass apply with two workgroups per leaf, by role, so that twice as
// many compute units pull factors: the diagonal workgroup (even blockIdx)
// loads U_k, computes U_k (U_k^T r) and publishes it as flagged words; the
// off-diagonal workgroup (odd) loads the slabs, restricts and publishes
// W_l[k]^T r, gathers the partner halves' restrictions and the diagonal
// result in the same poll rounds, prolongs and writes y.  Only the
// off-diagonal workgroup advances the leaf's epoch, and it does so after it
// has seen the diagonal workgroup's words, which were stamped with the epoch
// the diagonal workgroup read at its start: both agree on the call.
template <int LEV>
__global__ __launch_bounds__(NTR) void k_apply_split(Geom G, Bufs B, const float* __restrict__ rin,
                                                     float* __restrict__ yout) {
  static_assert(LEV > 0, "the split needs tile levels");
  __shared__ RSmem<float> sm;
  extern __shared__ int4 fdyn4[];
  float* stR = reinterpret_cast<float*>(fdyn4);
  const int tid = threadIdx.x;
  const int item = blockIdx.x >> 1;
  const bool diag_role = (blockIdx.x & 1) == 0;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  float rv = 0.f, gate = 0.f;
  if (tid < LEAF) {
    rv = rin[leaf0 + tid];
    if (!diag_role) gate = B.g[leaf0 + tid];
  }
  const unsigned want = ld_c(B.lle + item) + 1u;
  Resident<float, LEV> F;
  if (diag_role) {
    load_leaf(G, B, s, k, F);
    if (tid < LEAF) sm.r[tid] = rv;
    __syncthreads();
    restrict_u_partials<float, LEV>(F, sm.r, sm);
    __syncthreads();
    if (tid < LEAF) {
      float a = sm.red[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
      sm.t[tid] = a;
    }
    __syncthreads();
    diag_times<float, LEV>(F, sm.t, sm.yleaf);
    __syncthreads();
    if (tid < LEAF)
      st_c(B.lly + (size_t)item * LEAF + tid, ((unsigned long long)want << 32) | __float_as_uint(sm.yleaf[tid]));
    return;
  }
  load_slabs(G, B, s, k, F);
  if (tid < LEAF) sm.r[tid] = rv;
  __syncthreads();
  restrict_w_partials<float, LEV>(F, sm.r, sm);
  __syncthreads();
  if (tid < LEV * RANK) {
    float a = sm.redW[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
    const int l = tid / RANK, c = tid - l * RANK;
    st_c(B.llw + (((size_t)s * G.levels + l) * G.K + k) * RANK + c,
         ((unsigned long long)want << 32) | __float_as_uint(a));
  }
  gather_partners_diag_ll<LEV>(G, B, s, k, item, want, stR, sm.yleaf);
  __syncthreads();
  prolong_strips<float, LEV>(sm, stR, (const float*)nullptr, 0.0);
  prolong_offdiag<float, LEV>(F, sm);
  __syncthreads();
  if (tid < LEAF) yout[leaf0 + tid] = sm.yleaf[tid] + sm.yoff[tid] + gate * sm.r[tid];
  if (tid == 0) st_c(B.lle + item, want);
}

}  // namespace hpcg
