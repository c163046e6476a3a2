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
  stamp(blockIdx.x, 0);
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
#ifdef HPCG_TRACE
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  stamp(blockIdx.x, 7);
#endif
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
// has written.  The polls are bounded (B.apply_poll_limit, about a second by
// default): past the bound the workgroup raises the apply's own abort word,
// which stays set until the host reads it, and finishes with whatever words
// it has, so the output is undefined but every workgroup exits and every
// leaf's epoch still advances by one (the next call is consistent).

// The partners' restriction words polled and summed per level as they land:
// thread (column c = tid % 32, group g = tid / 32 of 16) loads, for every
// level l, the words of the partner half's leaves g, g + 16, ... at once, adds
// them in that order, and the two groups of a wave are folded into the wave's
// partial of each (level, column), stored at sm.redW[wave][MAX_LEVELS * RANK +
// l * RANK + c] (the half of redW the restriction does not use, so no barrier
// is needed before it): the first stage of prolong_strips over staged words,
// without staging them.  DIAG: also the leaf's diagonal-stage words (LEAF of
// them at B.lly[item], from its diagonal workgroup) into ydiag, in the same
// poll rounds.  No barrier.
template <int LEV>
constexpr int strip_slot0(int l) {
  int n = 0;
  for (int i = 0; i < l; ++i) n += ((1 << i) + 15) / 16;
  return n;
}

template <int LEV, bool DIAG>
__device__ __forceinline__ void gather_sum_ll(const Geom& G, const Bufs& B, int s, int k, int item, unsigned want,
                                              RSmem<float>& sm, float* ydiag) {
  static_assert(LEV > 0, "levels only");
  constexpr int NS = strip_slot0<LEV>(LEV);
  static_assert(NS <= 31, "poll mask");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 31, g = tid >> 5;
  const bool hi = (lane & 32) != 0;
  const unsigned long long* base = B.llw + (size_t)s * G.levels * G.K * RANK;
  auto addr = [&](int l, int i) { return base + ((size_t)l * G.K + (((k >> l) ^ 1) << l) + i) * RANK + c; };
  // The split kernel's off-diagonal workgroup reaches this poll right after
  // publishing its own words, before most partners' words can be visible: a
  // first round then finds few of them, and the rest cost a second round
  // trip.  A short wait first (12 x 64 clocks, ~0.3 us) lets one round find
  // nearly all of them (measured: N8k 5.92 -> 5.24 us, tet4k 5.30 -> 4.78;
  // with fewer than five levels no gain, so no wait).
  if constexpr (DIAG && LEV >= 5) __builtin_amdgcn_s_sleep(12);
  unsigned long long v[NS];
  unsigned pending = 0;
#pragma unroll
  for (int l = 0; l < LEV; ++l)
#pragma unroll
    for (int m = 0; m < ((1 << l) + 15) / 16; ++m) {
      const int i = g + 16 * m, j = strip_slot0<LEV>(l) + m;
      if (i < (1 << l)) {
        v[j] = ld_c(addr(l, i));
        pending |= 1u << j;
      }
    }
  const unsigned long long* dsrc = B.lly + (size_t)item * LEAF + tid;
  unsigned long long dv = 0;
  if (DIAG && tid < LEAF) {
    dv = ld_c(dsrc);
    pending |= 1u << NS;
  }
  auto settle = [&]() {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if ((pending & (1u << j)) && (unsigned)(v[j] >> 32) == want) pending &= ~(1u << j);
    if (DIAG && (pending & (1u << NS)) && (unsigned)(dv >> 32) == want) pending &= ~(1u << NS);
  };
  settle();
  stamp(blockIdx.x, 10);
  unsigned polls = 0;
  while (pending) {
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int l = 0; l < LEV; ++l)
#pragma unroll
      for (int m = 0; m < ((1 << l) + 15) / 16; ++m) {
        const int j = strip_slot0<LEV>(l) + m;
        if (pending & (1u << j)) v[j] = ld_c(addr(l, g + 16 * m));
      }
    if (DIAG && (pending & (1u << NS))) dv = ld_c(dsrc);
    settle();
    if (pending && ++polls > B.apply_poll_limit) {
      st_c(B.apply_abort, 1);
      break;
    }
  }
  float a[LEV];
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    a[l] = 0.f;
#pragma unroll
    for (int m = 0; m < ((1 << l) + 15) / 16; ++m)
      if (g + 16 * m < (1 << l)) a[l] += __uint_as_float((unsigned)v[strip_slot0<LEV>(l) + m]);
  }
  float* d = &sm.redW[wave][MAX_LEVELS * RANK + c];
#pragma unroll
  for (int l = 0; l + 1 < LEV; l += 2) d[(hi ? l + 1 : l) * RANK] = fold_x32(a[l], a[l + 1]);
  if constexpr (LEV % 2 == 1) {
    const float f = a[LEV - 1] + lane_x32(a[LEV - 1]);
    if (!hi) d[(LEV - 1) * RANK] = f;
  }
  if (DIAG && tid < LEAF) ydiag[tid] = __uint_as_float((unsigned)dv);
}

// Strip aggregation after gather_sum_ll (after a barrier): P_l[c] = the sum of
// the waves' partials.  One barrier.
template <int LEV>
__device__ __forceinline__ void strips_from_partials(RSmem<float>& sm) {
  const int tid = threadIdx.x;
  if (tid < LEV * RANK) {
    float a = sm.redW[0][MAX_LEVELS * RANK + tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.redW[w][MAX_LEVELS * RANK + tid];
    sm.P[tid] = a;
  }
  __syncthreads();
}

template <int LEV>
__global__ __launch_bounds__(NTR) void k_apply_fused(Geom G, Bufs B, const float* __restrict__ rin,
                                                     float* __restrict__ yout, int item0) {
  __shared__ RSmem<float> sm;
  const int tid = threadIdx.x;
  const int item = item0 + (int)blockIdx.x;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  stamp(blockIdx.x, 0);
  // r, the gate and the epoch are issued before the factors: the loads
  // return in order, so storing r to LDS then waits for r alone
  float rv = 0.f, gate = 0.f;
  if (tid < LEAF) {
    rv = rin[leaf0 + tid];
    gate = B.g[leaf0 + tid];
  }
  const unsigned want = ld_c(B.lle + item) + 1u;
  Resident<float, LEV> F;
  load_slabs(G, B, s, k, F);
  if (tid < LEAF) sm.r[tid] = rv;
  __syncthreads();
  stamp(blockIdx.x, 1);
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
  stamp(blockIdx.x, 2);
  // U_k only now, so that r and the slabs, which the partners wait for,
  // arrive ahead of it (the 64-system batch's launches 25.8 -> 24.9 us)
  load_leaf(G, B, s, k, F);
  restrict_u_partials<float, LEV>(F, sm.r, sm);
  __syncthreads();
  if (tid < LEAF) {
    float a = sm.red[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
    sm.t[tid] = a;
  }
  __syncthreads();
  stamp(blockIdx.x, 3);
  // the diagonal stage needs nothing from other leaves: it runs while the
  // partners' words are in flight
  prolong_diag<float, LEV>(F, sm);
  stamp(blockIdx.x, 4);
  if constexpr (LEV > 0) gather_sum_ll<LEV, false>(G, B, s, k, item, want, sm, nullptr);
  __syncthreads();
  stamp(blockIdx.x, 5);
  if constexpr (LEV > 0) strips_from_partials<LEV>(sm);
  stamp(blockIdx.x, 8);
  prolong_offdiag<float, LEV>(F, sm);
  stamp(blockIdx.x, 9);
  __syncthreads();
  stamp(blockIdx.x, 6);
  if (tid < LEAF) yout[leaf0 + tid] = sm.yleaf[tid] + sm.yoff[tid] + gate * sm.r[tid];
  if (tid == 0) st_c(B.lle + item, want);
#ifdef HPCG_TRACE
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  stamp(blockIdx.x, 7);
#endif
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
  const int tid = threadIdx.x;
  const int item = blockIdx.x >> 1;
  const bool diag_role = (blockIdx.x & 1) == 0;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  stamp(blockIdx.x, 0);
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
    stamp(blockIdx.x, 1);
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
    stamp(blockIdx.x, 2);
    return;
  }
  load_slabs(G, B, s, k, F);
  if (tid < LEAF) sm.r[tid] = rv;
  __syncthreads();
  stamp(blockIdx.x, 1);
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
  stamp(blockIdx.x, 2);
  gather_sum_ll<LEV, true>(G, B, s, k, item, want, sm, sm.yleaf);
  __syncthreads();
  stamp(blockIdx.x, 5);
  strips_from_partials<LEV>(sm);
  prolong_offdiag<float, LEV>(F, sm);
  __syncthreads();
  stamp(blockIdx.x, 6);
  if (tid < LEAF) yout[leaf0 + tid] = sm.yleaf[tid] + sm.yoff[tid] + gate * sm.r[tid];
  if (tid == 0) st_c(B.lle + item, want);
#ifdef HPCG_TRACE
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  stamp(blockIdx.x, 7);
#endif
}

}  // namespace hpcg
