// Single-pass H-matrix apply in the pages' own off-diagonal format
// ("Hierarchical Transformer Preconditioning for Interactive Physics
// Simulation", section 5 "Preconditioner Application", eqs. (2)-(5);
// Supplementary section 2 and Table 3): per leaf k the two bridges U~_k, V~_k
// of L x R and per tile m one R x R core B_m, O(N) factor bytes in place of the
// per-level slabs' O(N log N).
//
//   restriction          u^_k = U~_k^T r_k,  v^_k = V~_k^T r_k          (one pair per leaf)
//   strip aggregation    s^r_m = sum over R_m of u^,  s^c_m = sum over C_m of v^
//   coarse coupling      t^c_m = B_m^T s^r_m,  t^r_m = B_m s^c_m
//   prolongation         y_k += U~_k (sum of t^r over k's row-half tiles)
//                             + V~_k (sum of t^c over its column-half tiles)
//
// The coupling is linear, so it is applied by the producer before the
// exchange: the leaf of the row half of level l's tile m publishes B_m^T u^_k,
// a leaf of the column half B_m v^_k, and the partner-half sums that a
// consumer gathers are t^c_m and t^r_m themselves.  The words are those of
// the slab apply (level l, leaf k, 32 values with the call epoch), so the
// exchange is the same; the producer's 32 x 32 products run while the leaf
// factor U_k is still in flight, off the critical path.  The workgroup of a
// leaf holds U~_k and V~_k in the register layout of two level slabs, so the
// restriction and the prolongation are the slab kernels' with two "levels";
// the cores of the leaf's tiles go to LDS (row stride R + 1: both B and B^T
// are read without bank conflicts).
#pragma once
#include "hpcg_leaf.hpp"

namespace hpcg {

constexpr int CSTRIDE = RANK + 1;   // LDS row stride of a core

// Tile (core) index of leaf k at level l: level-major, j = k >> (l + 1) ascending.
__device__ __forceinline__ int core_index(int K, int l, int k) {
  int m = 0;
  for (int ll = 0; ll < l; ++ll) m += K >> (ll + 1);
  return m + (k >> (l + 1));
}

// U~_k, V~_k into the slab register layout of Resident<float, 2> (w[0], w[1]).
__device__ __forceinline__ void load_bridges(const Geom& G, const Bufs& B, int s, int k, Resident<float, 2>& F) {
  const int tid = threadIdx.x;
  const int c8 = tid & 7, row = tid >> 3;
  const size_t off = ((size_t)s * G.K + k) * LEAF * RANK;
  const float* U = B.Ub + off;
  const float* V = B.Vb + off;
  F.w[0][0] = *reinterpret_cast<const float4*>(U + row * RANK + 4 * c8);
  F.w[0][1] = *reinterpret_cast<const float4*>(U + (row + 64) * RANK + 4 * c8);
  F.w[1][0] = *reinterpret_cast<const float4*>(V + row * RANK + 4 * c8);
  F.w[1][1] = *reinterpret_cast<const float4*>(V + (row + 64) * RANK + 4 * c8);
}

// The cores of leaf k's LEV tiles into LDS (level l at cores + l * R * CSTRIDE).
// Each thread moves float4s of whole core rows, so the loads are issued first
// and the (strided) LDS stores wait for them only when the caller asks.
template <int LEV>
struct CoreRegs {
  static constexpr int PER = (LEV * RANK * RANK / 4 + NTR - 1) / NTR;   // float4 per thread
  float4 v[PER > 0 ? PER : 1];
};

template <int LEV>
__device__ __forceinline__ void load_cores(const Geom& G, const Bufs& B, int s, int k, CoreRegs<LEV>& C) {
  const int tid = threadIdx.x;
  const float* base = B.Bc + (size_t)s * B.ncores * RANK * RANK;
#pragma unroll
  for (int j = 0; j < CoreRegs<LEV>::PER; ++j) {
    const int e = tid + j * NTR;                 // float4 index over the LEV cores
    if (e < LEV * RANK * RANK / 4) {
      const int l = e / (RANK * RANK / 4), w = e - l * (RANK * RANK / 4);
      C.v[j] = reinterpret_cast<const float4*>(base + (size_t)core_index(G.K, l, k) * RANK * RANK)[w];
    }
  }
}

template <int LEV>
__device__ __forceinline__ void store_cores(const CoreRegs<LEV>& C, float* cores) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < CoreRegs<LEV>::PER; ++j) {
    const int e = tid + j * NTR;
    if (e < LEV * RANK * RANK / 4) {
      const int l = e / (RANK * RANK / 4), w = e - l * (RANK * RANK / 4);
      const int row = (4 * w) / RANK, col = (4 * w) % RANK;
      float* d = cores + l * RANK * CSTRIDE + row * CSTRIDE + col;
      d[0] = C.v[j].x;
      d[1] = C.v[j].y;
      d[2] = C.v[j].z;
      d[3] = C.v[j].w;
    }
  }
}

// u^ and v^ summed over the waves' partials, then per level l the coupled
// value published for the partners: B_m^T u^ when k is in the row half of its
// level-l tile m, B_m v^ when in the column half (two threads per output, each
// half of the 32-term dot, added with one lane swap).  One barrier.
template <int LEV>
__device__ __forceinline__ void couple_and_publish(const Geom& G, const Bufs& B, RSmem<float>& sm,
                                                   const float* cores, int s, int k, unsigned want) {
  const int tid = threadIdx.x;
  if (tid < 2 * RANK) {
    float a = sm.redW[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
    sm.ownR[tid] = a;                              // [0, R): u^, [R, 2R): v^
  }
  __syncthreads();
  const int o = tid >> 1, half = tid & 1;
  float t = 0.f;
  if (o < LEV * RANK) {
    const int l = o / RANK, i = o - l * RANK;
    const bool row_half = ((k >> l) & 1) == 0;
    const float* Bm = cores + l * RANK * CSTRIDE;
    const float* v = sm.ownR + (row_half ? 0 : RANK);
#pragma unroll
    for (int jj = 0; jj < RANK / 2; ++jj) {
      const int j = half * (RANK / 2) + jj;
      t = fmaf(row_half ? Bm[j * CSTRIDE + i] : Bm[i * CSTRIDE + j], v[j], t);
    }
  }
  t += __shfl_xor(t, 1);
  if (o < LEV * RANK && half == 0) {
    const int l = o / RANK, i = o - l * RANK;
    st_c(B.llw + (((size_t)s * G.levels + l) * G.K + k) * RANK + i, ((unsigned long long)want << 32) | __float_as_uint(t));
  }
}

// Strip aggregation of the gathered coupled values per side, from the waves'
// partials that gather_sum_ll leaves (level l, column c): sm.P[0, R) = the
// levels where k is in the row half (they multiply U~_k), sm.P[R, 2R) = the
// others (V~_k), across waves and levels in a fixed order.  One barrier.
template <int LEV>
__device__ __forceinline__ void bridge_sides_from_partials(RSmem<float>& sm, int k) {
  const int tid = threadIdx.x;
  if (tid < 2 * RANK) {
    const int side = tid / RANK, cc = tid - side * RANK;
    float p = 0.f;
    // every level's partials are read (no branch, so all reads are in flight
    // at once); the other side's levels add zero
#pragma unroll
    for (int l = 0; l < LEV; ++l) {
      float q = sm.redW[0][MAX_LEVELS * RANK + l * RANK + cc];
#pragma unroll
      for (int w = 1; w < NWR; ++w) q += sm.redW[w][MAX_LEVELS * RANK + l * RANK + cc];
      p += ((k >> l) & 1) == side ? q : 0.f;
    }
    sm.P[tid] = p;
  }
  __syncthreads();
}

// One launch over whole systems (item0 = first leaf of the launch; every
// leaf of a launch on its own compute unit).  SPLIT: two workgroups per leaf,
// the diagonal one (even blockIdx) computing U_k U_k^T r and publishing it as
// flagged words, the off-diagonal one doing the rest and gathering those words
// with the partners' in the same poll rounds (as k_apply_split).
template <int LEV, bool SPLIT>
__global__ __launch_bounds__(NTR) void k_apply_bridge(Geom G, Bufs B, const float* __restrict__ rin,
                                                      float* __restrict__ yout, int item0) {
  static_assert(LEV >= 1, "the bridge apply needs tile levels");
  __shared__ RSmem<float> sm;
  extern __shared__ int4 bdyn4[];
  float* cores = reinterpret_cast<float*>(bdyn4);                 // LEV x R x CSTRIDE
  const int tid = threadIdx.x;
  const int item = item0 + (SPLIT ? (int)(blockIdx.x >> 1) : (int)blockIdx.x);
  const bool diag_role = SPLIT && (blockIdx.x & 1) == 0;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  stamp(blockIdx.x, 0);
  float rv = 0.f, gate = 0.f;
  if (tid < LEAF) {
    rv = rin[leaf0 + tid];
    if (!diag_role) gate = B.g[leaf0 + tid];
  }
  const unsigned want = ld_c(B.lle + item) + 1u;
  Resident<float, 2> F;
  if (diag_role) {
    load_leaf(G, B, s, k, F);
    if (tid < LEAF) sm.r[tid] = rv;
    __syncthreads();
    stamp(blockIdx.x, 1);
    restrict_u_partials<float, 2>(F, sm.r, sm);
    __syncthreads();
    if (tid < LEAF) {
      float a = sm.red[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
      sm.t[tid] = a;
    }
    __syncthreads();
    diag_times<float, 2>(F, sm.t, sm.yleaf);
    __syncthreads();
    if (tid < LEAF)
      st_c(B.lly + (size_t)item * LEAF + tid, ((unsigned long long)want << 32) | __float_as_uint(sm.yleaf[tid]));
    stamp(blockIdx.x, 2);
    return;
  }
  load_bridges(G, B, s, k, F);
  CoreRegs<LEV> C;
  load_cores<LEV>(G, B, s, k, C);
  if (tid < LEAF) sm.r[tid] = rv;
  store_cores<LEV>(C, cores);
  __syncthreads();
  stamp(blockIdx.x, 1);
  restrict_w_partials<float, 2>(F, sm.r, sm);
  __syncthreads();
  couple_and_publish<LEV>(G, B, sm, cores, s, k, want);
  stamp(blockIdx.x, 2);
  if constexpr (!SPLIT) {
    load_leaf(G, B, s, k, F);
    restrict_u_partials<float, 2>(F, sm.r, sm);
    __syncthreads();
    if (tid < LEAF) {
      float a = sm.red[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
      sm.t[tid] = a;
    }
    __syncthreads();
    stamp(blockIdx.x, 3);
    prolong_diag<float, 2>(F, sm);
    stamp(blockIdx.x, 4);
  }
  gather_sum_ll<LEV, SPLIT>(G, B, s, k, item, want, sm, sm.yleaf);
  __syncthreads();
  stamp(blockIdx.x, 5);
  bridge_sides_from_partials<LEV>(sm, k);
  stamp(blockIdx.x, 8);
  prolong_offdiag<float, 2>(F, sm);
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
