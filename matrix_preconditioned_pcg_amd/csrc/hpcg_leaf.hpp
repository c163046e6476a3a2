// Leaf-resident building blocks for gfx950: one workgroup of NTR = 512
// threads (8 wave64 wavefronts) per leaf, U_k and the leaf's level slabs held
// in VGPRs, and the restriction / prolongation steps of the H-matrix apply on
// them.  Shared by the single-pass apply and the register-resident solve.
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

constexpr int NTR = 512;
constexpr int NWR = NTR / 64;

template <typename T>
struct alignas(16) RSmem {
  T r[LEAF];
  T q[LEAF];
  T z[LEAF];
  T p[LEAF];                         // p of the current iteration (own rows)
  T tr[LEAF];                        // U_k^T r
  T tq[LEAF];                        // U_k^T q
  T t[LEAF];                         // U_k^T r_new = tr - alpha tq
  T P[MAX_LEVELS * RANK];            // partner-half sums
  T ownR[MAX_LEVELS * RANK];         // this leaf's W_l[k]^T r
  T ownQ[MAX_LEVELS * RANK];         // this leaf's W_l[k]^T q
  T yleaf[LEAF];
  T yoff[LEAF];
  T yr[LEAF];                        // U_k U_k^T r (resident solve)
  T yq[LEAF];                        // U_k U_k^T q (resident solve)
  T red[NWR][LEAF];                  // cross-wave reductions of t
  T redW[NWR][2 * MAX_LEVELS * RANK];  // cross-wave reductions (restriction, strip sums)
  double dred[NWR];
  double dred2[NWR];
  double dsc[4];
  int flag[4];
};

// Agent-scope (XCD-coherent) load and store of one value.
template <typename T>
__device__ __forceinline__ T ld_c(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_c(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Register budget of the leaf steps (see tid_of): with fp64 vectors and six
// or more levels the hoisted addresses no longer fit beside the resident
// factors, so the steps recompute them; from seven levels the partner staging
// does too.  (Measured per level: below these the hoisted form is faster.)
template <typename T, int LEV>
constexpr bool kFresh = sizeof(T) == 8 && LEV >= 6;
template <typename T, int LEV>
constexpr bool kFreshDma = sizeof(T) == 8 && LEV >= 7;

template <typename T, int LEV>
struct Resident {
  float4 u[8];
  float4 w[LEV > 0 ? LEV : 1][2];
};

// Per-wave partials of U_k^T v into sm.red[wave] (thread = 4-column slot cs
// of 32, row group rg of 16; the two row groups of a wave are added with xor
// 32).  No barrier.
template <typename T, int LEV>
__device__ __forceinline__ void restrict_u_partials(const Resident<T, LEV>& F, const T* v, RSmem<T>& sm) {
  const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
  const int cs = tid & 31, rg = tid >> 5;
  Vec4<T> acc{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 8; ++m) axpy4(acc, F.u[m], v[rg + 16 * m]);
  // lanes < 32 finish components x and z, lanes >= 32 components y and w
  const T f0 = fold_x32(acc.x, acc.y), f1 = fold_x32(acc.z, acc.w);
  T* d = &sm.red[wave][4 * cs + (lane >> 5)];
  d[0] = f0;
  d[2] = f1;
}

// Per-wave partials of W_l[k]^T v for every level into sm.redW[wave].
// Thread = (4-column slot cs of 8, rows row and row + 64); the eight rows of
// a wave (lane bits 3..5) are folded per pair of levels with a
// transpose-reduce: 8 values -> 1 per lane in 4 + 2 + 1 shuffles.  No barrier.
template <typename T, int LEV>
__device__ __forceinline__ void restrict_w_partials(const Resident<T, LEV>& F, const T* v, RSmem<T>& sm) {
  if constexpr (LEV > 0) {
    const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
    const int cs = tid & 7, row = tid >> 3;
    const T r0 = v[row], r1 = v[row + 64];
    const bool b5 = (lane & 32) != 0, b4 = (lane & 16) != 0, b3 = (lane & 8) != 0;
    const int which = (b5 ? 4 : 0) + (b4 ? 2 : 0) + (b3 ? 1 : 0);   // value index a lane ends with
#pragma unroll
    for (int l0 = 0; l0 < LEV; l0 += 2) {
      T x[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        Vec4<T> acc{0, 0, 0, 0};
        if (l0 + h < LEV) {
          axpy4(acc, F.w[l0 + h < LEV ? l0 + h : 0][0], r0);
          axpy4(acc, F.w[l0 + h < LEV ? l0 + h : 0][1], r1);
        }
        x[4 * h + 0] = acc.x; x[4 * h + 1] = acc.y; x[4 * h + 2] = acc.z; x[4 * h + 3] = acc.w;
      }
      T a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = fold_x32(x[i], x[4 + i]);
      T bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) bb[i] = fold_x16(a[i], a[2 + i]);
      T kk = b3 ? bb[1] : bb[0];
      kk += lane_x8(b3 ? bb[0] : bb[1]);
      // value index `which` = 4h + component: level l0 + which/4, column 4cs + which%4
      const int l = l0 + (which >> 2);
      if (l < LEV) sm.redW[wave][l * RANK + 4 * cs + (which & 3)] = kk;
    }
  }
}

// The leaf's level slabs into the register layout of Resident.
template <typename T, int LEV>
__device__ __forceinline__ void load_slabs(const Geom& G, const Bufs& B, int s, int k, Resident<T, LEV>& F) {
  if constexpr (LEV > 0) {
    const int tid = threadIdx.x;
    const int c8 = tid & 7, row = tid >> 3;
#pragma unroll
    for (int l = 0; l < LEV; ++l) {
      const float* Wl = B.W + (((size_t)s * G.levels + l) * G.K + k) * LEAF * RANK;
      F.w[l][0] = *reinterpret_cast<const float4*>(Wl + row * RANK + 4 * c8);
      F.w[l][1] = *reinterpret_cast<const float4*>(Wl + (row + 64) * RANK + 4 * c8);
    }
  }
}

// U_k into the register layout of Resident.
template <typename T, int LEV>
__device__ __forceinline__ void load_leaf(const Geom& G, const Bufs& B, int s, int k, Resident<T, LEV>& F) {
  const int tid = threadIdx.x;
  const int cs = tid & 31, rg = tid >> 5;
  const float* Uk = B.U + ((size_t)s * G.K + k) * LEAF * LEAF;
#pragma unroll
  for (int m = 0; m < 8; ++m) F.u[m] = *reinterpret_cast<const float4*>(Uk + (rg + 16 * m) * LEAF + 4 * cs);
}

// U_k and the leaf's level slabs into the register layout of Resident (slabs
// first: the single-pass apply publishes their restriction before it needs
// U_k).
template <typename T, int LEV>
__device__ __forceinline__ void load_factors(const Geom& G, const Bufs& B, int s, int k, Resident<T, LEV>& F) {
  load_slabs(G, B, s, k, F);
  load_leaf(G, B, s, k, F);
}

// Strip aggregation (eq. (3)) from the staged partner restrictions of r
// (stR, level l at stage row 2^l - 1) and of q (stQ): sm.P[l] = sum(stR) -
// alpha sum(stQ), or sum(stR) with stQ == nullptr.  With r_from_prev the
// partner sums of r are not staged: sm.P still holds them (the previous
// P, by linearity) and becomes sm.P - alpha sum(stQ).  16 groups of threads
// per column (group g adds the partner leaves g, g + 16, ... in that order),
// then across waves; two barriers.  (The single-pass apply and the resident
// solve's iterations add the partner words in this order as they land
// instead of staging them; this form serves the set-up and the squared form.)
template <typename T, int LEV>
__device__ __forceinline__ void prolong_strips(RSmem<T>& sm, const T* stR, const T* stQ, double alpha,
                                               bool r_from_prev = false) {
  const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
  const int c = tid & 31, g = tid >> 5;
  const bool hi = (lane & 32) != 0;
  constexpr int NL = LEV > 0 ? LEV : 1;
  T a[NL], b[NL];
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    const T* vr = stR + (size_t)((1 << l) - 1) * RANK + c;
    a[l] = 0;
    b[l] = 0;
#pragma unroll
    for (int m = 0; m < ((1 << l) + 15) / 16; ++m) {
      const int i = g + 16 * m;
      if (i < (1 << l)) {
        if (!r_from_prev) a[l] += vr[i * RANK];
        if (stQ) b[l] += stQ[(size_t)((1 << l) - 1) * RANK + c + i * RANK];
      }
    }
  }
  // the two 32-lane halves of the wave are folded pairwise (fold_x32)
  T* dR = &sm.redW[wave][c];
  T* dQ = &sm.redW[wave][MAX_LEVELS * RANK + c];
  auto fold_levels = [&](const T* v, T* d) {
#pragma unroll
    for (int l = 0; l + 1 < LEV; l += 2) d[(hi ? l + 1 : l) * RANK] = fold_x32(v[l], v[l + 1]);
    if constexpr (LEV % 2 == 1) {
      const T f = v[LEV - 1] + lane_x32(v[LEV - 1]);
      if (!hi) d[(LEV - 1) * RANK] = f;
    }
  };
  if (!r_from_prev && stQ) {
#pragma unroll
    for (int l = 0; l < LEV; ++l) (hi ? dQ : dR)[l * RANK] = fold_x32(a[l], b[l]);
  } else if (stQ) {
    fold_levels(b, dQ);
  } else if (!r_from_prev) {
    fold_levels(a, dR);
  }
  __syncthreads();
  if (tid < LEV * RANK) {
    T a;
    if (r_from_prev) {
      a = sm.P[tid];
    } else {
      a = sm.redW[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
    }
    if (stQ) {
      T b = sm.redW[0][MAX_LEVELS * RANK + tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) b += sm.redW[w][MAX_LEVELS * RANK + tid];
      a = (T)((double)a - alpha * (double)b);
    }
    sm.P[tid] = a;
  }
  __syncthreads();
}

// Diagonal stage y = U_k t (t, y in LDS): rows rg + 16m (m < 8), dots over 32
// column slots; the eight rows of a lane are folded with a transpose-reduce
// (7 + 2 shuffles).  No barrier.
template <typename T, int LEV>
__device__ __forceinline__ void diag_times(const Resident<T, LEV>& F, const T* t, T* y) {
  const int tid = tid_of<kFresh<T, LEV>>();
  const int cs = tid & 31, rg = tid >> 5;
  const Vec4<T> t4 = lds4(&t[4 * cs]);
  T v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = dot4(F.u[m], t4);
  const bool b4 = (cs & 16) != 0, b3 = (cs & 8) != 0, b2 = (cs & 4) != 0;
  T a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = fold_x16(v[i], v[4 + i]);   // xor 16: the upper four rows if b4
  T bb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {           // xor 8
    const T keep = b3 ? a[2 + i] : a[i], send = b3 ? a[i] : a[2 + i];
    bb[i] = keep + lane_x8(send);
  }
  T kk = b2 ? bb[1] : bb[0];              // bit 2 (lane j pairs with 7 - j)
  kk += lane_m4(b2 ? bb[0] : bb[1]);
  kk = group4_sum(kk);
  if ((cs & 3) == 0) y[rg + 16 * ((b4 ? 4 : 0) + (b3 ? 2 : 0) + (b2 ? 1 : 0))] = kk;
}

// Diagonal stage U_k sm.t into sm.yleaf.  No barrier.
template <typename T, int LEV>
__device__ __forceinline__ void prolong_diag(const Resident<T, LEV>& F, RSmem<T>& sm) {
  diag_times<T, LEV>(F, sm.t, sm.yleaf);
}

// Off-diagonal prolongation sum_l W_l[k] sm.P[l] into sm.yoff (eq. (5)).
// No barrier.
template <typename T, int LEV>
__device__ __forceinline__ void prolong_offdiag(const Resident<T, LEV>& F, RSmem<T>& sm) {
  const int tid = tid_of<kFresh<T, LEV>>();
  if constexpr (LEV > 0) {
    const int cs = tid & 7, row = tid >> 3;
    T o0 = 0, o1 = 0;
#pragma unroll
    for (int l = 0; l < LEV; ++l) {
      const Vec4<T> p4 = lds4(&sm.P[l * RANK + 4 * cs]);
      o0 += dot4(F.w[l][0], p4);
      o1 += dot4(F.w[l][1], p4);
    }
    o0 = group8_sum(o0);
    o1 = group8_sum(o1);
    if (cs == 0) { sm.yoff[row] = o0; sm.yoff[row + 64] = o1; }
  } else {
    if (tid < LEAF) sm.yoff[tid] = 0;
  }
}

}  // namespace hpcg
