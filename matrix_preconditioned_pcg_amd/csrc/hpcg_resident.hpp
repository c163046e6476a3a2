// Register-resident persistent solve for gfx950.
//
// One workgroup of NTR = 512 threads (8 wave64 wavefronts, one workgroup per
// CU, up to 256 VGPRs per lane) owns one leaf of one system for the whole solve:
//   * its factors live in VGPRs: U_k as eight float4 per thread (rows rg + 16m,
//     columns 4cs..4cs+3 with cs = tid % 32, rg = tid / 32) and, per level l,
//     two rows of W_l[k] as float4 (rows tid/8 and tid/8 + 64, columns
//     4(tid % 8)..);
//   * its rows of r, q, z and p and its CSR rows live in LDS, x in registers;
//   * only what other leaves need crosses workgroups: z (the SpMV halo; the
//     halo's p = z + beta p is formed locally, beta being the same in every
//     workgroup), the per-leaf restrictions W_l[k]^T r_k and W_l[k]^T q_k, and
//     the scalar partials.
//
// No barrier inside an iteration.  Each value one workgroup needs from another
// travels as a flagged word (the value's bits and the step it belongs to,
// stored and loaded whole) that the reader polls directly, so a value costs
// one trip through the coherence point instead of a barrier plus a load.  The
// restriction is linear, so W^T r_new = W^T r - alpha W^T q: phase A, which
// owns the whole leaf's q, restricts q right after the SpMV, and phase BC forms
// the partner-half sums of (W^T r - alpha W^T q) and applies M to r_new.
// Every kRefresh iterations W^T r is recomputed exactly from r_new (into the
// other of two buffers) and its partner sums are staged afresh; in between
// they are carried forward by the same linear update.
//   A(it):  poll the halo's z and the system's r.r, r.z partials of step it-1;
//           convergence test on ||r_{it-1}||; beta; p = z + beta p;
//           q = A p (CSR rows, z and p in LDS); publish W_l[k]^T q and the
//           partial p.q; then U_k U_k^T q while those words travel
//   BC(it): poll the partners' W^T q (each thread adding its words per level
//           as they land: nothing is staged) and the p.q partials; alpha;
//           x += alpha p; r -= alpha q; z = U_k U_k^T r_new + sum_l W_l[k] P_l
//           + g r_new with P_l = partner-half sum of (W^T r - alpha W^T q);
//           at a refresh W^T r_new and U_k U_k^T r_new; publish z and the
//           partials r.r and r.z
// Per iteration the factors are never reloaded.
//
// Coherence without cache maintenance.  Every value one workgroup writes for
// another is stored and loaded with agent-scope accesses (sc1: written through
// to, and read from, the point where all XCDs agree), so no L2 write-back or
// invalidation is needed; a value written plainly (a refreshed W^T r) is
// acknowledged by every thread that wrote it, and a workgroup barrier passed,
// before the flagged partial words that announce it are stored (readers load
// it only after seeing those words).  The per-system barrier below remains for
// the set-up and the squared form.
#pragma once
#include "hpcg_kernels.hpp"
#include "hpcg_leaf.hpp"

namespace hpcg {

// Per-system barrier over agent-coherent data (see the header).  `epoch`
// counts this workgroup's barriers.  Arriving waits until this workgroup's
// stores are acknowledged, then stores the count on the workgroup's own
// 128-byte line; waiting polls the lines of the system's K workgroups (one
// wave, a line per lane) until all of them hold it.  No read-modify-write is
// on the path, so a barrier costs one store and one load after the last
// arrival, and the systems of a batch synchronize independently.
__device__ __forceinline__ void cgrid_arrive(const Bufs& B, int item, unsigned& epoch) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  ++epoch;
  if (threadIdx.x == 0) st_c(B.wgflag + (size_t)item * kFlagStride, epoch);
}

__device__ __forceinline__ bool cgrid_wait(const Bufs& B, int s, int K, unsigned epoch) {
  __shared__ int aborted_c;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned* f = B.wgflag + (size_t)s * K * kFlagStride;
    unsigned polls = 0;
    int ab = 0;
    for (;;) {
      int ready = 1;
      for (int j = lane; j < K; j += 64) ready &= (ld_c(f + (size_t)j * kFlagStride) >= epoch) ? 1 : 0;
      if (__all(ready)) break;
      __builtin_amdgcn_s_sleep(1);
      if (((++polls) & 1023u) == 0) {
        if (ld_c(B.abort_flag)) { ab = 1; break; }
        if (polls > (1u << 26)) {
          if (lane == 0) st_c(B.abort_flag, 1);
          ab = 1;
          break;
        }
      }
    }
    if (lane == 0) aborted_c = ab;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return aborted_c != 0;
}

__device__ __forceinline__ bool cgrid_barrier(const Bufs& B, int item, int s, int K, unsigned& epoch) {
  cgrid_arrive(B, item, epoch);
  return cgrid_wait(B, s, K, epoch);
}

// Sum over the workgroup in a fixed order.
template <bool FRESH, typename T>
__device__ __forceinline__ double wg_sum_r(double v, RSmem<T>& sm) {
  v = wave_sum(v);
  const int tid = tid_of<FRESH>();
  if ((tid & 63) == 0) sm.dred[tid >> 6] = v;
  __syncthreads();
  double s = sm.dred[0];
#pragma unroll
  for (int w = 1; w < NWR; ++w) s += sm.dred[w];
  __syncthreads();
  return s;
}

// Two workgroup sums with one pair of barriers.
template <bool FRESH, typename T>
__device__ __forceinline__ void wg_sum2_r(double& a, double& b, RSmem<T>& sm) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int tid = tid_of<FRESH>();
  if ((tid & 63) == 0) {
    sm.dred[tid >> 6] = a;
    sm.dred2[tid >> 6] = b;
  }
  __syncthreads();
  double sa = sm.dred[0], sb = sm.dred2[0];
#pragma unroll
  for (int w = 1; w < NWR; ++w) {
    sa += sm.dred[w];
    sb += sm.dred2[w];
  }
  __syncthreads();
  a = sa;
  b = sb;
}

// Every wave reads the system's K partials and sums them in the same order.
__device__ __forceinline__ double sum_partials_r(const double* part, int s, int K) {
  double v = 0.0;
  const double* p = part + (size_t)s * K;
  for (int j = threadIdx.x & 63; j < K; j += 64) v += ld_c(p + j);
  return wave_sum(v);
}

// Iterations between exact restrictions of r (the others use the linear
// update).  In fp64 each update adds at most the 2^-44 rounding of the
// exchanged W^T q words, relative to alpha W^T q; over 16 updates, in which
// ||r|| falls by far less than 2^20 on these systems, that stays far below
// the fp32 factors' rounding relative to the current r.  fp32 vectors refresh
// every second iteration: one update adds a rounding of the size fp32 vectors
// already carry.
template <typename T>
constexpr int kRefresh = sizeof(T) == 8 ? 16 : 2;

// Restriction of the LDS vector v: U_k^T v into tout (LDS, complete) and
// W_l[k]^T v into pout (global, [levels][K][RANK] of system s; skipped when
// null) and own (LDS).  With part_dst, the workgroup sum of `loc` is stored
// there as well (sharing the restriction's barriers).
template <typename T, int LEV>
__device__ __forceinline__ void r_restrict(const Geom& G, int s, int k, const Resident<T, LEV>& F,
                                           const T* v, T* tout, T* pout, T* own, RSmem<T>& sm,
                                           double loc = 0.0, double* part_dst = nullptr, bool with_u = true) {
  const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
  if (part_dst) {
    loc = wave_sum(loc);
    if (lane == 0) sm.dred[wave] = loc;
  }
  if (with_u) restrict_u_partials<T, LEV>(F, v, sm);
  restrict_w_partials<T, LEV>(F, v, sm);
  __syncthreads();
  if (part_dst && tid == 0) {
    double p = sm.dred[0];
#pragma unroll
    for (int w = 1; w < NWR; ++w) p += sm.dred[w];
    st_c(part_dst, p);
  }
  if (with_u && tid < LEAF) {
    T a = sm.red[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
    tout[tid] = a;
  }
  if constexpr (LEV > 0) {
    if (tid < LEV * RANK) {
      T a = sm.redW[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
      const int l = tid / RANK, c = tid - l * RANK;
      if (pout) st_c(pout + (((size_t)s * G.levels + l) * G.K + k) * RANK + c, a);
      own[tid] = a;
    }
  }
  __syncthreads();
}

// Issue the DMA of the partner halves' per-leaf restrictions of every level
// from src ([B][levels][K][RANK]) into `stage` (level l at row 2^l - 1); the
// caller waits with lds_dma_wait().
template <typename T, int LEV>
__device__ __forceinline__ void r_stage_partners(const Geom& G, const T* src, int s, int k, T* stage) {
  constexpr int CPV = RANK * sizeof(T) / 16;
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    const int kp0 = ((k >> l) ^ 1) << l;
    const T* from = src + (((size_t)s * G.levels + l) * G.K + kp0) * RANK;
    dma_to_lds_n<NWR, CPOL_AGENT, kFreshDma<T, LEV>>(stage + (size_t)((1 << l) - 1) * RANK, (1 << l) * CPV,
                      [&](int c) { return reinterpret_cast<const char*>(from) + 16 * c; });
  }
}

// y = U_k (U_k^T v) with tmp for U_k^T v (all LDS).  y is complete after the
// caller's next barrier.
template <typename T, int LEV>
__device__ __forceinline__ void leaf_apply(const Resident<T, LEV>& F, const T* v, T* tmp, T* y, RSmem<T>& sm) {
  const int tid = tid_of<kFresh<T, LEV>>();
  restrict_u_partials<T, LEV>(F, v, sm);
  __syncthreads();
  if (tid < LEAF) {
    T a = sm.red[0][tid];
#pragma unroll
    for (int w = 1; w < NWR; ++w) a += sm.red[w][tid];
    tmp[tid] = a;
  }
  __syncthreads();
  diag_times<T, LEV>(F, tmp, y);
}

// z = M r_new on the leaf's rows into sm.z.  Needs sm.t (= U_k^T r_new), sm.r
// (= r_new) and the staged partner restrictions of r (stR) and q (stQ):
// P_l = sum(stR) - alpha sum(stQ).  With stQ == nullptr, P_l = sum(stR).
template <typename T, int LEV>
__device__ __forceinline__ void r_prolong(const Resident<T, LEV>& F, RSmem<T>& sm, const T* stR, const T* stQ,
                                          double alpha, float gate) {
  const int tid = tid_of<kFresh<T, LEV>>();
  if constexpr (LEV > 0) prolong_strips<T, LEV>(sm, stR, stQ, alpha);
  if constexpr (LEV == 0) __syncthreads();   // sm.t and sm.r of the caller
  prolong_diag<T, LEV>(F, sm);
  prolong_offdiag<T, LEV>(F, sm);
  __syncthreads();
  if (tid < LEAF) sm.z[tid] = sm.yleaf[tid] + sm.yoff[tid] + (T)gate * sm.r[tid];
  __syncthreads();
}

// Flagged words: a 32-bit word of the value in the low half, the epoch in the
// high half, stored and loaded whole (8-byte agent-scope atomics), so a reader
// that sees the epoch it waits for holds that step's word.  An fp64 value is
// two such words.
__device__ __forceinline__ unsigned long long ll_word(unsigned v, unsigned e) {
  return ((unsigned long long)e << 32) | v;
}
__device__ __forceinline__ bool ll_ready(unsigned long long w, unsigned e) { return (unsigned)(w >> 32) == e; }

template <typename T>
__device__ __forceinline__ void ll_put(unsigned long long* p, T v, unsigned e) {
  if constexpr (sizeof(T) == 4) {
    st_c(p, ll_word(__float_as_uint(v), e));
  } else {
    st_c(p, ll_word((unsigned)__double2loint(v), e));
    st_c(p + 1, ll_word((unsigned)__double2hiint(v), e));
  }
}

// Polls of one flagged word are bounded by B.poll_limit (default 2^22, each
// well under a microsecond): a writer that never comes (an aborted workgroup)
// ends the wait with the abort flag.

// z of global row c (two words apart per row) once it carries epoch e.  The
// polls are pipelined two deep: the next load is in flight while the previous
// one is checked, so a word that lands is seen about half a round trip later.
template <typename T>
__device__ __forceinline__ T ll_get_z(const Bufs& B, int c, unsigned e, int& bad) {
  const unsigned long long* p = B.zll + 2 * (size_t)c;
  unsigned long long a0 = ld_c(p), a1 = (sizeof(T) == 8) ? ld_c(p + 1) : 0ull;
  for (unsigned polls = 0;; ++polls) {
    const unsigned long long b0 = ld_c(p), b1 = (sizeof(T) == 8) ? ld_c(p + 1) : 0ull;
    if constexpr (sizeof(T) == 4) {
      if (ll_ready(a0, e)) return __uint_as_float((unsigned)a0);
    } else {
      if (ll_ready(a0, e) && ll_ready(a1, e)) return __hiloint2double((int)(unsigned)a1, (int)(unsigned)a0);
    }
    if (polls > B.poll_limit || ((polls & 1023u) == 1023u && ld_c(B.abort_flag))) {
      st_c(B.abort_flag, 1);
      bad = 1;
      return T(0);
    }
    a0 = b0;
    a1 = b1;
  }
}

// The system's K flagged r.r and r.z partials of epoch e, summed by one wave in
// the fixed order of sum_partials_r (lane-strided, then the butterfly).
__device__ __forceinline__ void ll_get_partials(const Bufs& B, int s, int K, unsigned e, double& rr, double& rz,
                                                int& bad) {
  const int lane = threadIdx.x & 63;
  double a = 0.0, b = 0.0;
  for (int j = lane; j < K; j += 64) {
    const unsigned long long* p = B.pll + ((size_t)s * K + j) * 4;
    // pipelined two deep, as in ll_get_z
    unsigned long long w0 = ld_c(p), w1 = ld_c(p + 1), w2 = ld_c(p + 2), w3 = ld_c(p + 3);
    for (unsigned polls = 0;; ++polls) {
      const unsigned long long n0 = ld_c(p), n1 = ld_c(p + 1), n2 = ld_c(p + 2), n3 = ld_c(p + 3);
      if (ll_ready(w0, e) && ll_ready(w1, e) && ll_ready(w2, e) && ll_ready(w3, e)) {
        a += __hiloint2double((int)(unsigned)w1, (int)(unsigned)w0);
        b += __hiloint2double((int)(unsigned)w3, (int)(unsigned)w2);
        break;
      }
      if (polls > B.poll_limit || ((polls & 1023u) == 1023u && ld_c(B.abort_flag))) {
        st_c(B.abort_flag, 1);
        bad = 1;
        break;
      }
      w0 = n0; w1 = n1; w2 = n2; w3 = n3;
    }
  }
  rr = wave_sum(a);
  rz = wave_sum(b);
}

// A restriction value of W^T q as one flagged word.  fp32: the value's bits
// and the 32-bit epoch.  fp64: the value with its eight lowest mantissa bits
// replaced by an 8-bit step tag (1 .. 255, never 0 = cleared); the 44 bits
// left keep it within 2^-44 relative, far inside the fp32 factors' rounding.
// The tag is unambiguous because the words are cleared at every solve and a
// buffer (one per step parity) is rewritten only two steps later.
template <typename T>
__device__ __forceinline__ unsigned long long q_word(T v, unsigned tag, unsigned e) {
  if constexpr (sizeof(T) == 4) return ll_word(__float_as_uint(v), e);
  else return ((unsigned long long)__double_as_longlong(v) & ~0xFFull) | tag;
}
template <typename T>
__device__ __forceinline__ bool q_ready(unsigned long long w, unsigned tag, unsigned e) {
  if constexpr (sizeof(T) == 4) return ll_ready(w, e);
  else return (unsigned)(w & 0xFFull) == tag;
}
template <typename T>
__device__ __forceinline__ T q_value(unsigned long long w) {
  if constexpr (sizeof(T) == 4) return __uint_as_float((unsigned)w);
  else return __longlong_as_double((long long)(w & ~0xFFull));
}
__device__ __forceinline__ unsigned q_tag(int it) { return 1u + (unsigned)(it % 255); }

// Restriction of q for the partners, published as flagged words: W_l[k]^T q
// of step it into qll (parity par) and the workgroup's partial p.q (`loc`
// summed over the threads) into pqll.
template <typename T, int LEV>
__device__ __forceinline__ void r_restrict_q_ll(const Geom& G, const Bufs& B, int s, int k, int item,
                                                const Resident<T, LEV>& F, RSmem<T>& sm, double loc, int par,
                                                unsigned tag, unsigned e) {
  const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
  loc = wave_sum(loc);
  if (lane == 0) sm.dred[wave] = loc;
  restrict_w_partials<T, LEV>(F, sm.q, sm);
  __syncthreads();
  if (tid == 0) {
    double p = sm.dred[0];
#pragma unroll
    for (int w = 1; w < NWR; ++w) p += sm.dred[w];
    ll_put<double>(B.pqll + ((size_t)par * G.B * G.K + item) * 2, p, e);
  }
  if constexpr (LEV > 0) {
    if (tid < LEV * RANK) {
      T a = sm.redW[0][tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
      const int l = tid / RANK, c = tid - l * RANK;
      const size_t half = (size_t)G.B * G.levels * G.K * RANK;
      st_c(B.qll + par * half + (((size_t)s * G.levels + l) * G.K + k) * RANK + c, q_word<T>(a, tag, e));
    }
  }
  __syncthreads();
}

// The last wave's first thread (it holds the p.q partials' sum).
constexpr int NST = NTR - 64;

// The system's K flagged p.q partials of epoch e (parity par), summed by one
// wave in the fixed order of sum_partials_r.
__device__ __forceinline__ double ll_get_pq(const Bufs& B, int s, int K, size_t BK, int par, unsigned e, int& bad) {
  const int lane = threadIdx.x & 63;
  double a = 0.0;
  for (int j = lane; j < K; j += 64) {
    const unsigned long long* p = B.pqll + ((size_t)par * BK + (size_t)s * K + j) * 2;
    // pipelined two deep, as in ll_get_z
    unsigned long long w0 = ld_c(p), w1 = ld_c(p + 1);
    for (unsigned polls = 0;; ++polls) {
      const unsigned long long n0 = ld_c(p), n1 = ld_c(p + 1);
      if (ll_ready(w0, e) && ll_ready(w1, e)) {
        a += __hiloint2double((int)(unsigned)w1, (int)(unsigned)w0);
        break;
      }
      if (polls > B.poll_limit || ((polls & 1023u) == 1023u && ld_c(B.abort_flag))) {
        st_c(B.abort_flag, 1);
        bad = 1;
        break;
      }
      w0 = n0;
      w1 = n1;
    }
  }
  return wave_sum(a);
}

// Phase BC's poll of the partners' W^T q words, summed as they land.  Thread
// (column c = tid % 32, group g = tid / 32 of 16) polls, for every level l,
// the words of the partner half's leaves g, g + 16, ... and adds them in that
// order; the two groups of a wave are folded, and the wave's partial of each
// (level, column) goes to sm.redW[wave][MAX_LEVELS * RANK + l * RANK + c]:
// the values, slots and order in which prolong_strips sums staged words, so
// the partner sums are bitwise the same, without staging the words in LDS
// and reading them back.  Every word is loaded at once and the late ones
// re-polled together.  The last wave also polls the system's p.q partials and
// sums them in the order of ll_get_pq into sm.dsc[3].  No barrier.
template <int LEV>
constexpr int q_slot0(int l) {
  int n = 0;
  for (int i = 0; i < l; ++i) n += ((1 << i) + 15) / 16;
  return n;
}

template <typename T, int LEV>
__device__ __forceinline__ void ll_q_strips(const Geom& G, const Bufs& B, int s, int k, int par, unsigned tag,
                                            unsigned e, size_t BK, RSmem<T>& sm, int& bad) {
  static_assert(LEV > 0, "levels only");
  constexpr int NS = q_slot0<LEV>(LEV);
  static_assert(NS <= 32, "poll mask");
  const int tid = tid_of<kFresh<T, LEV>>(), lane = tid & 63, wave = tid >> 6;
  const int c = tid & 31, g = tid >> 5;
  const bool hi = (lane & 32) != 0;
  const unsigned long long* base =
      B.qll + (size_t)par * G.B * G.levels * G.K * RANK + (size_t)s * G.levels * G.K * RANK;
  auto addr = [&](int l, int i) { return base + ((size_t)l * G.K + (((k >> l) ^ 1) << l) + i) * RANK + c; };
  unsigned long long v[NS];
  unsigned pending = 0;
#pragma unroll
  for (int l = 0; l < LEV; ++l)
#pragma unroll
    for (int m = 0; m < ((1 << l) + 15) / 16; ++m) {
      const int i = g + 16 * m, j = q_slot0<LEV>(l) + m;
      if (i < (1 << l)) {
        v[j] = ld_c(addr(l, i));
        pending |= 1u << j;
      }
    }
  // the last wave: the p.q partial of leaf j = lane (and lane + 64) as its two
  // words.  From seven levels on (where registers run short) they take the
  // slots of levels 0 .. 3, which that wave's groups (14 and 15) never fill
  const bool pqw = wave == NWR - 1;
  const unsigned long long* pq = B.pqll + ((size_t)par * BK + (size_t)s * G.K) * 2;
  constexpr bool PQ_IN_SLOTS = LEV >= 7;
  unsigned long long wx[4];
  auto pw = [&](int i) -> unsigned long long& {
    if constexpr (PQ_IN_SLOTS) return v[i];
    else return wx[i];
  };
  unsigned long long& w0 = pw(0);
  unsigned long long& w1 = pw(1);
  unsigned long long& w2 = pw(2);
  unsigned long long& w3 = pw(3);
  unsigned ppend = 0;
  if (pqw) {
    if (lane < G.K) { w0 = ld_c(pq + 2 * lane); w1 = ld_c(pq + 2 * lane + 1); ppend |= 1u; }
    if (lane + 64 < G.K) { w2 = ld_c(pq + 2 * lane + 128); w3 = ld_c(pq + 2 * lane + 129); ppend |= 2u; }
  }
  for (unsigned polls = 0;; ++polls) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if ((pending & (1u << j)) && q_ready<T>(v[j], tag, e)) pending &= ~(1u << j);
    if ((ppend & 1u) && ll_ready(w0, e) && ll_ready(w1, e)) ppend &= ~1u;
    if ((ppend & 2u) && ll_ready(w2, e) && ll_ready(w3, e)) ppend &= ~2u;
    if (!pending && !ppend) break;
    if (polls > B.poll_limit || ((polls & 1023u) == 1023u && ld_c(B.abort_flag))) {
      st_c(B.abort_flag, 1);
      bad = 1;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int l = 0; l < LEV; ++l)
#pragma unroll
      for (int m = 0; m < ((1 << l) + 15) / 16; ++m) {
        const int j = q_slot0<LEV>(l) + m;
        if (pending & (1u << j)) v[j] = ld_c(addr(l, g + 16 * m));
      }
    if (ppend & 1u) { w0 = ld_c(pq + 2 * lane); w1 = ld_c(pq + 2 * lane + 1); }
    if (ppend & 2u) { w2 = ld_c(pq + 2 * lane + 128); w3 = ld_c(pq + 2 * lane + 129); }
  }
  T b[LEV];
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    b[l] = 0;
#pragma unroll
    for (int m = 0; m < ((1 << l) + 15) / 16; ++m)
      if (g + 16 * m < (1 << l)) b[l] += q_value<T>(v[q_slot0<LEV>(l) + m]);
  }
  T* dQ = &sm.redW[wave][MAX_LEVELS * RANK + c];
#pragma unroll
  for (int l = 0; l + 1 < LEV; l += 2) dQ[(hi ? l + 1 : l) * RANK] = fold_x32(b[l], b[l + 1]);
  if constexpr (LEV % 2 == 1) {
    const T f = b[LEV - 1] + lane_x32(b[LEV - 1]);
    if (!hi) dQ[(LEV - 1) * RANK] = f;
  }
  if (pqw) {
    double a = 0.0;
    if (lane < G.K) a += __hiloint2double((int)(unsigned)w1, (int)(unsigned)w0);
    if (lane + 64 < G.K) a += __hiloint2double((int)(unsigned)w3, (int)(unsigned)w2);
    for (int j = lane + 128; j < G.K && !bad; j += 64) {   // systems of more than 128 leaves
      const unsigned long long* p = pq + 2 * j;
      for (unsigned polls = 0;; ++polls) {
        const unsigned long long x0 = ld_c(p), x1 = ld_c(p + 1);
        if (ll_ready(x0, e) && ll_ready(x1, e)) {
          a += __hiloint2double((int)(unsigned)x1, (int)(unsigned)x0);
          break;
        }
        if (polls > B.poll_limit || ((polls & 1023u) == 1023u && ld_c(B.abort_flag))) {
          st_c(B.abort_flag, 1);
          bad = 1;
          break;
        }
      }
    }
    const double sum = wave_sum(a);
    if (lane == 0) sm.dsc[3] = sum;
  }
}

// z = M r_new on the leaf's rows into sm.z after ll_q_strips: the waves'
// partials of the partner sums of W^T q are in sm.redW; with r_from_prev the
// partner sums of W^T r are the previous sm.P, else they are summed from the
// staged words stR here (prolong_strips' order).  P_l = (sum of W^T r) - alpha
// (sum of W^T q); then z = (sm.yr - alpha sm.yq) + sum_l W_l[k] P_l + g r_new
// (U_k U_k^T r_new by the linear update of the leaf stage).
template <typename T, int LEV>
__device__ __forceinline__ void r_prolong_split_q(const Resident<T, LEV>& F, RSmem<T>& sm, const T* stR,
                                                  double alpha, float gate, bool r_from_prev) {
  const int tid = tid_of<kFresh<T, LEV>>();
  if constexpr (LEV > 0) {
    if (!r_from_prev) {
      const int lane = tid & 63, wave = tid >> 6, c = tid & 31, g = tid >> 5;
      const bool hi = (lane & 32) != 0;
      T a[LEV];
#pragma unroll
      for (int l = 0; l < LEV; ++l) {
        const T* vr = stR + (size_t)((1 << l) - 1) * RANK + c;
        a[l] = 0;
#pragma unroll
        for (int m = 0; m < ((1 << l) + 15) / 16; ++m)
          if (g + 16 * m < (1 << l)) a[l] += vr[(g + 16 * m) * RANK];
      }
      T* dR = &sm.redW[wave][c];
#pragma unroll
      for (int l = 0; l + 1 < LEV; l += 2) dR[(hi ? l + 1 : l) * RANK] = fold_x32(a[l], a[l + 1]);
      if constexpr (LEV % 2 == 1) {
        const T f = a[LEV - 1] + lane_x32(a[LEV - 1]);
        if (!hi) dR[(LEV - 1) * RANK] = f;
      }
      __syncthreads();
    }
    if (tid < LEV * RANK) {
      T a;
      if (r_from_prev) {
        a = sm.P[tid];
      } else {
        a = sm.redW[0][tid];
#pragma unroll
        for (int w = 1; w < NWR; ++w) a += sm.redW[w][tid];
      }
      T b = sm.redW[0][MAX_LEVELS * RANK + tid];
#pragma unroll
      for (int w = 1; w < NWR; ++w) b += sm.redW[w][MAX_LEVELS * RANK + tid];
      sm.P[tid] = (T)((double)a - alpha * (double)b);
    }
    __syncthreads();
  }
  prolong_offdiag<T, LEV>(F, sm);
  __syncthreads();
  if (tid < LEAF)
    sm.z[tid] = (T)((double)sm.yr[tid] - alpha * (double)sm.yq[tid]) + sm.yoff[tid] + (T)gate * sm.r[tid];
  __syncthreads();
}

// The grid covers systems s0 .. s0 + gridDim.x / K - 1 (a batch with more
// leaves than CUs is solved in groups of whole systems, one launch each).
//
// An iteration has no barrier.  Phase A needs only the neighbours' new z and
// the partials r.r and r.z, phase BC only the partners' W^T q and the partials
// p.q (and, after a refresh, W^T r): all of it travels as flagged words that
// the readers poll directly.  A workgroup can run at most one phase ahead of
// the slowest of its system (each phase needs every workgroup's partial of the
// previous one), so the phase A outputs are double-buffered by step parity.
// Every workgroup of a system computes the same sums in the same order, so
// they all take the same convergence decision and leave the loop together.
// FM selects the preconditioner form: FM_DIRECT (M = H), FM_SQUARED (M = H H)
// or FM_JACOBI (M = diag(A)^-1: no factors, no restrictions, only the SpMV
// halo and the partials cross workgroups; instantiated with LEV = 0).
constexpr int FM_DIRECT = 0, FM_SQUARED = 1, FM_JACOBI = 2;
template <typename T, int LEV, int FM>
__global__ __launch_bounds__(NTR) void k_resident(Geom G, Bufs B, int max_leaf_nnz, int max_halo, int s0) {
  constexpr bool SQ = (FM == FM_SQUARED), JAC = (FM == FM_JACOBI);
  static_assert(!JAC || LEV == 0, "the Jacobi form has no levels");
  __shared__ RSmem<T> sm;
  extern __shared__ int4 rdyn4[];
  int* colL = reinterpret_cast<int*>(rdyn4);              // leaf-local columns (own, then halo)
  float* valL = reinterpret_cast<float*>(colL + max_leaf_nnz);
  int* rpL = reinterpret_cast<int*>(valL + max_leaf_nnz);
  const int stage_rows = partner_rows(G);
  T* stR = reinterpret_cast<T*>(rdyn4 + (2 * max_leaf_nnz + LEAF + 1 + 3) / 4);
  // z and p of the previous step by leaf-local column: own rows, then the halo
  T* zc = stR + (size_t)stage_rows * RANK;
  T* pc = zc + LEAF + max_halo;
  int* hcolL = reinterpret_cast<int*>(pc + LEAF + max_halo);   // halo global columns
  const int tid = threadIdx.x;
  const int item = s0 * G.K + blockIdx.x;
  const int s = item / G.K, k = item - s * G.K;
  const int leaf0 = s * G.n + k * LEAF;
  SysState* st = B.st + s;
  const bool lead = (tid == 0 && k == 0);
  // W^T r in two halves of pleaf (ping-pong at refreshes); W^T q and the p.q
  // partials are flagged words (qll, pqll) by step parity
  const size_t half = (size_t)G.B * G.levels * G.K * RANK;
  T* pR[2] = {reinterpret_cast<T*>(B.pleaf), reinterpret_cast<T*>(B.pleaf) + half};
  T* pW = reinterpret_cast<T*>(B.tleaf);   // squared form: W^T w of w = H r
  const size_t BK = (size_t)G.B * G.K;
  int rbuf = 0;

  // ---- factors into registers, CSR rows and the halo list into LDS ----
  Resident<T, LEV> F;
  if constexpr (!JAC) load_factors(G, B, s, k, F);
  const int e_begin = B.row_ptr[leaf0];
  if (tid <= LEAF) rpL[tid] = B.row_ptr[leaf0 + tid] - e_begin;
  const int leaf_nnz = B.row_ptr[leaf0 + LEAF] - e_begin;
  for (int e = tid; e < leaf_nnz; e += NTR) {
    colL[e] = B.lcol[e_begin + e];
    valL[e] = B.val[e_begin + e];
  }
  const int h0 = B.hoff[item], nh = B.hoff[item + 1] - h0;
  for (int h = tid; h < nh; h += NTR) hcolL[h] = B.hcol[h0 + h];
  const float gate = (!JAC && tid < LEAF) ? B.g[leaf0 + tid] : 0.f;
  const double dinv = (JAC && tid < LEAF) ? B.dinv[leaf0 + tid] : 0.0;   // Jacobi: 1 / A_ii
  double x = 0.0;                      // x of row tid (tid < LEAF)
  unsigned epoch = 0;                  // barriers passed

  // Squared form M = H H: with w = H r in sm.z, z = H w into sm.z.  The
  // slabs' restriction of w is new data, so it costs one more exchange among
  // the system's workgroups; U_k U_k^T w overlaps its wait.  sm.P (the partner
  // sums of W^T r, carried to the next iteration) is kept aside meanwhile.
  auto squared = [&]() -> bool {
    if constexpr (!SQ) return true;
    if (tid < LEAF) sm.t[tid] = sm.z[tid];
    __syncthreads();
    r_restrict<T, LEV>(G, s, k, F, sm.t, sm.tq, pW, sm.ownQ, sm, 0.0, nullptr, false);
    cgrid_arrive(B, item, epoch);
    leaf_apply<T, LEV>(F, sm.t, sm.tq, sm.yleaf, sm);
    if (cgrid_wait(B, s, G.K, epoch)) return false;
    if constexpr (LEV > 0) {
      r_stage_partners<T, LEV>(G, pW, s, k, stR);
      if (tid < LEV * RANK) sm.ownR[tid] = sm.P[tid];
    }
    lds_dma_wait();
    if constexpr (LEV > 0) prolong_strips<T, LEV>(sm, stR, (const T*)nullptr, 0.0, false);
    prolong_offdiag<T, LEV>(F, sm);
    __syncthreads();
    if (tid < LEAF) sm.z[tid] = sm.yleaf[tid] + sm.yoff[tid] + (T)gate * sm.t[tid];
    if constexpr (LEV > 0) {
      if (tid < LEV * RANK) sm.P[tid] = sm.ownR[tid];
    }
    __syncthreads();
    return true;
  };

  // z (sm.z) and the partials r.r (given) and r.z of step i as flagged words
  // of epoch ep_base + i: everything the next phase A reads from this leaf.
  auto publish = [&](double loc_rr, int i) {
    const unsigned e = B.ep_base + (unsigned)i;
    // this workgroup's earlier stores (W^T r of a refresh) are acknowledged
    // first, by every thread, and the barrier inside wg_sum2_r separates that
    // from the partial words below: whoever sees those words sees W^T r too
    __builtin_amdgcn_s_waitcnt(0);
    double loc_rz = 0.0;
    if (tid < LEAF) {
      ll_put<T>(B.zll + 2 * (size_t)(leaf0 + tid), sm.z[tid], e);
      loc_rz = (double)sm.r[tid] * (double)sm.z[tid];
    }
    wg_sum2_r<kFresh<T, LEV>>(loc_rr, loc_rz, sm);
    if (tid == 0) {
      ll_put<double>(B.pll + (size_t)item * 4, loc_rr, e);
      ll_put<double>(B.pll + (size_t)item * 4 + 2, loc_rz, e);
    }
  };

  // ---- r = b, its restriction (t_r, W^T r), ||b||^2 ----
  double loc = 0.0;
  if (tid < LEAF) {
    const T bv = (T)B.b[leaf0 + tid];
    sm.r[tid] = bv;
    loc = (double)bv * (double)bv;
  }
  __syncthreads();
  if constexpr (!JAC) {
    r_restrict<T, LEV>(G, s, k, F, sm.r, sm.tr, pR[0], sm.ownR, sm);
    diag_times<T, LEV>(F, sm.tr, sm.yr);     // U_k U_k^T r0 (read in the first phase BC)
  }
  const double part_bb = wg_sum_r<kFresh<T, LEV>>(loc, sm);
  if (tid == 0) {
    st_c(B.rr_part + item, part_bb);
    if (k == 0) {
      st->relres = 1.0;
      st->brk = 0;
      st->brk_it = 0;
      set_state(st, ST_RUNNING, 0);
    }
  }
  if (cgrid_barrier(B, item, s, G.K, epoch)) return;

  // ---- z0 = M r0, published with r.z0 (no barrier: phase A polls for them) ----
  double bnorm = 1.0, rz_old = 1.0;
  {
    if constexpr (LEV > 0) r_stage_partners<T, LEV>(G, pR[0], s, k, stR);
    const double rr = sum_partials_r(B.rr_part, s, G.K);
    lds_dma_wait();
    bnorm = sqrt(rr);
    if (rr == 0.0) {                   // b = 0: x = 0 at step 0 (every workgroup sees rr = 0)
      if (lead) { st->bnorm = 0.0; st->relres = 0.0; set_state(st, ST_CONVERGED, 0); }
      if (tid < LEAF) B.x[leaf0 + tid] = 0.0;
      return;
    }
    if (lead) st->bnorm = bnorm;
    if constexpr (JAC) {
      if (tid < LEAF) sm.z[tid] = (T)(dinv * (double)sm.r[tid]);
    } else {
      if (tid < LEAF) sm.t[tid] = sm.tr[tid];
      __syncthreads();
      r_prolong<T, LEV>(F, sm, stR, (const T*)nullptr, 0.0, gate);
    }
    if constexpr (SQ) {
      if (!squared()) return;
    }
    publish(loc, 0);
  }

  double pend_rel = 0.0;
  // timeline build: stamps of one iteration (empty otherwise)
  constexpr int kTraceIt = 66;   // a plain iteration: no exact refresh, no restaging of W^T r
  auto stamp_it = [&](int it, int slot) {
    if (it == kTraceIt) stamp(blockIdx.x, slot);
  };
  for (int it = 1; it <= B.maxit + 2; ++it) {
    const unsigned ez = B.ep_base + (unsigned)(it - 1);   // epoch of z and the partials of step it-1
    stamp_it(it, 0);
    // ---------------- phase A (it) ----------------
    {
      const bool first = (it == 1);
      // the halo's z (flagged words) into LDS; wave 0 also collects the
      // partials r.r and r.z.  The halo's p is not read from its owners: every
      // workgroup of a system computes the same beta, so the copy of the
      // halo's p that this workgroup keeps in pc (updated below with the
      // owners' own formula) equals theirs bit for bit
      int bad = 0;
      for (int h = tid; h < nh; h += NTR) zc[LEAF + h] = ll_get_z<T>(B, hcolL[h], ez, bad);
      if (tid < LEAF) {
        zc[tid] = sm.z[tid];
        pc[tid] = sm.p[tid];
      }
      if (tid < 64) {
        double rr, rz;
        ll_get_partials(B, s, G.K, ez, rr, rz, bad);
        if (tid == 0) {
          sm.dsc[1] = rr;
          sm.dsc[2] = rz;
        }
      }
      if (__syncthreads_or(bad)) return;   // a bounded poll ran out: the abort flag is set
      stamp_it(it, 1);
      const double rr = sm.dsc[1], rz = sm.dsc[2];
      int fin = ST_RUNNING, fin_it = 0;
      if (it >= 2) {
        const double rel = sqrt(rr) / bnorm;
        pend_rel = rel;
        if (rel <= B.tol) { fin = ST_CONVERGED; fin_it = it - 1; }
        else if (it - 1 >= B.maxit) { fin = ST_NOT_CONVERGED; fin_it = B.maxit; }
      }
      if (fin == ST_RUNNING && (!(rz > 0.0) || !isfinite(rz))) { fin = ST_BREAKDOWN; fin_it = it - 1; }
      if (fin != ST_RUNNING) {
        if (lead) {
          st->relres = pend_rel;
          set_state(st, fin, fin_it);
        }
        break;
      }
      const double beta = first ? 0.0 : rz / rz_old;
      rz_old = rz;
      // SpMV: 4 threads per row, CSR rows from LDS, own columns from sm.z / sm.p,
      // halo columns from hz / hp; p = z + beta p formed on the fly
      const int row = tid >> 2, lr = tid & 3;
      const int e0 = rpL[row], e1 = rpL[row + 1];
      T acc = 0;
      for (int e = e0 + lr; e < e1; e += 4) {
        const int c = colL[e];
        acc = fma((T)valL[e], first ? zc[c] : pdir<T>(zc[c], pc[c], beta), acc);
      }
      acc = group4_sum(acc);
      T pn = 0;
      loc = 0.0;
      if (lr == 0) {
        pn = first ? sm.z[row] : pdir<T>(sm.z[row], sm.p[row], beta);
        sm.q[row] = acc;
        loc = (double)pn * (double)acc;
      }
      __syncthreads();                  // every SpMV read of sm.p and pc is done
      stamp_it(it, 2);
      if (lr == 0) sm.p[row] = pn;
      for (int h = tid; h < nh; h += NTR)
        pc[LEAF + h] = first ? zc[LEAF + h] : pdir<T>(zc[LEAF + h], pc[LEAF + h], beta);
      // the slab restriction of q and the partial p.q, published as flagged
      // words (what the partners read)
      r_restrict_q_ll<T, LEV>(G, B, s, k, item, F, sm, loc, it & 1, q_tag(it), B.ep_base + (unsigned)it);
      stamp_it(it, 3);
    }
    // U_k U_k^T q is this workgroup's alone: it overlaps the partners' words
    // in flight
    if constexpr (!JAC) leaf_apply<T, LEV>(F, sm.q, sm.tq, sm.yq, sm);
    stamp_it(it, 4);
    // ---------------- phase BC (it) ----------------
    double alpha = 0.0;
    {
      // The partner sums of W^T r are staged only after an exact refresh (and
      // for the initial r); otherwise they are the previous P (linearity).
      const bool r_from_prev = (it - 1) % kRefresh<T> != 0;
      if constexpr (LEV > 0) {
        if (!r_from_prev) r_stage_partners<T, LEV>(G, pR[rbuf], s, k, stR);
      }
      int bad = 0;
      if constexpr (LEV > 0) {
        ll_q_strips<T, LEV>(G, B, s, k, it & 1, q_tag(it), B.ep_base + (unsigned)it, BK, sm, bad);
      } else if (tid >= NST) {
        const double pqs = ll_get_pq(B, s, G.K, BK, it & 1, B.ep_base + (unsigned)it, bad);
        if (tid == NST) sm.dsc[3] = pqs;
      }
      __builtin_amdgcn_s_waitcnt(0);    // the W^T r stage has landed
      if (__syncthreads_or(bad)) return;
      stamp_it(it, 5);
      const double pq = sm.dsc[3];
      if (!(pq > 0.0) || !isfinite(pq)) {   // every workgroup of the system sees the same pq
        if (lead) set_state(st, ST_BREAKDOWN, it);
        break;
      }
      alpha = rz_old / pq;
      double loc_rr = 0.0;
      if (tid < LEAF) {
        const T rn = (T)((double)sm.r[tid] - alpha * (double)sm.q[tid]);
        sm.r[tid] = rn;
        x += alpha * (double)sm.p[tid];
        loc_rr = (double)rn * (double)rn;
      }
      if constexpr (JAC) {
        if (tid < LEAF) sm.z[tid] = (T)(dinv * (double)sm.r[tid]);
      } else {
        // (r_prolong_split_q synchronizes before it reads sm.r)
        r_prolong_split_q<T, LEV>(F, sm, stR, alpha, gate, r_from_prev);
      }
      stamp_it(it, 6);
      if constexpr (SQ) {
        if (!squared()) return;
      }
      // exact restriction every kRefresh steps, before z is published (the
      // partners' next phase BC reads it once they hold this step's words);
      // else the same linear update the partners use (its rounding drift is
      // bounded by the refreshes)
      const bool refresh = !JAC && (it % kRefresh<T> == 0);
      if (refresh) {
        // exact W^T r (into the other buffer: slow partners may still be
        // staging the previous one) and U U^T r
        rbuf ^= 1;
        r_restrict<T, LEV>(G, s, k, F, sm.r, sm.tr, pR[rbuf], sm.ownR, sm);
        diag_times<T, LEV>(F, sm.tr, sm.yr);
      }
      stamp_it(it, 7);
      publish(loc_rr, it);
      stamp_it(it, 8);
      if (!JAC && !refresh && tid < LEAF) sm.yr[tid] = (T)((double)sm.yr[tid] - alpha * (double)sm.yq[tid]);
    }
  }
  // ---- the solution of the leaf's rows ----
  if (tid < LEAF) B.x[leaf0 + tid] = x;
}

}  // namespace hpcg
