// Device-side building blocks of the H-matrix-preconditioned CG solve on gfx950.
//
// Work decomposition.  Every system's n rows are cut into leaves of LEAF = 128
// rows, and every leaf is served by `bpl` workgroups of NT = 256 threads (four
// wave64 wavefronts).  Workgroup j of leaf k
//   * restricts by columns: with the column slice U_k[:, C_j] (C_j = columns
//     [j*CW, (j+1)*CW), CW = LEAF/bpl) it forms the slice t_j = U_k[:, C_j]^T r_k
//     and at once the slot's share U_k[:, C_j] t_j of the diagonal-block product
//     U_k U_k^T r_k = sum_j U_k[:, C_j] t_j, so each U_k byte is read once per
//     apply; it also forms the complete per-leaf restriction W_l[k]^T r_k of the
//     levels l with l % bpl == j;
//   * prolongs and does the vector work by rows: rows [j*RB, (j+1)*RB) of the
//     leaf, RB = LEAF/bpl, adding the bpl diagonal-block shares in slot order.
//
// One PCG iteration is three phases with a device-wide dependency between them
// ("Hierarchical Transformer Preconditioning for Interactive Physics
// Simulation", section 5: apply, SpMV, SAXPYs and dot reductions form the whole
// inner loop):
//   A  beta = (r.z)/(r.z)_old;  p = z + beta p;  q = A p;  partial p.q
//   B  alpha = (r.z)/(p.q);  x += alpha p;  r -= alpha q;  partial r.r;
//      diagonal stage U_k U_k^T r_k by column slices and the restriction of the
//      new r (eq. (2)), W_l[k]^T r_k
//   C  convergence test on r.r;  strip aggregation over the partner half of
//      every level (eq. (3)), then z_k = (diagonal shares) + sum_l W_l[k] P_l
//      + g r_k (eqs. (4)-(5) with the coupling core equal to the identity);
//      partial r.z
//
// Memory traffic.  Each phase issues all of its loads in one batch: the factor
// rows it needs go straight from global memory into LDS with gfx950's
// global_load_lds_dwordx4 (no register staging), next to the scalar partials
// and vector slices, so a phase costs about one memory round trip.
//
// Precision.  Factors and matrix values are fp32 (the bytes that bound the
// apply).  The vector type T is a template parameter: T = float is the pages'
// split (fp32 vectors and apply arithmetic, fp64 scalars; Supplementary
// section 7), T = double carries r, z, p, q, the restriction results and all
// accumulations in fp64.  Scalars and x are fp64 in both.  Every sum of
// partials is evaluated in one fixed order wherever it is needed, so all
// workgroups agree bit for bit and a solve is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hpcg {

constexpr int LEAF = 128;
constexpr int RANK = 32;
constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr int MAX_LEVELS = 8;      // K <= 256 leaves per system

// In-kernel timeline, compiled in only with HPCG_TRACE (a separate build of
// the library): stamp(wg, slot) records thread 0's reading of the constant
// 100 MHz real-time counter into trace_table[wg][slot]; hpcg_trace_read copies
// the table to the host.  In the ordinary build stamp() is empty.
constexpr int kTraceSlots = 16;
constexpr int kTraceItems = 4096;
#ifdef HPCG_TRACE
__device__ unsigned long long trace_table[kTraceItems * kTraceSlots];
__device__ __forceinline__ void stamp(int wg, int slot) {
  if (threadIdx.x == 0 && wg < kTraceItems)
    trace_table[wg * kTraceSlots + slot] = __builtin_amdgcn_s_memrealtime();
}
// a plain value in place of a time (a workgroup's role, say)
__device__ __forceinline__ void stamp_value(int wg, int slot, unsigned long long v) {
  if (threadIdx.x == 0 && wg < kTraceItems) trace_table[wg * kTraceSlots + slot] = v;
}
#else
__device__ __forceinline__ void stamp(int, int) {}
__device__ __forceinline__ void stamp_value(int, int, unsigned long long) {}
#endif

enum : int { ST_RUNNING = 0, ST_CONVERGED = 1, ST_NOT_CONVERGED = 2, ST_BREAKDOWN = 3 };

// Preconditioner forms: M = H (the H-matrix itself), M = H H, M = diag(A)^-1.
enum : int { FORM_DIRECT = 0, FORM_SQUARED = 1, FORM_JACOBI = 2 };

// `status` changes only in phase C (and at init): a breakdown found in phase A
// or B is parked in `brk`/`brk_it` and turned into a status by the next phase C.
// A breakdown is parked only when the scalar that every workgroup of the system
// computes identically is bad, so within a phase every workgroup reaches the
// same decision, and every status read after a phase-C boundary is final.
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
  int bpl;       // workgroups per leaf
  int RB;        // rows per workgroup (LEAF / bpl), also the column-slice width CW
  int nblk_sys;  // K * bpl
  int nblk;      // B * nblk_sys
};

// Device buffers.  Vector and restriction buffers are sized for double; with
// T = float only the first half of each is used.
struct Bufs {
  const int* row_ptr;
  const int* col;
  const float* val;
  const float* U;      // [B][K][LEAF][LEAF]
  const float* W;      // [B][levels][K][LEAF][RANK]
  const float* g;      // [B*n]
  const float* b;      // [B*n]
  void* r;             // [2][B*n]: r of even and odd iterations
  void* z;
  void* q;
  void* p0;
  void* p1;
  double* x;
  void* tleaf;         // [B][K][bpl][LEAF]   diagonal-block shares U_k[:, C_j] U_k[:, C_j]^T r_k
  void* pleaf;         // [B][levels][K][RANK] W_l[k]^T r_k
  double* pq_part;     // [nblk]
  double* rr_part;
  double* rz_part;
  SysState* st;        // [B]
  unsigned* barrier;   // device-wide barrier arrival counter
  unsigned* wgflag;    // resident engine: per-workgroup barrier counts, one 128-byte line each
  unsigned long long* llw;  // fused apply: [B][levels][K][RANK] W_l[k]^T r as (value, epoch) words
  unsigned* lle;       // fused apply: [B*K] calls completed per leaf (the epoch)
  unsigned long long* lly;  // split apply: [B*K][LEAF] U_k U_k^T r as (value, epoch) words
  const float* Ub;     // bridge format: [B][K][LEAF][RANK] U~_k
  const float* Vb;     // bridge format: [B][K][LEAF][RANK] V~_k
  const float* Bc;     // bridge format: [B][ncores][RANK][RANK] B_m, level-major, j ascending
  int ncores;          // tiles (cores) per system
  int* abort_flag;     // set when a barrier wait exceeds its bound
  int* apply_abort;    // single-pass apply: set when a partner poll exceeds apply_poll_limit;
                       // cleared only by the host once it has read it
  int* itbase;         // graph engine: absolute iteration of the replay's first step
  int* replays;        // graph engine: replays finished
  void* w;             // [B*n] H r in the squared form
  const double* dinv;  // [B*n] 1 / A_ii
  const int* lcol;     // resident engine: [nnz] column as a leaf-local index: own rows
                       // 0 .. LEAF-1, else LEAF + the column's slot in the leaf's halo
  const int* hoff;     // resident engine: [B*K + 1] first halo slot of each leaf
  const int* hcol;     // resident engine: [halo slots] global column of each slot
  unsigned long long* zll;  // resident engine: [B*n][2] z as (word, epoch) pairs
  unsigned long long* pll;  // resident engine: [B*K][4] r.r and r.z partials as (word, epoch) pairs
  unsigned long long* qll;  // resident engine: [2][B][levels][K][RANK] W^T q words by step parity
  unsigned long long* pqll; // resident engine: [2][B*K][2] p.q partials as (word, epoch) pairs by step parity
  unsigned ep_base;    // resident engine: epoch of this solve's z0 (z of step i has ep_base + i)
  unsigned poll_limit; // resident engine: polls of one flagged word before the solve aborts
  unsigned apply_poll_limit;  // single-pass apply: poll rounds before a workgroup gives up
  int form;            // FORM_*
  double tol;
  int maxit;
};

template <typename T>
struct alignas(16) Smem {
  T r[LEAF];                          // phase B: r (then r_new) of the whole leaf; C: block rows
  T t[LEAF];                          // phase B: the slot's slice of U_k^T r_k; C: diagonal shares
  T P[MAX_LEVELS * RANK];             // phase C: partner-half sums per level
  union {
    struct {
      T redT[4 * NT];                 // phase B: U restriction partials [row group][column]
      T redW[NWAVE][MAX_LEVELS * RANK];  // phase B: slab restriction partials per wave
    };
    T redP[8][MAX_LEVELS * RANK];     // phase C: strip-aggregation partials
  };
  T yleaf[LEAF];
  T yoff[LEAF];
  double dred[NWAVE];                 // workgroup sums
  double dsc;                         // broadcast scalar
  int flag;                           // broadcast state
};

struct Blk {
  int item;   // item index (workgroup index after the XCD-aware permutation)
  int s;      // system
  int lb;     // workgroup within system
  int k;      // leaf
  int j;      // slot within leaf (column slice in B, row block in C and A)
  int lrow0;  // first row of the row block within the leaf
  int grow0;  // first global row of the row block
  int leaf0;  // first global row of the leaf
};

// XCD-aware placement.  Workgroups are dispatched to the eight XCDs round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  The item a
// workgroup serves is chosen so that XCD x gets the contiguous item range
// [x*nblk/8, (x+1)*nblk/8): every workgroup that touches leaf k in any phase
// runs on the same XCD, so leaf k's factor rows and vector slices can stay in
// that XCD's L2 from one kernel and one iteration to the next.
constexpr int NXCD = 8;

__device__ __forceinline__ int item_of(const Geom& G, int b) {
  if (G.nblk % NXCD) return b;
  return (b % NXCD) * (G.nblk / NXCD) + b / NXCD;
}

__device__ __forceinline__ Blk decode(const Geom& G, int wg) {
  Blk o;
  const int b = item_of(G, wg);
  o.item = b;
  o.s = b / G.nblk_sys;
  o.lb = b - o.s * G.nblk_sys;
  o.k = o.lb / G.bpl;
  o.j = o.lb - o.k * G.bpl;
  o.lrow0 = o.j * G.RB;
  o.leaf0 = o.s * G.n + o.k * LEAF;
  o.grow0 = o.leaf0 + o.lrow0;
  return o;
}

// ---------------------------------------------------------------------------
// LDS helpers
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_vptr;

// Copy `nchunks` 16-byte chunks into LDS at `dst` (16-byte aligned), packed in
// chunk order; chunk c comes from global address addr(c) (16-byte aligned).
// Each wave moves 64 consecutive chunks (1 KB) per global_load_lds_dwordx4; the
// caller waits with lds_dma_wait() before reading.
template <typename AddrFn>
__device__ __forceinline__ void dma_to_lds(void* dst, int nchunks, AddrFn addr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int q = wave; q * 64 < nchunks; q += NWAVE) {
    const int c = q * 64 + lane;
    lds_vptr l = (lds_vptr)((__attribute__((address_space(3))) char*)dst + q * 1024);
    if (c < nchunks) __builtin_amdgcn_global_load_lds(addr(c), l, 16, 0, 0);
  }
}

// threadIdx.x, with FRESH behind an empty asm.  The persistent solves call
// the steps that take it every iteration; the compiler otherwise hoists every
// address those steps derive from the thread index out of the solve loop,
// where the addresses hold registers for the whole solve.  Where that does not
// fit in the register file they spill to scratch, and each reload in the loop
// waits for every outstanding memory operation; recomputing an address costs a
// couple of integer operations.  Where it fits, the hoisted form is faster.
template <bool FRESH>
__device__ __forceinline__ int tid_of() {
  int t = threadIdx.x;
  if constexpr (FRESH) asm volatile("" : "+v"(t));
  return t;
}

// dma_to_lds for a workgroup of NW waves.  CPOL is the load's cache policy:
// 0 = default, CPOL_AGENT = agent-scope coherent (sc1: never served from a
// stale copy in another XCD's L2).
constexpr int CPOL_AGENT = 16;
template <int NW, int CPOL = 0, bool FRESH = false, typename AddrFn>
__device__ __forceinline__ void dma_to_lds_n(void* dst, int nchunks, AddrFn addr) {
  const int tid = tid_of<FRESH>(), lane = tid & 63, wave = tid >> 6;
  for (int q = wave; q * 64 < nchunks; q += NW) {
    const int c = q * 64 + lane;
    lds_vptr l = (lds_vptr)((__attribute__((address_space(3))) char*)dst + q * 1024);
    if (c < nchunks) __builtin_amdgcn_global_load_lds(addr(c), l, 16, 0, CPOL);
  }
}

// All outstanding global loads (including the DMAs into LDS) of every wave
// have landed after this.
__device__ __forceinline__ void lds_dma_wait() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <typename T>
struct Vec4 { T x, y, z, w; };

__device__ __forceinline__ float4 lds4f(const float* p) { return *reinterpret_cast<const float4*>(p); }

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

// ---------------------------------------------------------------------------
// Cross-lane exchanges without the LDS crossbar.  gfx950 maps xor-32 and
// xor-16 partners with v_permlane32_swap / v_permlane16_swap (the swapped
// half is selected by lane bit 5 / 4), xor 8 with DPP row_ror:8, xor 2 and
// xor 1 with DPP quad_perm, and pairs lane j with 7 - j inside each group of
// eight with DPP row_half_mirror (a perfect matching between the lower and
// upper four lanes, which is all a reduction over those lanes needs).
// 64-bit values are exchanged word by word.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_word(int w) {
  return __builtin_amdgcn_update_dpp(0, w, CTRL, 0xf, 0xf, false);
}

template <typename T, typename Fn>
__device__ __forceinline__ T per_word(T v, Fn fn) {
  if constexpr (sizeof(T) == 4) {
    return __int_as_float(fn(__float_as_int(v)));
  } else {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    return __hiloint2double(fn(hi), fn(lo));
  }
}

template <typename T>
__device__ __forceinline__ T lane_x1(T v) { return per_word(v, [](int w) { return dpp_word<0xb1>(w); }); }
template <typename T>
__device__ __forceinline__ T lane_x2(T v) { return per_word(v, [](int w) { return dpp_word<0x4e>(w); }); }
template <typename T>
__device__ __forceinline__ T lane_m4(T v) { return per_word(v, [](int w) { return dpp_word<0x141>(w); }); }
template <typename T>
__device__ __forceinline__ T lane_x8(T v) { return per_word(v, [](int w) { return dpp_word<0x128>(w); }); }
template <typename T>
__device__ __forceinline__ T lane_x16(T v) {
  return per_word(v, [](int w) {
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)w, (unsigned)w, false, false);
    return (int)((threadIdx.x & 16) ? p[0] : p[1]);
  });
}
template <typename T>
__device__ __forceinline__ T lane_x32(T v) {
  return per_word(v, [](int w) {
    const auto p = __builtin_amdgcn_permlane32_swap((unsigned)w, (unsigned)w, false, false);
    return (int)((threadIdx.x & 32) ? p[0] : p[1]);
  });
}

// Folding steps of a transpose-reduce: one swap moves a's partner into the
// lanes that keep a and b's partner into the lanes that keep b, so lanes with
// bit 5 (bit 4) clear end with a + a(lane ^ 32) (a + a(lane ^ 16)) and the
// others with b + b(partner), with no per-lane selects.  Each sum adds the same
// two values as the select-and-exchange form.
template <typename T, typename Swap>
__device__ __forceinline__ T fold_pair(T a, T b, Swap swap) {
  if constexpr (sizeof(T) == 4) {
    const auto p = swap(__float_as_uint(a), __float_as_uint(b));
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else {
    const auto lo = swap((unsigned)__double2loint(a), (unsigned)__double2loint(b));
    const auto hi = swap((unsigned)__double2hiint(a), (unsigned)__double2hiint(b));
    return __hiloint2double((int)hi[0], (int)lo[0]) + __hiloint2double((int)hi[1], (int)lo[1]);
  }
}
template <typename T>
__device__ __forceinline__ T fold_x32(T a, T b) {
  return fold_pair(a, b, [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane32_swap(x, y, false, false); });
}
template <typename T>
__device__ __forceinline__ T fold_x16(T a, T b) {
  return fold_pair(a, b, [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane16_swap(x, y, false, false); });
}

// Sum over groups of 4 / 8 consecutive lanes (every lane of the group gets it).
template <typename T>
__device__ __forceinline__ T group4_sum(T v) { v += lane_x1(v); return v + lane_x2(v); }
template <typename T>
__device__ __forceinline__ T group8_sum(T v) { v = group4_sum(v); return v + lane_m4(v); }

// Sum of a system's per-workgroup partials, computed by every wave in the same
// order (xor butterflies add commutative pairs), hence bitwise identical in
// every wave and every workgroup.  Loads are issued by the caller's batch.
__device__ __forceinline__ double wave_sum(double v) {
  v = group8_sum(v);
  v += lane_x8(v);
  v += lane_x16(v);
  return v + lane_x32(v);
}

__device__ __forceinline__ double load_partials(const double* part, int s, int nblk_sys) {
  double v = 0.0;
  const double* p = part + (size_t)s * nblk_sys;
  for (int j = threadIdx.x & 63; j < nblk_sys; j += 64) v += p[j];
  return v;
}

// Workgroup sum in a fixed order (deterministic).
template <typename T>
__device__ __forceinline__ double wg_sum(double v, double* red) {
  v = wave_sum(v);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ void park_breakdown(SysState* st, int it) {
  st->brk_it = it;
  __hip_atomic_store(&st->brk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_state(SysState* st, int status, int iters) {
  st->iters = iters;
  __hip_atomic_store(&st->status, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 reads the system state; the value reaches the whole workgroup through
// LDS.  Returns ST_RUNNING, a final status, or -1 when a breakdown is pending.
__device__ __forceinline__ int load_state(const SysState* st) {
  int v = __hip_atomic_load(&st->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v == ST_RUNNING && __hip_atomic_load(&st->brk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) v = -1;
  return v;
}

// Rows of R values that stage a leaf's partner-half restrictions: level l
// (l < levels) at rows 2^l - 1 .. 2^(l+1) - 2, one per leaf of the partner
// half; 2^levels - 1 in all (K - 1 for a full hierarchy), at least one.
__host__ __device__ inline int partner_rows(const Geom& G) {
  return G.levels > 0 ? (1 << G.levels) - 1 : 1;
}

// Dynamic-LDS bytes of the restriction and prolongation stages.
__host__ __device__ inline int levels_of_slot(const Geom& G, int j) {
  return j < G.levels ? (G.levels - 1 - j) / G.bpl + 1 : 0;
}
__host__ __device__ inline size_t restrict_lds_bytes(const Geom& G) {
  return (size_t)4 * ((size_t)LEAF * G.RB + (size_t)levels_of_slot(G, 0) * LEAF * RANK);
}
template <typename T>
__host__ __device__ inline size_t prolong_lds_bytes(const Geom& G) {
  const size_t factors = (size_t)4 * (size_t)G.levels * G.RB * RANK;
  return factors + (size_t)partner_rows(G) * RANK * sizeof(T);
}

// ---------------------------------------------------------------------------
// Restriction (eq. (2)) and the diagonal stage by column slices: from sm.r (the
// leaf's r, all LEAF rows) compute t_j = U_k[:, C_j]^T r_k, the slot's share
// U_k[:, C_j] t_j of the diagonal-block product, and the per-leaf restriction
// of the slot's levels.  Factors were DMA'd to dyn: U slice [LEAF][CW], then
// each owned level's slab [LEAF][RANK].  Writes tleaf (shares) and pleaf.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void issue_restrict_dma(const Geom& G, const Bufs& B, const Blk& bk, float* dyn) {
  const int CW = G.RB;
  const float* Uk = B.U + ((size_t)bk.s * G.K + bk.k) * LEAF * LEAF + (size_t)bk.j * CW;
  const int cpr = CW / 4;  // chunks per row of the slice
  dma_to_lds(dyn, LEAF * cpr, [&](int c) { return Uk + (size_t)(c / cpr) * LEAF + 4 * (c % cpr); });
  float* dw = dyn + LEAF * CW;
  const int nl = levels_of_slot(G, bk.j);
  for (int m = 0; m < nl; ++m) {
    const int l = bk.j + m * G.bpl;
    const float* Wl = B.W + (((size_t)bk.s * G.levels + l) * G.K + bk.k) * LEAF * RANK;
    dma_to_lds(dw + (size_t)m * LEAF * RANK, LEAF * RANK / 4, [&](int c) { return Wl + 4 * c; });
  }
}

// Sum over the lanes of a wave that share lane % slots (slots = 4, 8, 16 or
// 32): xor partners at distances slots .. 32.
template <typename T>
__device__ __forceinline__ T rowgroup_sum(T v, int slots) {
  if (slots <= 4) v += __shfl_xor(v, 4);
  if (slots <= 8) v += lane_x8(v);
  if (slots <= 16) v += lane_x16(v);
  return v + lane_x32(v);
}

// Sum over groups of `width` consecutive lanes (width = 4, 8, 16 or 32).
template <typename T>
__device__ __forceinline__ T group_sum(T v, int width) {
  v = group4_sum(v);
  if (width > 4) v += lane_m4(v);
  if (width > 8) v += lane_x8(v);
  if (width > 16) v += lane_x16(v);
  return v;
}

template <typename T>
__device__ __forceinline__ void restrict_leaf(const Geom& G, const Bufs& B, const Blk& bk, const float* dyn,
                                              Smem<T>& sm) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int CW = G.RB;
  const int slots = CW / 4;              // 4-column slots of the slice
  T* share = reinterpret_cast<T*>(B.tleaf) + (((size_t)bk.s * G.K + bk.k) * G.bpl + bk.j) * LEAF;
  T* pleaf = reinterpret_cast<T*>(B.pleaf);
  {
    // t_j: thread = (4-column slot c4, row group rg); RG row groups.  The row
    // groups of a wave (lane bits log2(slots) .. 5) are summed across lanes,
    // then the four waves through LDS.
    const int RG = NT / slots;
    const int c4 = tid % slots, rg = tid / slots;
    Vec4<T> acc{0, 0, 0, 0};
    for (int i = rg; i < LEAF; i += RG) axpy4(acc, lds4f(dyn + i * CW + 4 * c4), sm.r[i]);
    acc.x = rowgroup_sum(acc.x, slots); acc.y = rowgroup_sum(acc.y, slots);
    acc.z = rowgroup_sum(acc.z, slots); acc.w = rowgroup_sum(acc.w, slots);
    if ((tid & 63) < slots) {
      T* d = &sm.redT[wave * CW + 4 * c4];
      d[0] = acc.x; d[1] = acc.y; d[2] = acc.z; d[3] = acc.w;
    }
  }
  {
    // owned levels: thread = (4-column slot cs of 8, row group rg of 32); the
    // rows of a wave (lane bits 3..5) are summed with xor 8, 16, 32
    const int cs = tid & 7, rg = tid >> 3;
    const int nl = levels_of_slot(G, bk.j);
    const float* dw = dyn + LEAF * CW;
    for (int m = 0; m < nl; ++m) {
      const float* Wm = dw + (size_t)m * LEAF * RANK;
      Vec4<T> acc{0, 0, 0, 0};
#pragma unroll
      for (int i = rg; i < LEAF; i += 32) axpy4(acc, lds4f(Wm + i * RANK + 4 * cs), sm.r[i]);
      acc.x += lane_x8(acc.x); acc.y += lane_x8(acc.y); acc.z += lane_x8(acc.z); acc.w += lane_x8(acc.w);
      acc.x += lane_x16(acc.x); acc.y += lane_x16(acc.y); acc.z += lane_x16(acc.z); acc.w += lane_x16(acc.w);
      acc.x += lane_x32(acc.x); acc.y += lane_x32(acc.y); acc.z += lane_x32(acc.z); acc.w += lane_x32(acc.w);
      if ((tid & 63) < 8) {
        T* d = &sm.redW[wave][m * RANK + 4 * cs];
        d[0] = acc.x; d[1] = acc.y; d[2] = acc.z; d[3] = acc.w;
      }
    }
  }
  __syncthreads();
  {
    if (tid < CW) {
      T a = sm.redT[tid];
#pragma unroll
      for (int w = 1; w < NWAVE; ++w) a += sm.redT[w * CW + tid];
      sm.t[tid] = a;
    }
    const int nl = levels_of_slot(G, bk.j);
    for (int e = tid; e < nl * RANK; e += NT) {
      T a = sm.redW[0][e];
#pragma unroll
      for (int w = 1; w < NWAVE; ++w) a += sm.redW[w][e];
      const int m = e / RANK, c = e - m * RANK;
      const int l = bk.j + m * G.bpl;
      pleaf[(((size_t)bk.s * G.levels + l) * G.K + bk.k) * RANK + c] = a;
    }
  }
  __syncthreads();
  {
    // the slot's diagonal share: row i's dot of U_k[i, C_j] with t_j, `slots`
    // lanes per row (4 columns each), NT / slots rows per pass
    const int c4 = tid % slots, ri = tid / slots, rows = NT / slots;
    const Vec4<T> t4 = lds4(&sm.t[4 * c4]);
    for (int i = ri; i < LEAF; i += rows) {
      const T v = group_sum(dot4(lds4f(dyn + i * CW + 4 * c4), t4), slots);
      if (c4 == 0) share[i] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Prolongation (eqs. (3)-(5)) and assembly on the workgroup's row block.  DMA:
// slab rows [levels][RB][RANK], the partner half's per-leaf restrictions of
// every level (stage, level l at row 2^l - 1), the bpl diagonal shares of the
// block rows.  Needs sm.r (block rows) and g; returns y for row tid (tid < RB).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void issue_prolong_dma(const Geom& G, const Bufs& B, const Blk& bk, float* dyn,
                                                  Smem<T>& sm) {
  const int RB = G.RB;
  float* dw = dyn;
  for (int l = 0; l < G.levels; ++l) {
    const float* Wl = B.W + (((size_t)bk.s * G.levels + l) * G.K + bk.k) * LEAF * RANK + (size_t)bk.lrow0 * RANK;
    dma_to_lds(dw + (size_t)l * RB * RANK, RB * RANK / 4, [&](int c) { return Wl + 4 * c; });
  }
  T* stage = reinterpret_cast<T*>(dw + (size_t)G.levels * RB * RANK);
  const T* pleaf = reinterpret_cast<const T*>(B.pleaf);
  constexpr int CPV = RANK * sizeof(T) / 16;   // chunks per restriction vector
  for (int l = 0; l < G.levels; ++l) {
    const int kp0 = ((bk.k >> l) ^ 1) << l;
    const T* src = pleaf + (((size_t)bk.s * G.levels + l) * G.K + kp0) * RANK;
    dma_to_lds(stage + (size_t)((1 << l) - 1) * RANK, (1 << l) * CPV,
               [&](int c) { return reinterpret_cast<const char*>(src) + 16 * c; });
  }
  // shares: slot j' rows [lrow0, lrow0 + RB) into sm.t[j' * RB ...]
  const T* sh = reinterpret_cast<const T*>(B.tleaf) + ((size_t)bk.s * G.K + bk.k) * G.bpl * LEAF + bk.lrow0;
  const int cps = RB * (int)sizeof(T) / 16;    // chunks per slot
  dma_to_lds(sm.t, G.bpl * cps, [&](int c) {
    const int j = c / cps;
    return reinterpret_cast<const char*>(sh + (size_t)j * LEAF) + 16 * (c - j * cps);
  });
}

template <typename T>
__device__ __forceinline__ T prolong_rows(const Geom& G, const Bufs& B, const Blk& bk, const float* dyn,
                                          Smem<T>& sm) {
  const int tid = threadIdx.x;
  const int RB = G.RB;
  const float* dw = dyn;
  const T* stage = reinterpret_cast<const T*>(dw + (size_t)G.levels * RB * RANK);
  // strip aggregation (eq. (3)): P_l[c] = sum over the 2^l partner leaves
  {
    const int c = tid & 31, g = tid >> 5;
    for (int l = 0; l < G.levels; ++l) {
      const T* v = stage + (size_t)((1 << l) - 1) * RANK + c;
      T acc = 0;
      for (int i = g; i < (1 << l); i += 8) acc += v[i * RANK];
      sm.redP[g][l * RANK + c] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < G.levels * RANK; e += NT) {
    T a = sm.redP[0][e];
#pragma unroll
    for (int g = 1; g < 8; ++g) a += sm.redP[g][e];
    sm.P[e] = a;
  }
  __syncthreads();
  // prolongation (eq. (5)): per row, sum over levels of slab row . P_l
  {
    const int cs = tid & 7, rg = tid >> 3;
    for (int i = rg; i < RB; i += 32) {
      T acc = 0;
      for (int l = 0; l < G.levels; ++l)
        acc += dot4(lds4f(dw + ((size_t)l * RB + i) * RANK + 4 * cs), lds4(&sm.P[l * RANK + 4 * cs]));
      acc = group8_sum(acc);
      if (cs == 0) sm.yoff[i] = acc;
    }
  }
  __syncthreads();
  T y = 0;
  if (tid < RB) {
    T d = sm.t[tid];
    for (int j = 1; j < G.bpl; ++j) d += sm.t[j * RB + tid];
    y = d + sm.yoff[tid] + (T)B.g[bk.grow0 + tid] * sm.r[tid];
  }
  return y;
}

// r after iteration it (0 = initial) lives in half it & 1 of the r buffer.
template <typename T>
__device__ __forceinline__ T* r_buf(const Geom& G, const Bufs& B, int it) {
  return reinterpret_cast<T*>(B.r) + ((it & 1) ? (size_t)G.B * G.n : 0);
}

// p_new = z + beta p_old, evaluated identically wherever it is needed so that
// the stored p and the p the SpMV multiplies are the same numbers.
template <typename T>
__device__ __forceinline__ T pdir(T z, T pold, double beta) {
  return (T)((double)z + beta * (double)pold);
}

// ---------------------------------------------------------------------------
// Phases.  b = workgroup index (mapped to an item by decode); it = iteration
// (1-based; 0 = initial).
// ---------------------------------------------------------------------------

// Phase B (and the initial restriction when it == 0: r = b, x = 0).
// Phase B (and the initial restriction when it == 0: r = b, x = 0).  stage 1
// (squared form only): restriction of w = H r for the second factor.
template <typename T>
__device__ __forceinline__ void phase_B(const Geom& G, const Bufs& B, int b, int it, Smem<T>& sm, float* dyn,
                                        int stage = 0) {
  const Blk bk = decode(G, b);
  const int tid = threadIdx.x;
  SysState* st = B.st + bk.s;
  const bool init = (it == 0);
  if (stage == 1) {
    issue_restrict_dma<T>(G, B, bk, dyn);
    if (tid == 0) sm.flag = load_state(st);
    if (tid < LEAF) sm.r[tid] = reinterpret_cast<const T*>(B.w)[bk.leaf0 + tid];
    lds_dma_wait();
    if (sm.flag != ST_RUNNING) return;
    restrict_leaf(G, B, bk, dyn, sm);
    return;
  }
  const bool restrict_r = (B.form != FORM_JACOBI);
  // every slot of a leaf reads the leaf's whole old r while each writes only
  // its own rows of the new r, so old and new live in different buffers
  const T* rold = r_buf<T>(G, B, it - 1);
  T* rnew = r_buf<T>(G, B, it);
  // ---- one batch of loads ----
  if (restrict_r) issue_restrict_dma<T>(G, B, bk, dyn);
  const double pqv = init ? 0.0 : load_partials(B.pq_part, bk.s, G.nblk_sys);
  int state = ST_RUNNING;
  double rzv = 0.0;
  if (tid == 0 && !init) {
    state = load_state(st);
    rzv = st->rz[(it - 1) & 1];
  }
  T rv = 0, qv = 0, pv = 0;
  double xv = 0.0;
  const bool own = (tid >= bk.lrow0 && tid < bk.lrow0 + G.RB);
  if (tid < LEAF) {
    if (init) {
      rv = (T)B.b[bk.leaf0 + tid];
    } else {
      rv = rold[bk.leaf0 + tid];
      qv = reinterpret_cast<const T*>(B.q)[bk.leaf0 + tid];
      if (own) {
        pv = reinterpret_cast<const T*>((it & 1) ? B.p1 : B.p0)[bk.leaf0 + tid];
        xv = B.x[bk.leaf0 + tid];
      }
    }
  }
  const double pq = wave_sum(pqv);
  if (tid == 0) { sm.flag = state; sm.dsc = rzv; }
  lds_dma_wait();
  if (!init) {
    if (sm.flag != ST_RUNNING) return;
    if (!(pq > 0.0) || !isfinite(pq)) {
      if (tid == 0 && bk.lb == 0) park_breakdown(st, it);
      return;
    }
  }
  const double alpha = init ? 0.0 : sm.dsc / pq;
  double loc = 0.0;
  if (tid < LEAF) {
    const T rn = init ? rv : (T)((double)rv - alpha * (double)qv);
    sm.r[tid] = rn;
    if (own) {
      rnew[bk.leaf0 + tid] = rn;
      B.x[bk.leaf0 + tid] = init ? 0.0 : xv + alpha * (double)pv;
      loc = (double)rn * (double)rn;
    }
  }
  __syncthreads();
  if (restrict_r) restrict_leaf(G, B, bk, dyn, sm);
  const double rr = wg_sum<T>(loc, sm.dred);
  if (tid == 0) {
    B.rr_part[bk.item] = rr;
    if (init && bk.lb == 0) {
      st->relres = 1.0;
      st->brk = 0;
      st->brk_it = 0;
      set_state(st, ST_RUNNING, 0);
    }
  }
}

// stage 0: convergence test, z = M r, partial r.z (direct and Jacobi forms);
// squared form: stage 1 = test and w = H r, stage 2 = z = H w and r.z.
template <typename T>
__device__ __forceinline__ void phase_C(const Geom& G, const Bufs& B, int b, int it, Smem<T>& sm, float* dyn,
                                        int stage = 0) {
  const Blk bk = decode(G, b);
  const int tid = threadIdx.x;
  SysState* st = B.st + bk.s;
  const bool lead = (tid == 0 && bk.lb == 0);
  const bool jacobi = (B.form == FORM_JACOBI);
  if (stage == 2) {
    issue_prolong_dma<T>(G, B, bk, dyn, sm);
    if (tid == 0) sm.flag = load_state(st);
    T rv = 0;
    if (tid < G.RB) {
      rv = r_buf<T>(G, B, it)[bk.grow0 + tid];
      sm.r[tid] = reinterpret_cast<const T*>(B.w)[bk.grow0 + tid];   // the vector H is applied to
    }
    lds_dma_wait();
    if (sm.flag != ST_RUNNING) return;
    const T zv = prolong_rows(G, B, bk, dyn, sm);
    double loc = 0.0;
    if (tid < G.RB) {
      reinterpret_cast<T*>(B.z)[bk.grow0 + tid] = zv;
      loc = (double)rv * (double)zv;
    }
    const double rz = wg_sum<T>(loc, sm.dred);
    if (tid == 0) B.rz_part[bk.item] = rz;
    return;
  }
  // ---- one batch of loads ----
  if (!jacobi) issue_prolong_dma<T>(G, B, bk, dyn, sm);
  const double rrv = load_partials(B.rr_part, bk.s, G.nblk_sys);
  int state = ST_RUNNING;
  double bnorm = 0.0;
  if (tid == 0) {
    state = (it == 0) ? ST_RUNNING : load_state(st);
    bnorm = st->bnorm;
  }
  const T* r = r_buf<T>(G, B, it);
  T rv = 0;
  if (tid < G.RB) rv = r[bk.grow0 + tid];
  const double rr = wave_sum(rrv);
  if (tid == 0) { sm.flag = state; sm.dsc = bnorm; }
  if (tid < G.RB) sm.r[tid] = rv;
  lds_dma_wait();
  const int cur = sm.flag;
  if (cur == -1) {
    if (lead) set_state(st, ST_BREAKDOWN, st->brk_it);
    return;
  }
  if (cur != ST_RUNNING) return;
  if (it == 0) {
    if (lead) st->bnorm = sqrt(rr);
    if (rr == 0.0) {
      if (lead) { st->relres = 0.0; set_state(st, ST_CONVERGED, 0); }
      return;
    }
  } else {
    const double rel = sqrt(rr) / sm.dsc;
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
  if (jacobi) {
    double loc = 0.0;
    if (tid < G.RB) {
      const T zv = (T)((double)sm.r[tid] * B.dinv[bk.grow0 + tid]);
      reinterpret_cast<T*>(B.z)[bk.grow0 + tid] = zv;
      loc = (double)sm.r[tid] * (double)zv;
    }
    const double rz = wg_sum<T>(loc, sm.dred);
    if (tid == 0) B.rz_part[bk.item] = rz;
    return;
  }
  const T zv = prolong_rows(G, B, bk, dyn, sm);
  if (stage == 1) {                       // squared form: w = H r, no partial yet
    if (tid < G.RB) reinterpret_cast<T*>(B.w)[bk.grow0 + tid] = zv;
    return;
  }
  double loc = 0.0;
  if (tid < G.RB) {
    reinterpret_cast<T*>(B.z)[bk.grow0 + tid] = zv;
    loc = (double)sm.r[tid] * (double)zv;
  }
  const double rz = wg_sum<T>(loc, sm.dred);
  if (tid == 0) B.rz_part[bk.item] = rz;
}

// Phase A: beta, p = z + beta p, q = A p (row block), partial p.q.
template <typename T>
__device__ __forceinline__ void phase_A(const Geom& G, const Bufs& B, int b, int it, Smem<T>& sm) {
  const Blk bk = decode(G, b);
  const int tid = threadIdx.x;
  SysState* st = B.st + bk.s;
  const T* z = reinterpret_cast<const T*>(B.z);
  const T* pold = reinterpret_cast<const T*>((it & 1) ? B.p0 : B.p1);
  T* pnew = reinterpret_cast<T*>((it & 1) ? B.p1 : B.p0);
  const bool first = (it == 1);
  // ---- loads: scalars, own row, row extent ----
  const double rzv = load_partials(B.rz_part, bk.s, G.nblk_sys);
  int state = ST_RUNNING;
  double rzold = 1.0;
  if (tid == 0) {
    state = load_state(st);
    if (!first) rzold = st->rz[(it - 2) & 1];
  }
  const int TPR = NT / G.RB;
  const int i = tid / TPR, lr = tid - i * TPR;
  const int grow = bk.grow0 + i;
  const int e0 = B.row_ptr[grow], e1 = B.row_ptr[grow + 1];
  T zown = 0, pown = 0;
  if (lr == 0) {
    zown = z[grow];
    if (!first) pown = pold[grow];
  }
  const double rz = wave_sum(rzv);
  if (tid == 0) { sm.flag = state; sm.dsc = rzold; }
  __syncthreads();
  if (sm.flag != ST_RUNNING) return;
  if (!(rz > 0.0) || !isfinite(rz)) {
    if (tid == 0 && bk.lb == 0) park_breakdown(st, it - 1);
    return;
  }
  const double beta = first ? 0.0 : rz / sm.dsc;
  if (tid == 0 && bk.lb == 0) st->rz[(it - 1) & 1] = rz;
  // ---- SpMV of p_new on the fly: entries in passes of 4 per thread ----
  T acc = 0;
  for (int e = e0 + lr; e < e1; e += 4 * TPR) {
    int c[4];
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int eu = e + u * TPR;
      c[u] = eu < e1 ? B.col[eu] : grow;
      v[u] = eu < e1 ? B.val[eu] : 0.f;
    }
    T pz[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pz[u] = first ? z[c[u]] : pdir<T>(z[c[u]], pold[c[u]], beta);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = fma((T)v[u], pz[u], acc);
  }
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
  double loc = 0.0;
  if (lr == 0) {
    const T pn = first ? zown : pdir<T>(zown, pown, beta);
    pnew[grow] = pn;
    reinterpret_cast<T*>(B.q)[grow] = acc;
    loc = (double)pn * (double)acc;
  }
  const double pq = wg_sum<T>(loc, sm.dred);
  if (tid == 0) B.pq_part[bk.item] = pq;
}

}  // namespace hpcg
