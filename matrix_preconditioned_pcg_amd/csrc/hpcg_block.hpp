// Block (multi-right-hand-side) apply Y = M R and block SpMV Y = A X on gfx950
// matrix cores.
//
// With a block of right-hand sides every stage of the apply is a real GEMM: the
// leaf stage is F_k R_k with R_k of 128 x nrhs and F_k = U_k U_k^T the dense
// leaf block (one product where U_k (U_k^T R_k) takes two), the restriction
// W_l[k]^T R_k, the prolongation W_l[k] P_l.  This is the probe-block product
// the pages' training objective needs (M A Z for a probe block Z of N x K_z,
// project page "Cosine Hutchinson Probe Loss" and "Training Setup"; Supplementary
// section 3, "Probe vectors"), and the multi-vector form of the apply of
// "Hierarchical Transformer Preconditioning for Interactive Physics Simulation",
// section 5, stages (i)-(ii), eqs. (2)-(5).
//
// Layout: R, Y, X are node-major, [B*n][nrhs] fp32 (the nrhs values of a node are
// contiguous).  A workgroup (4 wave64) owns one leaf and NCT 16-column tiles
// (up to four, so that each factor operand it loads feeds more products).
// The products are fp32 products formed on the fp16 matrix cores from fp16
// pairs (below): the operands of every product are held, or staged in LDS, in
// the order of the contraction index, so that a lane's eight contraction steps
// of an MFMA are one 16-byte read; A and B take the same order, so the sum is
// the same product.
//
// Three launches: (1) per (leaf, tile): Y = F_k R_k + g R with the dense leaf
// block F_k = U_k U_k^T (formed once per set of factors, k_leaf_blocks), and the
// per-leaf restrictions Q_l[k] = W_l[k]^T R_k; (2) per (level, half, element):
// the half sums of Q_l over every tile half (eq. (3)), in a fixed order; (3) per
// (leaf, tile): Y += sum_l W_l[k] P_l with P_l the partner half's sum (eqs.
// (4)-(5), identity core).  The block solve has (1) take its residual update
// and (3) its r.z partials (BlockUpd, BlockDot), so that neither needs a pass
// of its own over the block.
#pragma once
#include "hpcg_colstate.hpp"

namespace hpcg {

constexpr int BNC = 16;          // right-hand-side columns per workgroup
constexpr int BNT = 256;         // threads per workgroup

typedef float mf4 __attribute__((ext_vector_type(4)));

// fp32 products from fp16 pairs.  A value x of a scaled set (one power of two
// 2^e for the set, e from its largest magnitude so that it lands in
// [2^13, 2^14)) is held as hi = fp16(x 2^e), lo = fp16(x 2^e - hi): 22 bits of
// x.  A product a b is hi_a hi_b + hi_a lo_b + lo_a hi_b (each exact in the fp32
// accumulator; the dropped lo_a lo_b and the pairs' own rounding are ~2^-22 of
// |a b|), summed by v_mfma_f32_16x16x32_f16: lane l supplies A[l % 16][8 (l / 16)
// + i] and B[8 (l / 16) + i][l % 16], i < 8, and receives D[4 (l / 16) + v][l % 16];
// the result is unscaled by 2^-(e_a + e_b), exactly.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ mf4 mfma16(h8 a, h8 b, mf4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// hi lo, hi lo products of one K = 32 step (three MFMAs)
__device__ __forceinline__ mf4 mfma_pair(h8 ah, h8 al, h8 bh, h8 bl, mf4 c) {
  c = mfma16(ah, bh, c);
  c = mfma16(ah, bl, c);
  return mfma16(al, bh, c);
}
// the scale exponent of a set whose largest magnitude is m
__device__ __forceinline__ int pair_exponent(float m) {
  if (!(m > 0.f) || !isfinite(m)) return 0;
  int x;
  (void)frexpf(m, &x);
  return 14 - x;
}
__device__ __forceinline__ void to_pair(float v, int e, _Float16& hi, _Float16& lo) {
  const float sv = ldexpf(v, e);
  hi = (_Float16)sv;
  lo = (_Float16)(sv - (float)hi);
}

// Factors of the block apply as fp16 pairs: the dense leaf blocks (exponent per
// leaf), the slabs in their own layout for the prolongation and transposed
// (rank-major) for the restriction (exponent per slab).
struct BlockFactors16 {
  const _Float16* Fh; const _Float16* Fl; const int* Fe;    // [B][K][LEAF][LEAF], [B][K]
  const _Float16* Wh; const _Float16* Wl;                   // [B][levels][K][LEAF][RANK]
  const _Float16* Th; const _Float16* Tl;                   // [B][levels][K][RANK][LEAF]
  const int* We;                                            // [B][levels][K]
};

struct BlockGeom {
  int n, K, levels, B;   // as Geom
  int nrhs;              // columns of R / Y (multiple of BNC)
  int tiles;             // column tiles of a leaf: nrhs / (BNC NCT), NCT the kernels' tiles per workgroup
};

// Workgroup -> (system, leaf, column tile).  Workgroups are dispatched to the
// eight XCDs round-robin; the items are dealt so that each XCD gets a
// contiguous item range, i.e. all column tiles of a leaf run on one XCD and
// read that leaf's factors through the same L2.
struct BItem { int s, k, ct, leaf0; };
__device__ __forceinline__ BItem bitem(const BlockGeom& G) {
  BItem o;
  const int nblk = G.B * G.K * G.tiles;
  const int b = (nblk % NXCD) ? (int)blockIdx.x
                              : (int)(blockIdx.x % NXCD) * (nblk / NXCD) + (int)(blockIdx.x / NXCD);
  o.ct = b % G.tiles;
  const int lk = b / G.tiles;
  o.s = lk / G.K;
  o.k = lk - o.s * G.K;
  o.leaf0 = o.s * G.n + o.k * LEAF;
  return o;
}

// The same dealing over two workgroups per item (SPLIT): role 0 and role 1 of
// an item are consecutive in the dealt order, so they run on one XCD.
__device__ __forceinline__ BItem bitem2(const BlockGeom& G, int& role) {
  BItem o;
  const int nblk = 2 * G.B * G.K * G.tiles;
  const int b = (nblk % NXCD) ? (int)blockIdx.x
                              : (int)(blockIdx.x % NXCD) * (nblk / NXCD) + (int)(blockIdx.x / NXCD);
  role = b & 1;
  const int item = b >> 1;
  o.ct = item % G.tiles;
  const int lk = item / G.tiles;
  o.s = lk / G.K;
  o.k = lk - o.s * G.K;
  o.leaf0 = o.s * G.n + o.k * LEAF;
  return o;
}

// Q layout: [B][levels][K][RANK][nrhs].
__device__ __forceinline__ size_t q_index(const BlockGeom& G, int s, int l, int k, int row) {
  return ((((size_t)s * G.levels + l) * G.K + k) * RANK + row) * G.nrhs;
}

// The block solve's residual update, taken by the leaf stage as it loads R
// (UPD): first the PQ step of the workgroup's columns (hpcg_colstate.hpp) from
// the p.q partials, then R <- R - alpha_c (A P) column by column, in fp64 and
// rounded to fp32 once, a column whose alpha is 0 keeping its R; the new R is
// written back and the apply runs on it, and the workgroup leaves its (system,
// leaf, column) partials of the new R . R.
struct BlockUpd {
  ColState* cs;          // [B][nrhs]; leaf 0's workgroups store the PQ step
  const double* pq;      // [B][K][nrhs] partials of P . A P
  const float* AP;       // A P, node-major like R
  float* R;              // where the new R goes (the buffer R is read from)
  double* rr;            // [B][K][nrhs] partials of the new R . R
};

// The block solve's r.z partials, taken by the prolongation as it stores Z
// (DOT): per (system, leaf, column), the fp64 sum of R Z over the leaf's rows.
struct BlockDot {
  const float* R;
  double* rz;            // [B][K][nrhs]
};

// Dense leaf blocks F_k = U_k U_k^T, formed once per set of factors so that
// the block apply's leaf stage is one product F_k R_k: every entry summed in
// fp64 over the leaf's 128 columns in column order, then held as an fp16 pair
// with one exponent for the leaf (F_k is exactly symmetric).  One workgroup per
// leaf; U_k is staged in LDS with rows padded to 129 words, so the lanes' walks
// down a column hit distinct banks.  Thread t owns row t % 128 of half t / 128
// of the columns and writes them as column entries (F_k is symmetric),
// coalesced across lanes.
__global__ __launch_bounds__(BNT) void k_leaf_blocks(const float* __restrict__ U, _Float16* __restrict__ Fh,
                                                     _Float16* __restrict__ Fl, int* __restrict__ Fe) {
  constexpr int PAD = LEAF + 1;
  __shared__ float Us[LEAF * PAD];
  __shared__ float wmax[NWAVE];
  const size_t leaf = blockIdx.x;
  const float* Uk = U + leaf * LEAF * LEAF;
  for (int e = threadIdx.x; e < LEAF * LEAF; e += BNT) Us[(e / LEAF) * PAD + e % LEAF] = Uk[e];
  __syncthreads();
  const int i = threadIdx.x % LEAF, j0 = (threadIdx.x / LEAF) * (LEAF / 2);
  double acc[LEAF / 2];
#pragma unroll
  for (int jj = 0; jj < LEAF / 2; ++jj) acc[jj] = 0.0;
  for (int k = 0; k < LEAF; ++k) {
    const double ui = Us[i * PAD + k];
#pragma unroll
    for (int jj = 0; jj < LEAF / 2; ++jj) acc[jj] = fma(ui, (double)Us[(j0 + jj) * PAD + k], acc[jj]);
  }
  float m = 0.f;
#pragma unroll
  for (int jj = 0; jj < LEAF / 2; ++jj) m = fmaxf(m, fabsf((float)acc[jj]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wmax[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) m = fmaxf(m, wmax[w]);
  const int e = pair_exponent(m);
  if (threadIdx.x == 0) Fe[leaf] = e;
  const size_t base = leaf * LEAF * LEAF;
#pragma unroll
  for (int jj = 0; jj < LEAF / 2; ++jj) {
    _Float16 hi, lo;
    to_pair((float)acc[jj], e, hi, lo);
    Fh[base + (size_t)(j0 + jj) * LEAF + i] = hi;
    Fl[base + (size_t)(j0 + jj) * LEAF + i] = lo;
  }
}

// Slabs as fp16 pairs (one exponent per slab), in the slab layout [row][rank]
// and transposed [rank][row].  One workgroup per (system, level, leaf) slab.
__global__ __launch_bounds__(BNT) void k_split_slabs(const float* __restrict__ W, _Float16* __restrict__ Wh,
                                                     _Float16* __restrict__ Wl, _Float16* __restrict__ Th,
                                                     _Float16* __restrict__ Tl, int* __restrict__ We) {
  constexpr int N = LEAF * RANK, PER = N / BNT;
  __shared__ float wmax[NWAVE];
  const size_t base = (size_t)blockIdx.x * N;
  float v[PER];
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    v[u] = W[base + threadIdx.x + u * BNT];
    m = fmaxf(m, fabsf(v[u]));
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wmax[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) m = fmaxf(m, wmax[w]);
  const int e = pair_exponent(m);
  if (threadIdx.x == 0) We[blockIdx.x] = e;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + u * BNT, row = idx / RANK, c = idx - row * RANK;
    _Float16 hi, lo;
    to_pair(v[u], e, hi, lo);
    Wh[base + idx] = hi;
    Wl[base + idx] = lo;
    Th[base + (size_t)c * LEAF + row] = hi;
    Tl[base + (size_t)c * LEAF + row] = lo;
  }
}

// (1) leaf stage, gate and restriction: Y = F_k R_k + g R (F_k = U_k U_k^T,
// k_leaf_blocks) and Q_l = W_l[k]^T R_k, both as fp16-pair products (above).
// The R tile comes through a DMA into LDS (fp32, for the UPD update and the
// gate) and is then held transposed as fp16 pairs with one exponent per column
// (from the column's largest magnitude over the leaf's rows), where a lane's
// eight contraction steps of one MFMA are one 16-byte read.  A workgroup owns
// NCT 16-column tiles (BW = 16 NCT columns): every F_k and W_l[k] operand it
// loads feeds the MFMAs of all NCT tiles.  SPLIT runs the leaf stage (role 0)
// and the restriction (role 1) of an item in two workgroups, each with its own
// copy of the R tile (both take the UPD update, the same arithmetic; role 0
// writes it back and leaves the partials).  At most 256 VGPRs (two waves per
// SIMD), so that two workgroups share a compute unit.
constexpr int RT_STRIDE = 136;   // R^T pair rows in LDS, halfs (272 B: conflict-free 16-byte reads)
template <int LEV, int NCT, bool UPD = false, bool SPLIT = false>
__global__ __launch_bounds__(BNT, 2) void k_block_restrict(BlockGeom G, BlockFactors16 fw,
                                                           const float* __restrict__ g, const float* R,
                                                           float* __restrict__ Y, float* __restrict__ Q, BlockUpd up) {
  constexpr int BW = BNC * NCT;
  constexpr int C4 = BW / 4;                 // 16-byte chunks per tile row
  constexpr int CH = LEAF * C4 / BNT;        // chunks of the tile per thread
  constexpr int WL = (LEV + 1) / 2;          // levels of a wave, at most
  __shared__ __attribute__((aligned(16))) float Rs[LEAF * BW];              // R_k tile, [row][BW]
  __shared__ __attribute__((aligned(16))) _Float16 Rth[BW * RT_STRIDE];     // R^T pairs, [col][row]
  __shared__ __attribute__((aligned(16))) _Float16 Rtl[BW * RT_STRIDE];
  __shared__ int eR[BW];                                                    // exponent per column
  __shared__ float cmax[BNT];                                               // per (row group, column)
  __shared__ double red[UPD ? NWAVE * BW : 1];
  __shared__ double pq_red[UPD ? BNT : 1];                                  // p.q group sums
  __shared__ double alpha_s[UPD ? BW : 1];
  int role = 0;
  const BItem it = SPLIT ? bitem2(G, role) : bitem(G);
  const bool leaf_role = !SPLIT || role == 0;      // leaf stage, gate, write-back
  const int wgi = (int)blockIdx.x;
  stamp(wgi, 0);
  stamp_value(wgi, 7, (unsigned long long)(SPLIT ? role : 2));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  const size_t leaf = (size_t)it.s * G.K + it.k;
  // restriction work of this wave: rank tile (w & 1) of levels par, par + 2, ...
  const int mt = w & 1, par = w >> 1;
  // leaf-stage A operands: rows 32w + r and 32w + 16 + r of F_k, step s covers
  // columns 32 s + 8 q .. + 7
  h8 fa_h[4], fa_l[4], fb_h[4], fb_l[4];
  float gv[8];
  int eF = 0;
  auto load_leaf = [&]() {
    const _Float16* Fa_h = fw.Fh + leaf * LEAF * LEAF + (size_t)(32 * w + r) * LEAF + 8 * q;
    const _Float16* Fa_l = fw.Fl + leaf * LEAF * LEAF + (size_t)(32 * w + r) * LEAF + 8 * q;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      fa_h[st] = *reinterpret_cast<const h8*>(Fa_h + 32 * st);
      fa_l[st] = *reinterpret_cast<const h8*>(Fa_l + 32 * st);
      fb_h[st] = *reinterpret_cast<const h8*>(Fa_h + 16 * LEAF + 32 * st);
      fb_l[st] = *reinterpret_cast<const h8*>(Fa_l + 16 * LEAF + 32 * st);
    }
    eF = fw.Fe[leaf];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      gv[v] = g[it.leaf0 + 32 * w + 4 * q + v];
      gv[4 + v] = g[it.leaf0 + 32 * w + 16 + 4 * q + v];
    }
  };
  // restriction A operands of the wave's levels: row 16 mt + r of W_l[k]^T, step
  // s covers rows 32 s + 8 q .. + 7 of the slab.  SPLIT: every level's at once;
  // in one workgroup two levels' worth, a level's issued a level ahead.
  constexpr int NB = SPLIT ? (WL > 0 ? WL : 1) : 2;
  h8 wt_h[NB][4], wt_l[NB][4];
  int eW[NB];
  auto load_slot = [&](int b, int l) {
    const size_t slab = ((size_t)it.s * LEV + l) * G.K + it.k;
    const size_t o = slab * LEAF * RANK + (size_t)(16 * mt + r) * LEAF + 8 * q;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      wt_h[b][st] = *reinterpret_cast<const h8*>(fw.Th + o + 32 * st);
      wt_l[b][st] = *reinterpret_cast<const h8*>(fw.Tl + o + 32 * st);
    }
    eW[b] = fw.We[slab];
  };
  auto load_restr = [&]() {
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < WL; ++i)
        if (par + 2 * i < LEV) load_slot(i, par + 2 * i);
    } else {
      if (par < LEV) load_slot(0, par);
    }
  };
  // UPD: the column's state as the PQ step reads it, loaded before anything else
  constexpr int GP = BNT / BW;               // threads per column
  const int pcol = tid % BW, gp = tid / BW;
  double rz_col = 0.0;
  int st_col = 0, it_col = 0;
  if constexpr (UPD) {
    if (gp == 0) {
      const ColState* cp = up.cs + (size_t)it.s * G.nrhs + c0 + pcol;
      rz_col = cp->rz;
      st_col = cp->status;
      it_col = cp->iters;
    }
  }
  // R tile: 128 rows x 4 BW bytes, straight into LDS
  dma_to_lds(Rs, LEAF * BW / 4, [&](int c) {
    return R + (size_t)(it.leaf0 + c / (BW / 4)) * G.nrhs + c0 + 4 * (c % (BW / 4));
  });
  // UPD: the thread's chunks c = tid + BNT i of the tile, all in its four
  // columns cc..cc+3 (BNT is a multiple of C4)
  const int cc = c0 + 4 * (tid % C4);
  double al[4] = {0.0, 0.0, 0.0, 0.0}, rr4[4] = {0.0, 0.0, 0.0, 0.0};
  mf4 ap[UPD ? CH : 1];
  if constexpr (UPD) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + BNT * i) / C4;
      ap[i] = *reinterpret_cast<const mf4*>(up.AP + (size_t)(it.leaf0 + row) * G.nrhs + cc);
    }
  }
  // UPD: the PQ step of the tile's columns while the tile is in flight: thread
  // (gp, col) adds its partials in leaf order, thread (0, col) the GP group
  // sums in order
  auto take_alpha = [&]() {
    if constexpr (UPD) {
      const int col = pcol;
      const size_t idx = (size_t)it.s * G.nrhs + c0 + col;
      pq_red[tid] = bs_strided_sum(up.pq + (size_t)it.s * G.K * G.nrhs + c0 + col, G.K, G.nrhs, gp, GP);
      __syncthreads();
      if (gp == 0) {
        double pq = pq_red[col];
#pragma unroll
        for (int k = 1; k < GP; ++k) pq += pq_red[k * BW + col];
        ColState st;
        st.rz = rz_col;
        st.status = st_col;
        st.iters = it_col;
        bs_step_pq(st, pq);
        alpha_s[col] = st.alpha;
        if (it.k == 0 && leaf_role) {
          up.cs[idx].alpha = st.alpha;
          up.cs[idx].rz_prev = st.rz_prev;
          up.cs[idx].iters = st.iters;
          up.cs[idx].status_pq = st.status_pq;
        }
      }
      __syncthreads();
#pragma unroll
      for (int v = 0; v < 4; ++v) al[v] = alpha_s[4 * (tid % C4) + v];
    }
  };
  // every load so far has landed; the UPD update of the R tile, the columns'
  // exponents and the R^T pairs
  auto wait_update = [&]() {
    lds_dma_wait();
    stamp(wgi, 1);
    if constexpr (UPD) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + BNT * i, row = c / C4;
        mf4 v = *reinterpret_cast<const mf4*>(&Rs[4 * c]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (al[t] != 0.0) v[t] = (float)((double)v[t] - al[t] * (double)ap[i][t]);
          rr4[t] = fma((double)v[t], (double)v[t], rr4[t]);
        }
        *reinterpret_cast<mf4*>(&Rs[4 * c]) = v;
        if (leaf_role) *reinterpret_cast<mf4*>(up.R + (size_t)(it.leaf0 + row) * G.nrhs + cc) = v;
      }
      if (leaf_role) {
        // R.R partials of the wave (fixed butterfly); summed over the waves at the end
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int o = C4; o < 64; o <<= 1) rr4[t] += __shfl_xor(rr4[t], o);
        }
        if (lane < C4) {
#pragma unroll
          for (int t = 0; t < 4; ++t) red[w * BW + 4 * lane + t] = rr4[t];
        }
      }
    }
    __syncthreads();                 // the whole tile in LDS (and updated)
    // the R^T pairs, a column pass: thread t takes column t % BW and the RPT
    // rows of row group t / BW; the column's exponent from its largest
    // magnitude over the row groups; eight pairs per 16-byte store
    constexpr int RG = BNT / BW, RPT = LEAF / RG;
    const int col = tid % BW, rg = tid / BW;
    float v[RPT];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      v[i] = Rs[(rg * RPT + i) * BW + col];
      m = fmaxf(m, fabsf(v[i]));
    }
    cmax[rg * BW + col] = m;
    __syncthreads();
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) m = fmaxf(m, cmax[g2 * BW + col]);
    const int e = pair_exponent(m);
    if (rg == 0) eR[col] = e;
#pragma unroll
    for (int c8 = 0; c8 < RPT / 8; ++c8) {
      h8 hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 a, b;
        to_pair(v[8 * c8 + i], e, a, b);
        hi[i] = a;
        lo[i] = b;
      }
      *reinterpret_cast<h8*>(&Rth[col * RT_STRIDE + rg * RPT + 8 * c8]) = hi;
      *reinterpret_cast<h8*>(&Rtl[col * RT_STRIDE + rg * RPT + 8 * c8]) = lo;
    }
    __syncthreads();
    stamp(wgi, 2);
  };
  // the R^T pair operands of tile j: step s covers rows 32 s + 8 q .. + 7
  auto load_b = [&](int j, h8 (&bh)[4], h8 (&bl)[4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bh[st] = *reinterpret_cast<const h8*>(&Rth[(16 * j + r) * RT_STRIDE + 32 * st + 8 * q]);
      bl[st] = *reinterpret_cast<const h8*>(&Rtl[(16 * j + r) * RT_STRIDE + 32 * st + 8 * q]);
    }
  };
  // restriction Q_l = W_l[k]^T R_k.  SPLIT: tiles outer, the wave's levels
  // inner (a tile's R operands are read once); in one workgroup levels outer,
  // the next level's operands issued here and not hoisted.
  auto restrict_one = [&](int b, int l, int j, const h8 (&bh)[4], const h8 (&bl)[4]) {
    mf4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = mfma_pair(wt_h[b][st], wt_l[b][st], bh[st], bl[st], acc);
    const float sc = ldexpf(1.f, -(eW[b] + eR[16 * j + r]));
    float* Qo = Q + q_index(G, it.s, l, it.k, 16 * mt + 4 * q) + c0 + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) Qo[(size_t)v * G.nrhs + 16 * j] = acc[v] * sc;
  };
  auto restriction = [&]() {
    if constexpr (SPLIT) {
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        h8 bh[4], bl[4];
        load_b(j, bh, bl);
#pragma unroll
        for (int i = 0; i < WL; ++i) {
          const int l = par + 2 * i;
          if (l >= LEV) break;
          restrict_one(i, l, j, bh, bl);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int l = par + 2 * i;
        if (l >= LEV) break;
        asm volatile("" ::: "memory");
        if (l + 2 < LEV) load_slot((i + 1) & 1, l + 2);
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          h8 bh[4], bl[4];
          load_b(j, bh, bl);
          restrict_one(i & 1, l, j, bh, bl);
        }
      }
    }
    stamp(wgi, 4);
  };
  // Y = F_k R_k + g R: this wave's rows [32w, 32w + 32), tile by tile
  auto leaf_stage = [&]() {
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      h8 bh[4], bl[4];
      load_b(j, bh, bl);
      mf4 ya = {0, 0, 0, 0}, yb = {0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        ya = mfma_pair(fa_h[st], fa_l[st], bh[st], bl[st], ya);
        yb = mfma_pair(fb_h[st], fb_l[st], bh[st], bl[st], yb);
      }
      const float sc = ldexpf(1.f, -(eF + eR[16 * j + r]));
      const int cj = c0 + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ia = 32 * w + 4 * q + v, ib = ia + 16;
        Y[(size_t)(it.leaf0 + ia) * G.nrhs + cj] = ya[v] * sc + gv[v] * Rs[ia * BW + 16 * j + r];
        Y[(size_t)(it.leaf0 + ib) * G.nrhs + cj] = yb[v] * sc + gv[4 + v] * Rs[ib * BW + 16 * j + r];
      }
    }
    stamp(wgi, 6);
  };
  if (SPLIT && role == 1) {        // the restriction alone
    load_restr();
    take_alpha();
    wait_update();
    restriction();
    return;
  }
  load_leaf();
  if constexpr (!SPLIT) load_restr();
  take_alpha();
  wait_update();
  leaf_stage();
  if constexpr (!SPLIT) restriction();
  if constexpr (UPD) {
    // R.R partials: the four waves' sums (left in red by the update) in order
    if (tid < BW)
      up.rr[((size_t)it.s * G.K + it.k) * G.nrhs + c0 + tid] =
          ((red[tid] + red[BW + tid]) + red[2 * BW + tid]) + red[3 * BW + tid];
  }
}

// (2) half sums: H_l[h] = sum of Q_l[k] over the 2^l leaves k of half h, for
// levels 1 and up (a level-0 half is one leaf: the prolongation reads its Q_0
// itself).  Same layout as Q (half index in place of the leaf index).  A
// thread adds a run of at most eight consecutive leaves (its loads all in
// flight at once, added in leaf order); the P = 2^l / 8 runs of a half's
// element sit in one wave, 64 / P lanes apart, and are combined pairwise in
// leaf order, adjacent runs first (a fixed tree: one order, every call).  A level's threads come in whole
// waves (RANK * nrhs is a multiple of 64).
// Grid: x over a system's (level, half, element, run) quadruples, y over the
// systems (a stride of gridDim.y past 65535 systems); the index arithmetic is
// 32-bit (a system's quadruples are far fewer than 2^31).
constexpr int HS_RUN = 8;
__host__ __device__ inline unsigned halfsum_runs(int l) { return (1 << l) > HS_RUN ? (1u << l) / HS_RUN : 1u; }
__global__ __launch_bounds__(256) void k_block_halfsum(BlockGeom G, const float* __restrict__ Q,
                                                       float* __restrict__ H) {
  const unsigned per = (unsigned)RANK * (unsigned)G.nrhs;   // elements per (level, leaf)
  unsigned rem = blockIdx.x * blockDim.x + threadIdx.x;
  int l = 1;
  unsigned level_threads = (unsigned)(G.K >> 1) * per;   // l = 1: one run per element
  while (l < G.levels && rem >= level_threads) {
    rem -= level_threads;
    ++l;
    level_threads = (unsigned)(G.K >> l) * per * halfsum_runs(l);
  }
  if (l >= G.levels) return;                       // whole waves
  const int span = 1 << l;
  const unsigned P = halfsum_runs(l), gap = 64u / P, lane = threadIdx.x & 63u;
  const int n = span / (int)P;                     // leaves of a run, at most HS_RUN
  const unsigned idx = (rem / 64u) * gap + lane % gap, run = lane / gap;
  const unsigned h = idx / per, e = idx - h * per;
  for (int s = (int)blockIdx.y; s < G.B; s += (int)gridDim.y) {
    const float* src = Q + q_index(G, s, l, (int)h * span + (int)run * n, 0) + e;
    float v[HS_RUN];
#pragma unroll
    for (int u = 0; u < HS_RUN; ++u) v[u] = u < n ? src[(size_t)u * per] : 0.f;
    float a = v[0];
#pragma unroll
    for (int u = 1; u < HS_RUN; ++u)
      if (u < n) a += v[u];
    for (unsigned o = gap; o < 64u; o <<= 1) a += __shfl_xor(a, (int)o);
    if (run == 0) H[q_index(G, s, l, (int)h, 0) + e] = a;
  }
}

// (3) prolongation: Y_k += sum_l W_l[k] H_l[(k >> l) ^ 1] as fp16-pair products
// (the slab rows held as pairs with the slab's exponent, the partner half sums
// as pairs with one exponent per (level, column), taken from the largest of the
// column's 32 values).  The levels run in two stages: the first stage's
// products while the second stage's operands are still arriving; the products
// keep level order.
constexpr int PH_STRIDE = 40;   // half-sum pair rows in LDS, halfs (80 B)
template <int LEV, int NCT, bool DOT = false>
__global__ __launch_bounds__(BNT) void k_block_prolong(BlockGeom G, BlockFactors16 fw,
                                                       const float* __restrict__ Q, const float* __restrict__ H,
                                                       float* __restrict__ Y, BlockDot dt) {
  constexpr int BW = BNC * NCT;
  constexpr int NL = LEV > 0 ? LEV : 1;
  constexpr int NS = (NL + 1) / 2;                                             // levels of a stage, at most
  __shared__ float Hs[NS * RANK * BW];                                         // [l - l0][rank][col]
  __shared__ __attribute__((aligned(16))) _Float16 Phh[NL * BW * PH_STRIDE];   // [l][col][rank]
  __shared__ __attribute__((aligned(16))) _Float16 Phl[NL * BW * PH_STRIDE];
  __shared__ int eH[NL * BW];                                                  // exponent per (l, col)
  __shared__ double red[DOT ? NWAVE * BW : 1];
  const BItem it = bitem(G);
  stamp((int)blockIdx.x, 8);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  constexpr int LA = (LEV + 1) / 2, LB = LEV - LA;
  constexpr int PE = RANK * BW / BNT;        // half-sum elements per thread and level
  // slab rows 32w + r (a) and 32w + 16 + r (b), rank 8q .. 8q + 7
  h8 wa_h[NL], wa_l[NL], wb_h[NL], wb_l[NL];
  int eW[NL];
  auto load_w = [&](int l0, int l1) {
#pragma unroll
    for (int l = l0; l < l1; ++l) {
      const size_t slab = ((size_t)it.s * LEV + l) * G.K + it.k;
      const size_t o = slab * LEAF * RANK + (size_t)(32 * w + r) * RANK + 8 * q;
      wa_h[l] = *reinterpret_cast<const h8*>(fw.Wh + o);
      wa_l[l] = *reinterpret_cast<const h8*>(fw.Wl + o);
      wb_h[l] = *reinterpret_cast<const h8*>(fw.Wh + o + 16 * RANK);
      wb_l[l] = *reinterpret_cast<const h8*>(fw.Wl + o + 16 * RANK);
      eW[l] = fw.We[slab];
    }
  };
  auto load_h = [&](float* hv, int l0, int nl) {
#pragma unroll
    for (int u = 0; u < nl * PE; ++u) {
      const int e = tid + u * BNT;
      const int l = l0 + e / (RANK * BW), rem = e % (RANK * BW);
      const int row = rem / BW, col = rem - row * BW;
      // level 0's halves are single leaves: the partner's restriction itself
      hv[u] = (l == 0 ? Q : H)[q_index(G, it.s, l, (it.k >> l) ^ 1, row) + c0 + col];
    }
  };
  // levels [l0, l0 + nl): the half sums into LDS as they are laid out (fp32;
  // the two stages take turns in one buffer), then a column pass: a thread per
  // (level, column), its 32 values' exponent and their pairs, eight per
  // 16-byte store
  auto stage_h = [&](const float* hv, int l0, int nl) {
#pragma unroll
    for (int u = 0; u < nl * PE; ++u) Hs[tid + u * BNT] = hv[u];
  };
  auto pair_h = [&](int l0, int nl) {
    for (int p = tid; p < nl * BW; p += BNT) {
      const int l = l0 + p / BW, col = p % BW;
      float v[RANK];
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < RANK; ++i) {
        v[i] = Hs[((l - l0) * RANK + i) * BW + col];
        m = fmaxf(m, fabsf(v[i]));
      }
      const int e = pair_exponent(m);
      eH[l * BW + col] = e;
#pragma unroll
      for (int c8 = 0; c8 < RANK / 8; ++c8) {
        h8 hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          _Float16 a, b;
          to_pair(v[8 * c8 + i], e, a, b);
          hi[i] = a;
          lo[i] = b;
        }
        *reinterpret_cast<h8*>(&Phh[(l * BW + col) * PH_STRIDE + 8 * c8]) = hi;
        *reinterpret_cast<h8*>(&Phl[(l * BW + col) * PH_STRIDE + 8 * c8]) = lo;
      }
    }
  };
  // accumulators start from the leaf stage's Y
  mf4 ya[NCT], yb[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ya[j][v] = Y[(size_t)(it.leaf0 + 32 * w + 4 * q + v) * G.nrhs + c0 + 16 * j + r];
      yb[j][v] = Y[(size_t)(it.leaf0 + 32 * w + 16 + 4 * q + v) * G.nrhs + c0 + 16 * j + r];
    }
  }
  auto products = [&](int l0, int l1) {
#pragma unroll
    for (int l = l0; l < l1; ++l) {
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int col = 16 * j + r;
        const h8 bh = *reinterpret_cast<const h8*>(&Phh[(l * BW + col) * PH_STRIDE + 8 * q]);
        const h8 bl = *reinterpret_cast<const h8*>(&Phl[(l * BW + col) * PH_STRIDE + 8 * q]);
        const mf4 z = {0, 0, 0, 0};
        const mf4 pa = mfma_pair(wa_h[l], wa_l[l], bh, bl, z);
        const mf4 pb = mfma_pair(wb_h[l], wb_l[l], bh, bl, z);
        const float sc = ldexpf(1.f, -(eW[l] + eH[l * BW + col]));
        ya[j] += pa * sc;
        yb[j] += pb * sc;
      }
    }
  };
  float ha[LA * PE], hb[LB > 0 ? LB * PE : 1];
  load_w(0, LA);
  load_h(ha, 0, LA);
  load_w(LA, LEV);
  if constexpr (LB > 0) load_h(hb, LA, LB);
  // DOT: R at the lane's accumulator elements
  float rv[DOT ? NCT : 1][8];
  if constexpr (DOT) {
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        rv[j][v] = dt.R[(size_t)(it.leaf0 + 32 * w + 4 * q + v) * G.nrhs + c0 + 16 * j + r];
        rv[j][4 + v] = dt.R[(size_t)(it.leaf0 + 32 * w + 16 + 4 * q + v) * G.nrhs + c0 + 16 * j + r];
      }
    }
  }
  stage_h(ha, 0, LA);
  __syncthreads();
  pair_h(0, LA);
  __syncthreads();
  stamp((int)blockIdx.x, 9);
  products(0, LA);
  if constexpr (LB > 0) {
    stage_h(hb, LA, LB);
    __syncthreads();
    pair_h(LA, LB);
    __syncthreads();
    products(LA, LEV);
  }
  stamp((int)blockIdx.x, 10);
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      Y[(size_t)(it.leaf0 + 32 * w + 4 * q + v) * G.nrhs + c0 + 16 * j + r] = ya[j][v];
      Y[(size_t)(it.leaf0 + 32 * w + 16 + 4 * q + v) * G.nrhs + c0 + 16 * j + r] = yb[j][v];
    }
  }
  stamp((int)blockIdx.x, 11);
  if constexpr (DOT) {
    // R.Z partials: the lane's eight rows, then the four lane groups q (fixed
    // butterfly), then the four waves in order
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      double d = 0.0;
#pragma unroll
      for (int v = 0; v < 4; ++v) d = fma((double)rv[j][v], (double)ya[j][v], d);
#pragma unroll
      for (int v = 0; v < 4; ++v) d = fma((double)rv[j][4 + v], (double)yb[j][v], d);
      d += __shfl_xor(d, 16);
      d += __shfl_xor(d, 32);
      if (q == 0) red[w * BW + 16 * j + r] = d;
    }
    __syncthreads();
    if (tid < BW)
      dt.rz[((size_t)it.s * G.K + it.k) * G.nrhs + c0 + tid] =
          ((red[tid] + red[BW + tid]) + red[2 * BW + tid]) + red[3 * BW + tid];
  }
}

// Block SpMV: thread = (row, 4 consecutive columns).
__global__ __launch_bounds__(256) void k_spmv_block(const int* __restrict__ row_ptr, const int* __restrict__ col,
                                                    const float* __restrict__ val, const float* __restrict__ X,
                                                    float* __restrict__ Y, int nrows, int nrhs) {
  const int groups = nrhs / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / groups);
  if (row >= nrows) return;
  const int c4 = (int)(idx - (size_t)row * groups) * 4;
  mf4 acc = {0, 0, 0, 0};
  const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  // four entries per round: their indices, then their X rows, are all in
  // flight together; the entries past the row's end are skipped
  for (int e = e0; e < e1; e += 4) {
    int c[4];
    float a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = e + u < e1;
      c[u] = in ? col[e + u] : row;
      a[u] = in ? val[e + u] : 0.f;
    }
    mf4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const mf4*>(X + (size_t)c[u] * nrhs + c4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (e + u < e1) {
        acc.x = fmaf(a[u], x[u].x, acc.x);
        acc.y = fmaf(a[u], x[u].y, acc.y);
        acc.z = fmaf(a[u], x[u].z, acc.z);
        acc.w = fmaf(a[u], x[u].w, acc.w);
      }
    }
  }
  *reinterpret_cast<mf4*>(Y + (size_t)row * nrhs + c4) = acc;
}

}  // namespace hpcg
