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
// (two where nrhs is a multiple of 32, so that each factor operand it loads
// feeds twice the products).
// Products use v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).  Lane l of a
// wave supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// D[4 (l / 16) + v][l % 16], v = 0..3.  Where an operand is read along the
// contraction index from memory that is contiguous in it, a lane reads four
// consecutive k with one 16-byte load and feeds them to four MFMAs (lane group
// q = l / 16 contracts k0 + 4q + t in MFMA t); A and B use the same order, so
// the sum is the same product.
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
#include "hpcg_device.hpp"

namespace hpcg {

constexpr int BNC = 16;          // right-hand-side columns per workgroup
constexpr int BNT = 256;         // threads per workgroup
constexpr int TS_STRIDE = 132;   // R^T rows in LDS (== 4 mod 64: conflict-free 16-byte reads)
constexpr int PS_STRIDE = 36;    // P^T rows in LDS (== 36 mod 64: conflict-free 16-byte reads)

typedef float mf4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mf4 mfma4(float a, float b, mf4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

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
// (UPD): R <- R - alpha_c (A P) column by column, in fp64 and rounded to fp32
// once, a column whose alpha is 0 keeping its R; the new R is written back and
// the apply runs on it, and the workgroup leaves its (system, leaf, column)
// partials of the new R . R.
struct BlockUpd {
  const double* alpha;   // alpha of (system s, column c) at alpha[(s nrhs + c) stride]
  int stride;
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
// fp64 over the leaf's 128 columns in column order and rounded to fp32 once
// (F_k is then exactly symmetric).  One workgroup per leaf; U_k is staged in
// LDS with rows padded to 129 words, so the lanes' walks down a column hit
// distinct banks.  Thread t owns row t % 128 of half t / 128 of the columns and
// writes them as column entries (F_k is symmetric), coalesced across lanes.
__global__ __launch_bounds__(BNT) void k_leaf_blocks(const float* __restrict__ U, float* __restrict__ F) {
  constexpr int PAD = LEAF + 1;
  __shared__ float Us[LEAF * PAD];
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
  float* Fk = F + leaf * LEAF * LEAF;
#pragma unroll
  for (int jj = 0; jj < LEAF / 2; ++jj) Fk[(size_t)(j0 + jj) * LEAF + i] = (float)acc[jj];
}

// (1) leaf stage, gate and restriction: Y = F_k R_k + g R (F_k = U_k U_k^T,
// k_leaf_blocks) and Q_l = W_l[k]^T R_k.  All global operand loads of a stage
// are issued before its products.  A workgroup owns NCT 16-column tiles (BW =
// 16 NCT columns): every F_k and W_l[k] operand it loads feeds the MFMAs of all
// NCT tiles.  R is only read through the DMA into LDS, before any write of the
// UPD update; the leaf stage reads it through a transposed copy (Ts), where a
// lane's four contraction steps of one MFMA group are one 16-byte read.  SPLIT
// runs the leaf stage (role 0) and the restriction (role 1) of an item in two
// workgroups, each with its own copy of the R tile (both take the UPD update,
// the same arithmetic; role 0 writes it back and leaves the partials).  With
// SPLIT, role 1 loads the operands of all its levels at once; in one workgroup
// the levels' operands are double-buffered (a level's loads are issued a level
// ahead).  At most 256 VGPRs (two waves per SIMD), so that two workgroups share
// a compute unit.
template <int LEV, int NCT, bool UPD = false, bool SPLIT = false>
__global__ __launch_bounds__(BNT, 2) void k_block_restrict(BlockGeom G, const float* __restrict__ F,
                                                           const float* __restrict__ W, const float* __restrict__ g,
                                                           const float* R, float* __restrict__ Y,
                                                           float* __restrict__ Q, BlockUpd up) {
  constexpr int BW = BNC * NCT;
  constexpr int C4 = BW / 4;                 // 16-byte chunks per tile row
  constexpr int CH = LEAF * C4 / BNT;        // chunks of the tile per thread
  constexpr int WL = (LEV + 1) / 2;          // levels of a wave, at most
  __shared__ __attribute__((aligned(16))) float Rs[LEAF * BW];          // R_k tile, [row][BW]
  __shared__ __attribute__((aligned(16))) float Ts[BW * TS_STRIDE];     // R_k^T, [col][row]
  __shared__ double red[UPD ? NWAVE * BW : 1];
  int role = 0;
  const BItem it = SPLIT ? bitem2(G, role) : bitem(G);
  const bool leaf_role = !SPLIT || role == 0;      // leaf stage, gate, write-back
  const int wgi = (int)blockIdx.x;
  stamp(wgi, 0);
  stamp_value(wgi, 7, (unsigned long long)(SPLIT ? role : 2));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  const float* Fk = F + ((size_t)it.s * G.K + it.k) * LEAF * LEAF;
  // restriction work of this wave: rank tile (w & 1) of levels par, par + 2, ...
  const int mt = w & 1, par = w >> 1;
  auto wlev = [&](int l) {
    return W + (((size_t)it.s * LEV + l) * G.K + it.k) * LEAF * RANK + 16 * mt + r;
  };
  auto load_level = [&](float (&dst)[32], int l) {
    const float* Wl = wlev(l);
#pragma unroll
    for (int s = 0; s < 32; ++s) dst[s] = Wl[(size_t)(4 * s + q) * RANK];
  };
  // leaf-stage A operands: rows 32w + r and 32w + 16 + r of F_k, columns
  // 16 ch + 4 q .. + 3 (MFMA t of group ch contracts k = 16 ch + 4 q + t), and
  // the gate at the lane's rows of Y
  mf4 af[LEAF / 16], bf[LEAF / 16];
  float gv[8];
  auto load_leaf = [&]() {
    const float* Fa = Fk + (size_t)(32 * w + r) * LEAF + 4 * q;
    const float* Fb = Fa + 16 * LEAF;
#pragma unroll
    for (int ch = 0; ch < LEAF / 16; ++ch) {
      af[ch] = *reinterpret_cast<const mf4*>(Fa + 16 * ch);
      bf[ch] = *reinterpret_cast<const mf4*>(Fb + 16 * ch);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      gv[v] = g[it.leaf0 + 32 * w + 4 * q + v];
      gv[4 + v] = g[it.leaf0 + 32 * w + 16 + 4 * q + v];
    }
  };
  float wv[SPLIT ? WL : 2][32];
  auto load_restr = [&]() {
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < WL; ++i)
        if (par + 2 * i < LEV) load_level(wv[i], par + 2 * i);
    } else {
      if (par < LEV) load_level(wv[0], par);
    }
  };
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
    for (int v = 0; v < 4; ++v) al[v] = up.alpha[((size_t)it.s * G.nrhs + cc + v) * up.stride];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + BNT * i) / C4;
      ap[i] = *reinterpret_cast<const mf4*>(up.AP + (size_t)(it.leaf0 + row) * G.nrhs + cc);
    }
  }
  // every load so far has landed; the UPD update of the R tile and, for the
  // leaf stage, the transposed copy
  auto wait_update = [&](bool transpose) {
    lds_dma_wait();
    stamp(wgi, 1);
    if (UPD || transpose) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + BNT * i, row = c / C4, col = 4 * (c % C4);
        mf4 v = *reinterpret_cast<const mf4*>(&Rs[4 * c]);
        if constexpr (UPD) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (al[t] != 0.0) v[t] = (float)((double)v[t] - al[t] * (double)ap[i][t]);
            rr4[t] = fma((double)v[t], (double)v[t], rr4[t]);
          }
          *reinterpret_cast<mf4*>(&Rs[4 * c]) = v;
          if (leaf_role) *reinterpret_cast<mf4*>(up.R + (size_t)(it.leaf0 + row) * G.nrhs + cc) = v;
        }
        if (transpose) {
#pragma unroll
          for (int t = 0; t < 4; ++t) Ts[(col + t) * TS_STRIDE + row] = v[t];
        }
      }
      if (UPD && leaf_role) {
        // R.R partials of the wave: lanes with the same columns differ in lane
        // bits >= log2(C4) (fixed butterfly); summed over the waves at the end
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
      __syncthreads();
    }
    stamp(wgi, 2);
  };
  // restriction Q_l = W_l[k]^T R_k, two accumulation chains (even / odd k
  // steps) summed at the end.  SPLIT: every level's operands are in registers,
  // so the tiles are the outer loop and a tile's R operands are read once.
  auto restriction = [&]() {
    if constexpr (SPLIT) {
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        float rv[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) rv[s] = Rs[(4 * s + q) * BW + 16 * j + r];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < WL; ++i) {
          const int l = par + 2 * i;
          if (l >= LEV) break;
          mf4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < 32; s += 2) {
            a0 = mfma4(wv[i][s], rv[s], a0);
            a1 = mfma4(wv[i][s + 1], rv[s + 1], a1);
          }
          const mf4 acc = a0 + a1;
          float* Qo = Q + q_index(G, it.s, l, it.k, 16 * mt + 4 * q) + c0 + r;
#pragma unroll
          for (int v = 0; v < 4; ++v) Qo[(size_t)v * G.nrhs + 16 * j] = acc[v];
        }
      }
      stamp(wgi, 4);
      return;
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int l = par + 2 * i;
      if (l >= LEV) break;
      // the level two ahead, issued here and not hoisted (that would hold
      // every level's operands at once)
      asm volatile("" ::: "memory");
      if (l + 2 < LEV) load_level(wv[(i + 1) & 1], l + 2);
      const float(&wa)[32] = wv[i & 1];
      float* Qo = Q + q_index(G, it.s, l, it.k, 16 * mt + 4 * q) + c0 + r;
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        float rv[32];
#pragma unroll
        for (int s = 0; s < 32; ++s) rv[s] = Rs[(4 * s + q) * BW + 16 * j + r];
        __builtin_amdgcn_sched_barrier(0);
        mf4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 32; s += 2) {
          a0 = mfma4(wa[s], rv[s], a0);
          a1 = mfma4(wa[s + 1], rv[s + 1], a1);
        }
        const mf4 acc = a0 + a1;
#pragma unroll
        for (int v = 0; v < 4; ++v) Qo[(size_t)v * G.nrhs + 16 * j] = acc[v];
      }
    }
    stamp(wgi, 4);
  };
  // Y = F_k R_k + g R: this wave's rows [32w, 32w + 32), tile by tile
  auto leaf_stage = [&]() {
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      mf4 ya = {0, 0, 0, 0}, yb = {0, 0, 0, 0};
      mf4 bt[LEAF / 16];           // the tile's R^T operands, read ahead of the products
#pragma unroll
      for (int ch = 0; ch < LEAF / 16; ++ch)
        bt[ch] = *reinterpret_cast<const mf4*>(&Ts[(16 * j + r) * TS_STRIDE + 16 * ch + 4 * q]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ch = 0; ch < LEAF / 16; ++ch) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ya = mfma4(af[ch][t], bt[ch][t], ya);
          yb = mfma4(bf[ch][t], bt[ch][t], yb);
        }
      }
      const int cj = c0 + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ia = 32 * w + 4 * q + v, ib = ia + 16;
        Y[(size_t)(it.leaf0 + ia) * G.nrhs + cj] = ya[v] + gv[v] * Rs[ia * BW + 16 * j + r];
        Y[(size_t)(it.leaf0 + ib) * G.nrhs + cj] = yb[v] + gv[4 + v] * Rs[ib * BW + 16 * j + r];
      }
    }
    stamp(wgi, 6);
  };
  if (SPLIT && role == 1) {        // the restriction alone: its operands of every level at once
    load_restr();
    wait_update(false);
    restriction();
    return;
  }
  load_leaf();
  if constexpr (!SPLIT) load_restr();
  wait_update(true);
  leaf_stage();
  if constexpr (!SPLIT) restriction();
  if constexpr (UPD) {
    // R.R partials: the four waves' sums (left in red by the update) in order
    if (tid < BW)
      up.rr[((size_t)it.s * G.K + it.k) * G.nrhs + c0 + tid] =
          ((red[tid] + red[BW + tid]) + red[2 * BW + tid]) + red[3 * BW + tid];
  }
}

// (2) half sums: H_l[h] = sum of Q_l[k] over the 2^l leaves k of half h, summed
// in leaf order.  Same layout as Q (half index in place of the leaf index).
// Grid: x over a system's (level, half, element) triples, y over the systems
// (a stride of gridDim.y past 65535 systems); the index arithmetic is 32-bit
// (a system's triples are far fewer than 2^31).
__global__ void k_block_halfsum(BlockGeom G, const float* __restrict__ Q, float* __restrict__ H) {
  constexpr int HB = 8;                            // loads in flight per batch
  const unsigned per = (unsigned)RANK * (unsigned)G.nrhs;   // elements per (level, leaf)
  unsigned rem = blockIdx.x * blockDim.x + threadIdx.x;
  int l = 0;
  unsigned level_elems = (unsigned)G.K * per;      // l = 0
  while (l < G.levels && rem >= level_elems) {
    rem -= level_elems;
    ++l;
    level_elems = (unsigned)(G.K >> l) * per;
  }
  if (l >= G.levels) return;
  const unsigned h = rem / per, e = rem - h * per;
  const int span = 1 << l;
  for (int s = (int)blockIdx.y; s < G.B; s += (int)gridDim.y) {
    const float* src = Q + q_index(G, s, l, (int)h * span, 0) + e;
    // the sum keeps leaf order
    float a = 0.f;
    int i = 0;
    for (; i + HB <= span; i += HB) {
      float v[HB];
#pragma unroll
      for (int u = 0; u < HB; ++u) v[u] = src[(size_t)(i + u) * per];
#pragma unroll
      for (int u = 0; u < HB; ++u) a += v[u];
    }
    for (; i < span; ++i) a += src[(size_t)i * per];
    H[q_index(G, s, l, (int)h, 0) + e] = a;
  }
}

// (3) prolongation: Y_k += sum_l W_l[k] H_l[(k >> l) ^ 1].  Every level's slab
// rows are loaded in one batch up front and feed the MFMAs of all NCT tiles.
template <int LEV, int NCT, bool DOT = false>
__global__ __launch_bounds__(BNT) void k_block_prolong(BlockGeom G, const float* __restrict__ W,
                                                       const float* __restrict__ H, float* __restrict__ Y,
                                                       BlockDot dt) {
  constexpr int BW = BNC * NCT;
  __shared__ __attribute__((aligned(16))) float Ps[(LEV > 0 ? LEV : 1) * BW * PS_STRIDE];   // [l][col][rank]
  __shared__ double red[DOT ? NWAVE * BW : 1];
  const BItem it = bitem(G);
  stamp((int)blockIdx.x, 8);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  // two stages of levels: the first stage's products run while the second
  // stage's operands are still arriving; the products keep level order
  constexpr int LA = (LEV + 1) / 2, LB = LEV - LA;
  constexpr int PE = RANK * BW / BNT;        // half-sum elements per thread and level
  mf4 aw[LEV > 0 ? LEV : 1][2], bw[LEV > 0 ? LEV : 1][2];
  auto load_w = [&](int l0, int l1) {
#pragma unroll
    for (int l = l0; l < l1; ++l) {
      const float* Wa = W + ((((size_t)it.s * LEV + l) * G.K + it.k) * LEAF + 32 * w + r) * RANK + 4 * q;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        aw[l][ch] = *reinterpret_cast<const mf4*>(Wa + 16 * ch);
        bw[l][ch] = *reinterpret_cast<const mf4*>(Wa + 16 * RANK + 16 * ch);
      }
    }
  };
  // partner half sums of levels [l0, l0 + NL): loads, then their transposed
  // stores into LDS
  auto load_h = [&](float* hv, int l0, int nl) {
#pragma unroll
    for (int u = 0; u < nl * PE; ++u) {
      const int e = tid + u * BNT;
      const int l = l0 + e / (RANK * BW), rem = e % (RANK * BW);
      const int row = rem / BW, col = rem - row * BW;
      hv[u] = H[q_index(G, it.s, l, (it.k >> l) ^ 1, row) + c0 + col];
    }
  };
  auto store_h = [&](const float* hv, int l0, int nl) {
#pragma unroll
    for (int u = 0; u < nl * PE; ++u) {
      const int e = tid + u * BNT;
      const int l = l0 + e / (RANK * BW), rem = e % (RANK * BW);
      const int row = rem / BW, col = rem - row * BW;
      Ps[(l * BW + col) * PS_STRIDE + row] = hv[u];
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
      for (int ch = 0; ch < RANK / 16; ++ch) {
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          const mf4 bp = *reinterpret_cast<const mf4*>(&Ps[(l * BW + 16 * j + r) * PS_STRIDE + 16 * ch + 4 * q]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            ya[j] = mfma4(aw[l][ch][t], bp[t], ya[j]);
            yb[j] = mfma4(bw[l][ch][t], bp[t], yb[j]);
          }
        }
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
  store_h(ha, 0, LA);
  __syncthreads();
  stamp((int)blockIdx.x, 9);
  products(0, LA);
  if constexpr (LB > 0) {
    store_h(hb, LA, LB);
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
