// Block (multi-right-hand-side) apply Y = M R and block SpMV Y = A X on gfx950
// matrix cores.
//
// With a block of right-hand sides every stage of the apply is a real GEMM: the
// leaf stage is U_k (U_k^T R_k) with R_k of 128 x nrhs, the restriction
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
// Three launches: (1) per (leaf, tile): T = U_k^T R_k, Y = U_k T + g R, and the
// per-leaf restrictions Q_l[k] = W_l[k]^T R_k; (2) per (level, half, element):
// the half sums of Q_l over every tile half (eq. (3)), in a fixed order; (3) per
// (leaf, tile): Y += sum_l W_l[k] P_l with P_l the partner half's sum (eqs.
// (4)-(5), identity core).
#pragma once
#include "hpcg_device.hpp"

namespace hpcg {

constexpr int BNC = 16;          // right-hand-side columns per workgroup
constexpr int BNT = 256;         // threads per workgroup
constexpr int TS_STRIDE = 132;   // T^T rows in LDS (== 4 mod 64: conflict-free 16-byte reads)
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

// Q layout: [B][levels][K][RANK][nrhs].
__device__ __forceinline__ size_t q_index(const BlockGeom& G, int s, int l, int k, int row) {
  return ((((size_t)s * G.levels + l) * G.K + k) * RANK + row) * G.nrhs;
}

// (1) leaf stage, gate and restriction.  All global operand loads of a stage
// are issued before its products, and the next level's before this level's.
// A workgroup owns NCT 16-column tiles (BW = 16 NCT columns): every U_k and
// W_l[k] operand it loads feeds the MFMAs of all NCT tiles.
template <int LEV, int NCT>
__global__ __launch_bounds__(BNT) void k_block_restrict(BlockGeom G, const float* __restrict__ U,
                                                        const float* __restrict__ W, const float* __restrict__ g,
                                                        const float* __restrict__ R, float* __restrict__ Y,
                                                        float* __restrict__ Q) {
  constexpr int BW = BNC * NCT;
  __shared__ __attribute__((aligned(16))) float Rs[LEAF * BW];          // R_k tile, [row][BW]
  __shared__ __attribute__((aligned(16))) float Ts[BW * TS_STRIDE];     // T^T, [col][row]
  const BItem it = bitem(G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  const float* Uk = U + ((size_t)it.s * G.K + it.k) * LEAF * LEAF;
  // restriction work of this wave: rank tile (w & 1) of levels (w >> 1), +2, ...
  const int mt = w & 1;
  auto wlev = [&](int l) {
    return W + (((size_t)it.s * LEV + l) * G.K + it.k) * LEAF * RANK + 16 * mt + r;
  };
  // R tile: 128 rows x 4 BW bytes, straight into LDS
  dma_to_lds(Rs, LEAF * BW / 4, [&](int c) {
    return R + (size_t)(it.leaf0 + c / (BW / 4)) * G.nrhs + c0 + 4 * (c % (BW / 4));
  });
  // GEMM 1 A operands: U[4s + q][32w + r] and U[4s + q][32w + 16 + r], s = 0..31
  float ua[32], ub[32], wa[32];
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const float* row = Uk + (size_t)(4 * s + q) * LEAF + 32 * w + r;
    ua[s] = row[0];
    ub[s] = row[16];
  }
  if (LEV > (w >> 1)) {
    const float* Wl = wlev(w >> 1);
#pragma unroll
    for (int s = 0; s < 32; ++s) wa[s] = Wl[(size_t)(4 * s + q) * RANK];
  }
  lds_dma_wait();
  // T = U_k^T R_k: this wave's rows [32w, 32w + 32) of T, for every tile
  mf4 ta[NCT], tb[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) ta[j] = tb[j] = mf4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 32; ++s) {
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const float bv = Rs[(4 * s + q) * BW + 16 * j + r];
      ta[j] = mfma4(ua[s], bv, ta[j]);
      tb[j] = mfma4(ub[s], bv, tb[j]);
    }
  }
  // T^T into LDS: lane holds T[32w + 4q + v][16j + r] (and + 16)
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    *reinterpret_cast<mf4*>(&Ts[(16 * j + r) * TS_STRIDE + 32 * w + 4 * q]) = ta[j];
    *reinterpret_cast<mf4*>(&Ts[(16 * j + r) * TS_STRIDE + 32 * w + 16 + 4 * q]) = tb[j];
  }
  // restriction Q_l = W_l[k]^T R_k, two accumulation chains (even / odd k
  // steps) summed at the end
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    if ((l & 1) != (w >> 1)) continue;
    float wn[32];
    if (l + 2 < LEV) {
      const float* Wn = wlev(l + 2);
#pragma unroll
      for (int s = 0; s < 32; ++s) wn[s] = Wn[(size_t)(4 * s + q) * RANK];
    }
    float* Qo = Q + q_index(G, it.s, l, it.k, 16 * mt + 4 * q) + c0 + r;
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      mf4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 32; s += 2) {
        a0 = mfma4(wa[s], Rs[(4 * s + q) * BW + 16 * j + r], a0);
        a1 = mfma4(wa[s + 1], Rs[(4 * s + 4 + q) * BW + 16 * j + r], a1);
      }
      const mf4 acc = a0 + a1;
#pragma unroll
      for (int v = 0; v < 4; ++v) Qo[(size_t)v * G.nrhs + 16 * j] = acc[v];
    }
    if (l + 2 < LEV) {
#pragma unroll
      for (int s = 0; s < 32; ++s) wa[s] = wn[s];
    }
  }
  // GEMM 2 operands: rows 32w + r and 32w + 16 + r of U_k (L2-resident by now)
  const float* Ua = Uk + (size_t)(32 * w + r) * LEAF + 4 * q;
  const float* Ub = Ua + 16 * LEAF;
  mf4 au[LEAF / 16], bu[LEAF / 16];
#pragma unroll
  for (int ch = 0; ch < LEAF / 16; ++ch) {
    au[ch] = *reinterpret_cast<const mf4*>(Ua + 16 * ch);
    bu[ch] = *reinterpret_cast<const mf4*>(Ub + 16 * ch);
  }
  __syncthreads();
  // Y = U_k T + g R: this wave's rows [32w, 32w + 32), tile by tile
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    mf4 ya = {0, 0, 0, 0}, yb = {0, 0, 0, 0};
#pragma unroll
    for (int ch = 0; ch < LEAF / 16; ++ch) {
      const mf4 bt = *reinterpret_cast<const mf4*>(&Ts[(16 * j + r) * TS_STRIDE + 16 * ch + 4 * q]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ya = mfma4(au[ch][t], bt[t], ya);
        yb = mfma4(bu[ch][t], bt[t], yb);
      }
    }
    const int cj = c0 + 16 * j + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ia = 32 * w + 4 * q + v, ib = ia + 16;
      Y[(size_t)(it.leaf0 + ia) * G.nrhs + cj] = ya[v] + g[it.leaf0 + ia] * Rs[ia * BW + 16 * j + r];
      Y[(size_t)(it.leaf0 + ib) * G.nrhs + cj] = yb[v] + g[it.leaf0 + ib] * Rs[ib * BW + 16 * j + r];
    }
  }
}

// (2) half sums: H_l[h] = sum of Q_l[k] over the 2^l leaves k of half h, summed
// in leaf order.  Same layout as Q (half index in place of the leaf index).
__global__ void k_block_halfsum(BlockGeom G, const float* __restrict__ Q, float* __restrict__ H) {
  const size_t per = (size_t)RANK * G.nrhs;       // elements per (level, leaf)
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // enumerate (s, l, h, e) with h < K >> l: level l owns (K >> l) * per elements
  size_t rem = idx;
  int l = 0;
  size_t level_elems = (size_t)G.K * per;         // l = 0
  size_t sys_total = 0;
  for (int ll = 0; ll < G.levels; ++ll) sys_total += (size_t)(G.K >> ll) * per;
  const int s = (int)(rem / sys_total);
  if (s >= G.B) return;
  rem -= (size_t)s * sys_total;
  while (l < G.levels && rem >= level_elems) {
    rem -= level_elems;
    ++l;
    level_elems = (size_t)(G.K >> l) * per;
  }
  if (l >= G.levels) return;
  const int h = (int)(rem / per);
  const size_t e = rem - (size_t)h * per;
  const int span = 1 << l;
  const float* src = Q + q_index(G, s, l, h * span, 0) + e;
  // loads in batches of 8 in flight; the sum keeps leaf order
  float a = 0.f;
  int i = 0;
  for (; i + 8 <= span; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(i + u) * per];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  for (; i < span; ++i) a += src[(size_t)i * per];
  H[q_index(G, s, l, h, 0) + e] = a;
}

// (3) prolongation: Y_k += sum_l W_l[k] H_l[(k >> l) ^ 1].  Every level's slab
// rows are loaded in one batch up front and feed the MFMAs of all NCT tiles.
template <int LEV, int NCT>
__global__ __launch_bounds__(BNT) void k_block_prolong(BlockGeom G, const float* __restrict__ W,
                                                       const float* __restrict__ H, float* __restrict__ Y) {
  constexpr int BW = BNC * NCT;
  __shared__ __attribute__((aligned(16))) float Ps[(LEV > 0 ? LEV : 1) * BW * PS_STRIDE];   // [l][col][rank]
  const BItem it = bitem(G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int c0 = it.ct * BW;
  mf4 aw[LEV > 0 ? LEV : 1][2], bw[LEV > 0 ? LEV : 1][2];
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
    const float* Wa = W + ((((size_t)it.s * LEV + l) * G.K + it.k) * LEAF + 32 * w + r) * RANK + 4 * q;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      aw[l][ch] = *reinterpret_cast<const mf4*>(Wa + 16 * ch);
      bw[l][ch] = *reinterpret_cast<const mf4*>(Wa + 16 * RANK + 16 * ch);
    }
  }
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
  // partner half sums, transposed into LDS: all loads first, then the stores
  constexpr int PER = (LEV > 0 ? LEV : 1) * RANK * BW / BNT;   // elements per thread
  float hv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + u * BNT;
    const int l = e / (RANK * BW), rem = e - l * RANK * BW;
    const int row = rem / BW, col = rem - row * BW;
    hv[u] = H[q_index(G, it.s, l, (it.k >> l) ^ 1, row) + c0 + col];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + u * BNT;
    const int l = e / (RANK * BW), rem = e - l * RANK * BW;
    const int row = rem / BW, col = rem - row * BW;
    Ps[(l * BW + col) * PS_STRIDE + row] = hv[u];
  }
  __syncthreads();
#pragma unroll
  for (int l = 0; l < LEV; ++l) {
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
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      Y[(size_t)(it.leaf0 + 32 * w + 4 * q + v) * G.nrhs + c0 + 16 * j + r] = ya[j][v];
      Y[(size_t)(it.leaf0 + 32 * w + 16 + 4 * q + v) * G.nrhs + c0 + 16 * j + r] = yb[j][v];
    }
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
