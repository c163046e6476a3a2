// Host side of the C ABI declared in include/hpcg.h: argument checks, workspace
// carving, engine selection and the solve loop.  All device work is in
// hpcg_kernels.hpp / hpcg_device.hpp.
#include "hpcg.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hpcg_apply.hpp"
#include "hpcg_bridge.hpp"
#include "hpcg_resident.hpp"
#include "hpcg_block.hpp"
#include "hpcg_bsolve.hpp"

using namespace hpcg;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t row_ptr, col, val, U, W, g, b, r, z, q, p0, p1, x, tleaf, pleaf, pq, rr, rz, st, ctl;
  size_t Fh, Fl, Fe, Wh, Wl, Th, Tl, We;   // block apply: factors as fp16 pairs and their exponents
  size_t wgflag;              // resident engine: per-workgroup barrier lines
  size_t lcol, hoff, hcol;    // resident engine: leaf-local CSR columns and halo lists
  size_t zll, pll;            // resident engine: flagged z words and flagged partials
  size_t qll, pqll;           // resident engine: flagged W^T q words and p.q partials
  size_t fr, fd, frhs, fsc;   // outer refinement: residual, correction, scaled rhs, per-system scalars
  size_t w, dinv, ftmp;       // squared form: H r; Jacobi: 1 / A_ii; apply scratch
  size_t Ub, Vb, Bc;          // bridge-format factors as given (native bridge apply)
  size_t llw, lle, lly;       // single-pass apply: flagged restriction words, per-leaf epochs,
                              // flagged diagonal-stage words of the split variant
  size_t total;
};

// LDS of one gfx950 compute unit: a workgroup's static and dynamic LDS must fit.
constexpr size_t kMaxLds = 160 * 1024;

// control words, each on its own 256-byte line
constexpr unsigned kPollLimitDefault = 1u << 22;   // polls of one flagged word (resident engine)
constexpr unsigned kApplyPollDefault = 1u << 20;   // poll rounds of the single-pass apply (about a second)
// the apply's abort word sits beside the solve's (one 8-byte read covers both)
constexpr size_t kCtlBarrier = 0, kCtlAbort = 256, kCtlApplyAbort = 260, kCtlItbase = 512, kCtlReplays = 768,
                 kCtlBytes = 1024;

constexpr int kMaxSplit = 8;   // workgroups per leaf in the streaming kernels

// split = 0 picks the workgroups per leaf automatically, else 1, 2, 4 or 8.
bool make_geom(const hpcg_partition* p, Geom& G, std::string& why, int split);

// The standalone apply on large batches (B K >= 512 leaves, more than two per
// compute unit) runs 4 workgroups per leaf: 32 KB of LDS each instead of up to
// 128 KB, so several share a compute unit and their loads overlap.
Geom apply_geom(const hpcg_partition* p, const Geom& G, int split) {
  if (split != 0 || (int64_t)G.B * G.K < 512 || G.bpl >= 4) return G;
  Geom A;
  std::string why;
  return make_geom(p, A, why, 4) ? A : G;
}

// split = 0 picks the workgroups per leaf automatically, else 1, 2, 4 or 8.
bool make_geom(const hpcg_partition* p, Geom& G, std::string& why, int split) {
  if (!p) { why = "partition is NULL"; return false; }
  if (p->leaf != LEAF) { why = "leaf size must be 128"; return false; }
  if (p->rank != RANK) { why = "off-diagonal rank must be 32"; return false; }
  if (p->n <= 0 || p->n % LEAF) { why = "n must be a positive multiple of 128"; return false; }
  const int K = p->n / LEAF;
  if (K & (K - 1)) { why = "n/128 must be a power of two"; return false; }
  int full = 0;
  while ((1 << full) < K) ++full;
  if (p->levels < 0 || p->levels > full) { why = "levels must lie in [0, log2(n/128)]"; return false; }
  if (p->levels > MAX_LEVELS) { why = "at most 8 tile levels (256 leaves) per system"; return false; }
  if (p->batch < 1) { why = "batch must be >= 1"; return false; }
  if ((int64_t)p->batch * p->n >= (int64_t)1 << 30) { why = "batch*n too large"; return false; }
  G.n = p->n;
  G.K = K;
  G.levels = p->levels;
  G.B = p->batch;
  // workgroups per leaf: enough to give every CU a workgroup, and enough that
  // the restriction and prolongation stages fit LDS in fp64 mode
  int bpl = split > 0 ? split : 1;
  while (split == 0 && (int64_t)G.B * K * bpl < 256 && bpl < kMaxSplit) bpl *= 2;
  for (;;) {
    G.bpl = bpl;
    G.RB = LEAF / bpl;
    const size_t need = sizeof(Smem<double>) + std::max(restrict_lds_bytes(G), prolong_lds_bytes<double>(G));
    if (need <= kMaxLds || bpl == kMaxSplit) {
      if (need > kMaxLds) { why = "partition needs more LDS than a compute unit has"; return false; }
      break;
    }
    bpl *= 2;
  }
  G.nblk_sys = K * bpl;
  G.nblk = G.B * G.nblk_sys;
  return true;
}

// Tiles (cores) per system: K/2 + K/4 + ... over the levels present.
int tile_count(const Geom& G) {
  int c = 0;
  for (int l = 0; l < G.levels; ++l) c += G.K >> (l + 1);
  return c;
}

Layout make_layout(const Geom& G, int64_t nnz) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const size_t N = (size_t)G.B * G.n;
  L.row_ptr = take((N + 1) * 4);
  L.col = take((size_t)nnz * 4);
  L.val = take((size_t)nnz * 4);
  L.U = take((size_t)G.B * G.K * LEAF * LEAF * 4);
  // block apply: dense leaf blocks and slabs (also transposed) as fp16 pairs
  L.Fh = take((size_t)G.B * G.K * LEAF * LEAF * 2);
  L.Fl = take((size_t)G.B * G.K * LEAF * LEAF * 2);
  L.Fe = take((size_t)G.B * G.K * 4);
  {
    const size_t slabs = (size_t)G.B * G.levels * G.K;
    L.Wh = take(slabs * LEAF * RANK * 2);
    L.Wl = take(slabs * LEAF * RANK * 2);
    L.Th = take(slabs * LEAF * RANK * 2);
    L.Tl = take(slabs * LEAF * RANK * 2);
    L.We = take(slabs * 4);
  }
  L.W = take((size_t)G.B * G.levels * G.K * LEAF * RANK * 4);
  L.g = take(N * 4);
  L.b = take(N * 4);
  // solve vectors and restriction partials are sized for the fp64 vector mode
  L.r = take(2 * N * 8);
  L.z = take(N * 8);
  L.q = take(N * 8);
  L.p0 = take(N * 8);
  L.p1 = take(N * 8);
  L.x = take(N * 8);
  // pleaf holds two copies of W^T r for the resident engine's ping-pong
  // diagonal shares per (leaf, slot) (streaming engines) also hold W^T q
  // (resident engine); sized for the largest leaf split, like the partials
  const size_t items = (size_t)G.B * G.K * kMaxSplit;
  L.tleaf = take((size_t)G.B * G.K * std::max(kMaxSplit * LEAF, G.levels * RANK) * 8 + 16);
  L.pleaf = take(2 * (size_t)G.B * G.levels * G.K * RANK * 8 + 16);
  L.pq = take(items * 8);
  L.rr = take(items * 8);
  L.rz = take(items * 8);
  L.st = take((size_t)G.B * sizeof(SysState));
  L.ctl = take(kCtlBytes);
  L.wgflag = take((size_t)G.B * G.K * kFlagStride * 4);
  L.lcol = take((size_t)nnz * 4);
  L.hoff = take(((size_t)G.B * G.K + 1) * 4);
  L.hcol = take((size_t)nnz * 4);           // a leaf has at most as many halo columns as entries
  L.zll = take(N * 16);
  L.pll = take((size_t)G.B * G.K * 32);
  L.qll = take(2 * (size_t)G.B * G.levels * G.K * RANK * 8 + 16);
  L.pqll = take(2 * (size_t)G.B * G.K * 16);
  L.fr = take(N * 8);
  L.fd = take(N * 8);
  L.frhs = take(N * 4);
  L.fsc = take((size_t)G.B * 8 * 3);
  L.w = take(N * 8);
  L.dinv = take(N * 8);
  L.ftmp = take(N * 4);
  L.llw = take((size_t)G.B * G.levels * G.K * RANK * 8 + 16);
  L.lle = take((size_t)G.B * G.K * 4);
  L.lly = take((size_t)G.B * G.K * LEAF * 8);
  if (G.levels > 0) {
    L.Ub = take((size_t)G.B * G.K * LEAF * RANK * 4);
    L.Vb = take((size_t)G.B * G.K * LEAF * RANK * 4);
    L.Bc = take((size_t)G.B * tile_count(G) * RANK * RANK * 4);
  }
  L.total = off;
  return L;
}

thread_local std::string g_create_error;

}  // namespace

// Scratch of the allocation-free block apply: the per-leaf restrictions Q and
// their half sums H of one call (each block_half_bytes).  One copy per GPU,
// held until the process ends; every call on that GPU shares it.  Host code
// never uses the array's name as an address: the device address of each GPU's
// copy comes from hipGetSymbolAddress at set-up (scratch_address).
constexpr size_t kNoAllocScratchBytes = 32u << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

struct hpcg_ctx {
  hpcg_partition part{};
  int64_t nnz = 0;
  Geom G{};
  Bufs B{};
  Layout lay{};
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  char* ws = nullptr;
  bool factors_set = false;
  bool bridge_set = false;   // the factors came in the bridge format (native bridge apply possible)
  int engine_opt = HPCG_ENGINE_AUTO;
  int unroll = 8;
  int prec = HPCG_PREC_VEC64;
  int last_engine = 0;
  int num_cu = 0;
  size_t max_lds = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  int graph_unroll = 0;
  int graph_prec = -1;
  int graph_bpl = 0;
  int graph_form = -1;
  int fallback = 0;
  int last_fallback = 0;
  int split = 0;
  int block_split = 0;   // HPCG_OPT_BLOCK_SPLIT: 0 automatic, 1 one workgroup per item, 2 two
  int apply_path = HPCG_APPLY_AUTO;
  Geom Gapply{};           // geometry of the standalone apply kernels
  int last_apply_path = 0;
  int fused_per_cu = -1;
  int split_per_cu = -1;
  int bridge_per_cu = -1;
  int bridge_split_per_cu = -1;
  int split_apply = 1;     // single-pass apply with two workgroups per leaf where it fits
  double graph_tol = -1.0;
  int graph_maxit = -1;
  int last_grid = 0;
  int last_lds = 0;
  int max_leaf_nnz = 0;
  int max_halo = 0;        // most halo columns of a leaf (resident engine)
  unsigned ep_next = 1;    // resident engine: epoch base of the next solve
  int* h_flag = nullptr;   // pinned, device-mapped (word 0: graph engine, word 16: block solve)
  int* d_flag = nullptr;
  // block solve: the recorded iterations and what they were recorded for
  hipGraph_t bs_graph = nullptr;
  hipGraphExec_t bs_gexec = nullptr;
  const void* bs_key[2] = {nullptr, nullptr};
  int bs_nrhs = 0, bs_unroll = 0, bs_maxit = -1, bs_split = -1;
  double bs_tol = -1.0;
  SysState* h_st = nullptr;
  int* h_ctl = nullptr;    // pinned copy of the abort words (solve, apply)
  char* d_scratch = nullptr;   // this device's copy of `scratch`
  std::vector<int32_t> last_status;
  std::string err;
};

namespace {

// Clear the HIP runtime's sticky last error after a call whose failure we handle.
void clear_hip_error_fn() { (void)hipGetLastError(); }

hpcg_status fail(hpcg_ctx* h, hpcg_status s, const std::string& msg) {
  if (h) h->err = msg; else g_create_error = msg;
  return s;
}

hpcg_status hip_fail(hpcg_ctx* h, hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(h, HPCG_ERR_HIP, m);
}

#define HIP_OR_FAIL(h, call)                                  \
  do {                                                        \
    hipError_t e_ = (call);                                   \
    if (e_ != hipSuccess) return hip_fail((h), e_, #call);    \
  } while (0)

hpcg_status check_launch(hpcg_ctx* h, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(h, e, what);
  return HPCG_OK;
}

// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(int dev, char** out) {
  static std::mutex mu;
  static std::vector<std::pair<int, char*>> known;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& k : known)
    if (k.first == dev) {
      *out = k.second;
      return hipSuccess;
    }
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  known.emplace_back(dev, reinterpret_cast<char*>(ptr));
  *out = reinterpret_cast<char*>(ptr);
  return hipSuccess;
}

// The host has seen the single-pass apply's abort word set (after a
// synchronization): clear it and report the undefined output.
hpcg_status apply_timed_out(hpcg_ctx* h) {
  HIP_OR_FAIL(h, hipMemsetAsync(h->B.apply_abort, 0, sizeof(int), h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  return fail(h, HPCG_ERR_HIP, "a bounded partner wait of an earlier single-pass hpcg_apply_M ran out (other work "
                               "held the compute units, or HPCG_OPT_APPLY_POLL_LIMIT below the exchange latency): "
                               "that apply's output is undefined");
}

// Raise a kernel's dynamic-LDS limit when it needs more than the default.
// The limit is a per-kernel, per-process setting: remember what was granted so
// that repeated calls cost no runtime call.
hpcg_status allow_lds(hpcg_ctx* h, const void* fn, size_t bytes) {
  if (bytes <= 48 * 1024) return HPCG_OK;
  static std::mutex mu;
  static std::vector<std::pair<const void*, size_t>> granted;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& g : granted)
    if (g.first == fn && g.second >= bytes) return HPCG_OK;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    clear_hip_error_fn();
    return hip_fail(h, e, "hipFuncSetAttribute(MaxDynamicSharedMemorySize)");
  }
  granted.emplace_back(fn, bytes);
  return HPCG_OK;
}



void destroy_graph(hpcg_ctx* h) {
  if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  h->gexec = nullptr;
  h->graph = nullptr;
  h->graph_unroll = 0;
}

template <typename T>
hpcg_status build_graph(hpcg_ctx* h) {
  destroy_graph(h);
  const Geom G = h->G;
  const Bufs B = h->B;
  const size_t lds_b = restrict_lds_bytes(G), lds_c = prolong_lds_bytes<T>(G);
  hpcg_status s = allow_lds(h, reinterpret_cast<const void*>(&k_phase_B<T>), lds_b);
  if (s == HPCG_OK) s = allow_lds(h, reinterpret_cast<const void*>(&k_phase_C<T>), lds_c);
  if (s != HPCG_OK) return s;
  HIP_OR_FAIL(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  for (int j = 0; j < h->unroll; ++j) {
    hipLaunchKernelGGL(k_phase_A<T>, dim3(G.nblk), dim3(NT), 0, h->cap_stream, G, B, j);
    hipLaunchKernelGGL(k_phase_B<T>, dim3(G.nblk), dim3(NT), lds_b, h->cap_stream, G, B, j, -1, 0);
    if (B.form == FORM_SQUARED) {
      hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), lds_c, h->cap_stream, G, B, j, -1, 1);
      hipLaunchKernelGGL(k_phase_B<T>, dim3(G.nblk), dim3(NT), lds_b, h->cap_stream, G, B, j, -1, 1);
      hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), lds_c, h->cap_stream, G, B, j, -1, 2);
    } else {
      hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), lds_c, h->cap_stream, G, B, j, -1, 0);
    }
  }
  hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, h->cap_stream, G, B, h->unroll, h->d_flag);
  hipError_t e = hipStreamEndCapture(h->cap_stream, &h->graph);
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamEndCapture");
  e = hipGraphInstantiate(&h->gexec, h->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) return hip_fail(h, e, "hipGraphInstantiate");
  h->graph_unroll = h->unroll;
  h->graph_prec = h->prec;
  h->graph_bpl = G.bpl;
  h->graph_form = B.form;
  h->graph_tol = B.tol;
  h->graph_maxit = B.maxit;
  return HPCG_OK;
}

template <typename T>
hpcg_status run_graph(hpcg_ctx* h) {
  const Geom G = h->G;
  const Bufs B = h->B;
  if (!h->gexec || h->graph_unroll != h->unroll || h->graph_prec != h->prec || h->graph_tol != B.tol ||
      h->graph_maxit != B.maxit || h->graph_bpl != G.bpl || h->graph_form != B.form) {
    hpcg_status s = build_graph<T>(h);
    if (s != HPCG_OK) return s;
  }
  __atomic_store_n(h->h_flag, 0, __ATOMIC_RELEASE);
  hipLaunchKernelGGL(k_reset, dim3(1), dim3(64), 0, h->stream, B, 1, h->d_flag, G.B * G.K);
  hipLaunchKernelGGL(k_phase_B<T>, dim3(G.nblk), dim3(NT), restrict_lds_bytes(G), h->stream, G, B, 0, 0, 0);
  if (B.form == FORM_SQUARED) {
    hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), prolong_lds_bytes<T>(G), h->stream, G, B, 0, 0, 1);
    hipLaunchKernelGGL(k_phase_B<T>, dim3(G.nblk), dim3(NT), restrict_lds_bytes(G), h->stream, G, B, 0, 0, 1);
    hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), prolong_lds_bytes<T>(G), h->stream, G, B, 0, 0, 2);
  } else {
    hipLaunchKernelGGL(k_phase_C<T>, dim3(G.nblk), dim3(NT), prolong_lds_bytes<T>(G), h->stream, G, B, 0, 0, 0);
  }
  hpcg_status s = check_launch(h, "graph engine setup launch");
  if (s != HPCG_OK) return s;
  const int max_replays = (B.maxit + h->unroll - 1) / h->unroll;
  const int lookahead = 2;
  int launched = 0, seen = 0;
  bool done = false;
  while (!done) {
    while (launched < max_replays && launched - seen < lookahead) {
      HIP_OR_FAIL(h, hipGraphLaunch(h->gexec, h->stream));
      ++launched;
    }
    // wait until the next replay has published its flag
    unsigned spins = 0;
    for (;;) {
      const int f = __atomic_load_n(h->h_flag, __ATOMIC_ACQUIRE);
      if ((f >> 1) > seen) {
        seen = f >> 1;
        done = (f & 1) != 0 || seen >= max_replays;
        break;
      }
      if ((++spins & 1023u) == 0) {
        hipError_t q = hipStreamQuery(h->stream);
        if (q == hipSuccess) {
          const int f2 = __atomic_load_n(h->h_flag, __ATOMIC_ACQUIRE);
          if ((f2 >> 1) <= seen) return fail(h, HPCG_ERR_HIP, "graph engine: stream drained without progress flag");
        } else if (q != hipErrorNotReady) {
          return hip_fail(h, q, "hipStreamQuery");
        }
      }
    }
  }
  h->last_grid = G.nblk;
  h->last_lds = (int)std::max(restrict_lds_bytes(G), prolong_lds_bytes<T>(G));
  return HPCG_OK;
}

template <typename T>
const void* resident_kernel(int levels, int form) {
  if (form == FORM_JACOBI) return reinterpret_cast<const void*>(&k_resident<T, 0, FM_JACOBI>);
  const bool sq = (form == FORM_SQUARED);
  switch (levels * 2 + (sq ? 1 : 0)) {
#define HPCG_RESIDENT(LV)                                                              \
    case 2 * LV: return reinterpret_cast<const void*>(&k_resident<T, LV, FM_DIRECT>); \
    case 2 * LV + 1: return reinterpret_cast<const void*>(&k_resident<T, LV, FM_SQUARED>);
    HPCG_RESIDENT(0) HPCG_RESIDENT(1) HPCG_RESIDENT(2) HPCG_RESIDENT(3) HPCG_RESIDENT(4)
    HPCG_RESIDENT(5) HPCG_RESIDENT(6) HPCG_RESIDENT(7) HPCG_RESIDENT(8)
#undef HPCG_RESIDENT
    default: return nullptr;
  }
}

// Register-resident persistent solve: one 512-thread workgroup per leaf, all
// of a launch co-resident (one per CU).  A batch with more leaves than that is
// solved in groups of whole systems, one launch per group in stream order
// (systems are independent, so a group needs nothing from another).  Declines
// (ran = false) when one system alone has more leaves than the device has
// CUs.
template <typename T>
hpcg_status run_resident(hpcg_ctx* h, bool& ran) {
  ran = false;
  const Geom G = h->G;
  const Bufs B = h->B;
  // an explicit leaf split asks for the streaming engines (one workgroup per
  // slot of a leaf); the resident engine always gives a leaf one workgroup
  if (G.K > h->num_cu || h->split > 0) return HPCG_OK;
  const void* fn = resident_kernel<T>(G.levels, B.form);
  if (!fn) return HPCG_OK;
  // CSR rows, the partner stage of W^T r, z and p by leaf-local column (own
  // rows, then the halo), the halo's column list
  const size_t dyn = ((size_t)h->max_leaf_nnz * 8 + (LEAF + 1) * 4 + 15) / 16 * 16 +
                     (size_t)partner_rows(G) * RANK * sizeof(T) +
                     2 * ((size_t)LEAF + h->max_halo) * sizeof(T) + (size_t)h->max_halo * 4;
  if (dyn + sizeof(RSmem<T>) > kMaxLds) return HPCG_OK;
  hpcg_status s = allow_lds(h, fn, dyn);
  if (s != HPCG_OK) return s;
  int per_cu = 0;
  HIP_OR_FAIL(h, hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NTR, dyn));
  const int64_t cap = (int64_t)per_cu * h->num_cu;   // co-resident workgroups
  if (cap < G.K) return HPCG_OK;
  const int group = (int)std::min<int64_t>(G.B, cap / G.K);   // systems per launch
  hipLaunchKernelGGL(k_reset, dim3(1), dim3(64), 0, h->stream, B, 0, (int*)nullptr, G.B * G.K);
  // This solve's flagged words carry epochs ep_base + i, i = 0 .. maxit + 1:
  // never one that an earlier solve left in the buffers.  Near the end of the
  // 32-bit range the words are cleared and the count restarts.
  const uint64_t span = (uint64_t)B.maxit + 4;
  if ((uint64_t)h->ep_next + span >= 0xFFFFFFF0ull) {
    HIP_OR_FAIL(h, hipMemsetAsync(h->ws + h->lay.zll, 0,
                                  h->lay.pqll + 2 * (size_t)G.B * G.K * 16 - h->lay.zll, h->stream));
    h->ep_next = 1;
  }
  // the fp64 W^T q words carry only an 8-bit step tag: cleared every solve
  if (G.levels > 0)
    HIP_OR_FAIL(h, hipMemsetAsync(h->ws + h->lay.qll, 0, 2 * (size_t)G.B * G.levels * G.K * RANK * 8, h->stream));
  Geom Ga = G;
  Bufs Ba = B;
  Ba.ep_base = h->ep_next;
  h->ep_next += (unsigned)span;
  int mln = h->max_leaf_nnz, mh = h->max_halo;
  for (int s0 = 0; s0 < G.B; s0 += group) {
    int first = s0;
    void* args[] = {&Ga, &Ba, &mln, &mh, &first};
    const int nsys = std::min(group, G.B - s0);
    HIP_OR_FAIL(h, hipLaunchKernel(fn, dim3((unsigned)(nsys * G.K)), dim3(NTR), args, (unsigned)dyn, h->stream));
  }
  h->last_grid = group * G.K;
  h->last_lds = (int)dyn;
  ran = true;
  return HPCG_OK;
}

// One launch for the whole solve; the grid is as many workgroups as can be
// co-resident (at most one per (leaf, slot) item), per the occupancy query.
template <typename T>
hpcg_status run_persistent(hpcg_ctx* h, bool& ran) {
  ran = false;
  const Geom G = h->G;
  const Bufs B = h->B;
  if (B.form != FORM_DIRECT) return HPCG_OK;
  const size_t dyn = std::max(restrict_lds_bytes(G), prolong_lds_bytes<T>(G));
  const void* fn = reinterpret_cast<const void*>(&k_persistent<T>);
  hpcg_status s = allow_lds(h, fn, dyn);
  if (s != HPCG_OK) return s;
  int per_cu = 0;
  HIP_OR_FAIL(h, hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, dyn));
  const int64_t cap = (int64_t)per_cu * h->num_cu;
  if (cap <= 0) return HPCG_OK;
  const int grid = (int)std::min<int64_t>(cap, G.nblk);
  hipLaunchKernelGGL(k_reset, dim3(1), dim3(64), 0, h->stream, B, 0, (int*)nullptr, G.B * G.K);
  Geom Ga = G;
  Bufs Ba = B;
  void* args[] = {&Ga, &Ba};
  HIP_OR_FAIL(h, hipLaunchKernel(fn, dim3(grid), dim3(NT), args, (unsigned)dyn, h->stream));
  h->last_grid = grid;
  h->last_lds = (int)dyn;
  ran = true;
  return HPCG_OK;
}

}  // namespace

extern "C" {

size_t hpcg_workspace_bytes(const hpcg_partition* part, int64_t nnz_total) {
  Geom G;
  std::string why;
  if (!make_geom(part, G, why, 0) || nnz_total < 0) return 0;
  return make_layout(G, nnz_total).total;
}

hpcg_status hpcg_create(const hpcg_partition* part, const int32_t* d_row_ptr, const int32_t* d_col,
                        const float* d_val, int64_t nnz_total, void* d_workspace, size_t ws_bytes,
                        void* stream, hpcg_handle* out) {
  g_create_error.clear();
  if (!out) return fail(nullptr, HPCG_ERR_INVALID_ARG, "out is NULL");
  Geom G;
  std::string why;
  if (!make_geom(part, G, why, 0)) return fail(nullptr, HPCG_ERR_SHAPE, why);
  if (nnz_total < 0 || nnz_total >= ((int64_t)1 << 31)) return fail(nullptr, HPCG_ERR_SHAPE, "nnz_total out of range");
  if (!d_row_ptr || (nnz_total > 0 && (!d_col || !d_val)))
    return fail(nullptr, HPCG_ERR_INVALID_ARG, "CSR pointer is NULL");
  if (!d_workspace) return fail(nullptr, HPCG_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign)
    return fail(nullptr, HPCG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const Layout lay = make_layout(G, nnz_total);
  if (ws_bytes < lay.total) return fail(nullptr, HPCG_ERR_WORKSPACE, "workspace too small");

  hpcg_ctx* h = new hpcg_ctx();
  h->part = *part;
  h->nnz = nnz_total;
  h->G = G;
  h->Gapply = apply_geom(part, G, 0);
  h->lay = lay;
  h->stream = reinterpret_cast<hipStream_t>(stream);
  h->ws = reinterpret_cast<char*>(d_workspace);
  auto cleanup_fail = [&](hpcg_status s) {
    g_create_error = h->err;
    hpcg_destroy(h);
    return s;
  };
#define CREATE_HIP(call)                                              \
  do {                                                                \
    hipError_t e_ = (call);                                           \
    if (e_ != hipSuccess) return cleanup_fail(hip_fail(h, e_, #call)); \
  } while (0)

  int dev = 0;
  CREATE_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  CREATE_HIP(hipGetDeviceProperties(&prop, dev));
  h->num_cu = prop.multiProcessorCount;
  CREATE_HIP(scratch_address(dev, &h->d_scratch));
  int max_lds = 0;
  CREATE_HIP(hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  h->max_lds = max_lds > 0 ? (size_t)max_lds : 65536;
  CREATE_HIP(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  CREATE_HIP(hipHostMalloc(reinterpret_cast<void**>(&h->h_flag), 256, hipHostMallocMapped));
  CREATE_HIP(hipHostGetDevicePointer(reinterpret_cast<void**>(&h->d_flag), h->h_flag, 0));
  CREATE_HIP(hipHostMalloc(reinterpret_cast<void**>(&h->h_st), (size_t)G.B * sizeof(SysState), hipHostMallocDefault));
  CREATE_HIP(hipHostMalloc(reinterpret_cast<void**>(&h->h_ctl), 256, hipHostMallocDefault));
  *h->h_flag = 0;

  char* w = h->ws;
  Bufs& B = h->B;
  B.row_ptr = reinterpret_cast<const int*>(w + lay.row_ptr);
  B.col = reinterpret_cast<const int*>(w + lay.col);
  B.val = reinterpret_cast<const float*>(w + lay.val);
  B.U = reinterpret_cast<const float*>(w + lay.U);
  B.W = reinterpret_cast<const float*>(w + lay.W);
  B.g = reinterpret_cast<const float*>(w + lay.g);
  B.b = reinterpret_cast<const float*>(w + lay.b);
  B.r = w + lay.r;
  B.z = w + lay.z;
  B.q = w + lay.q;
  B.p0 = w + lay.p0;
  B.p1 = w + lay.p1;
  B.x = reinterpret_cast<double*>(w + lay.x);
  B.tleaf = w + lay.tleaf;
  B.pleaf = w + lay.pleaf;
  B.pq_part = reinterpret_cast<double*>(w + lay.pq);
  B.rr_part = reinterpret_cast<double*>(w + lay.rr);
  B.rz_part = reinterpret_cast<double*>(w + lay.rz);
  B.st = reinterpret_cast<SysState*>(w + lay.st);
  B.barrier = reinterpret_cast<unsigned*>(w + lay.ctl + kCtlBarrier);
  B.abort_flag = reinterpret_cast<int*>(w + lay.ctl + kCtlAbort);
  B.apply_abort = reinterpret_cast<int*>(w + lay.ctl + kCtlApplyAbort);
  B.itbase = reinterpret_cast<int*>(w + lay.ctl + kCtlItbase);
  B.replays = reinterpret_cast<int*>(w + lay.ctl + kCtlReplays);
  B.wgflag = reinterpret_cast<unsigned*>(w + lay.wgflag);
  B.lcol = reinterpret_cast<const int*>(w + lay.lcol);
  B.hoff = reinterpret_cast<const int*>(w + lay.hoff);
  B.hcol = reinterpret_cast<const int*>(w + lay.hcol);
  B.zll = reinterpret_cast<unsigned long long*>(w + lay.zll);
  B.pll = reinterpret_cast<unsigned long long*>(w + lay.pll);
  B.qll = reinterpret_cast<unsigned long long*>(w + lay.qll);
  B.pqll = reinterpret_cast<unsigned long long*>(w + lay.pqll);
  B.ep_base = 1u;
  B.poll_limit = kPollLimitDefault;
  B.apply_poll_limit = kApplyPollDefault;
  B.llw = reinterpret_cast<unsigned long long*>(w + lay.llw);
  B.lle = reinterpret_cast<unsigned*>(w + lay.lle);
  B.lly = reinterpret_cast<unsigned long long*>(w + lay.lly);
  B.Ub = reinterpret_cast<const float*>(w + lay.Ub);
  B.Vb = reinterpret_cast<const float*>(w + lay.Vb);
  B.Bc = reinterpret_cast<const float*>(w + lay.Bc);
  B.ncores = tile_count(G);
  B.w = w + lay.w;
  B.dinv = reinterpret_cast<const double*>(w + lay.dinv);
  B.form = FORM_DIRECT;
  B.tol = 1e-6;
  B.maxit = 1000;

  const size_t N = (size_t)G.B * G.n;
  CREATE_HIP(hipMemsetAsync(w + lay.ctl, 0, kCtlBytes, h->stream));
  CREATE_HIP(hipMemsetAsync(w + lay.llw, 0, lay.lly + (size_t)G.B * G.K * LEAF * 8 - lay.llw, h->stream));
  CREATE_HIP(hipMemcpyAsync(w + lay.row_ptr, d_row_ptr, (N + 1) * 4, hipMemcpyDeviceToDevice, h->stream));
  if (nnz_total > 0) {
    CREATE_HIP(hipMemcpyAsync(w + lay.col, d_col, (size_t)nnz_total * 4, hipMemcpyDeviceToDevice, h->stream));
    CREATE_HIP(hipMemcpyAsync(w + lay.val, d_val, (size_t)nnz_total * 4, hipMemcpyDeviceToDevice, h->stream));
  }
  // host-side structural checks of the CSR (create time only)
  std::vector<int32_t> rp(N + 1), cols((size_t)nnz_total);
  CREATE_HIP(hipMemcpyAsync(rp.data(), w + lay.row_ptr, (N + 1) * 4, hipMemcpyDeviceToHost, h->stream));
  if (nnz_total > 0)
    CREATE_HIP(hipMemcpyAsync(cols.data(), w + lay.col, (size_t)nnz_total * 4, hipMemcpyDeviceToHost, h->stream));
  CREATE_HIP(hipStreamSynchronize(h->stream));
  if (rp[0] != 0 || rp[N] != nnz_total) return cleanup_fail(fail(h, HPCG_ERR_SHAPE, "row_ptr must start at 0 and end at nnz_total"));
  for (size_t i = 0; i < N; ++i) {
    if (rp[i + 1] < rp[i]) return cleanup_fail(fail(h, HPCG_ERR_SHAPE, "row_ptr must be nondecreasing"));
    const int64_t lo = (int64_t)(i / G.n) * G.n, hi = lo + G.n;
    for (int32_t e = rp[i]; e < rp[i + 1]; ++e)
      if (cols[e] < lo || cols[e] >= hi)
        return cleanup_fail(fail(h, HPCG_ERR_SHAPE, "column index outside its system's block"));
  }
  hipLaunchKernelGGL(k_diag_inv, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, h->stream, h->B.row_ptr, h->B.col,
                     h->B.val, reinterpret_cast<double*>(h->ws + h->lay.dinv), (int)N, G.n);
  CREATE_HIP(hipGetLastError());
  for (size_t i0 = 0; i0 < N; i0 += LEAF)
    h->max_leaf_nnz = std::max(h->max_leaf_nnz, rp[i0 + LEAF] - rp[i0]);
  {
    // Resident engine: every CSR column as a leaf-local index (own rows 0 ..
    // LEAF-1, other columns LEAF + their slot in the leaf's halo, the sorted
    // distinct columns outside the leaf that its rows reference).
    std::vector<int32_t> lcol((size_t)nnz_total), hoff((size_t)G.B * G.K + 1, 0), hcol;
    std::vector<int32_t> halo;
    for (size_t item = 0; item < (size_t)G.B * G.K; ++item) {
      const int32_t lo = (int32_t)(item * LEAF), hi = lo + LEAF;
      halo.clear();
      for (int32_t e = rp[lo]; e < rp[hi]; ++e)
        if (cols[e] < lo || cols[e] >= hi) halo.push_back(cols[e]);
      std::sort(halo.begin(), halo.end());
      halo.erase(std::unique(halo.begin(), halo.end()), halo.end());
      hoff[item] = (int32_t)hcol.size();
      hcol.insert(hcol.end(), halo.begin(), halo.end());
      h->max_halo = std::max(h->max_halo, (int)halo.size());
      for (int32_t e = rp[lo]; e < rp[hi]; ++e) {
        const int32_t c = cols[e];
        lcol[e] = (c >= lo && c < hi) ? c - lo
                                      : LEAF + (int32_t)(std::lower_bound(halo.begin(), halo.end(), c) - halo.begin());
      }
    }
    hoff.back() = (int32_t)hcol.size();
    CREATE_HIP(hipMemcpyAsync(w + lay.hoff, hoff.data(), hoff.size() * 4, hipMemcpyHostToDevice, h->stream));
    if (nnz_total > 0)
      CREATE_HIP(hipMemcpyAsync(w + lay.lcol, lcol.data(), lcol.size() * 4, hipMemcpyHostToDevice, h->stream));
    if (!hcol.empty())
      CREATE_HIP(hipMemcpyAsync(w + lay.hcol, hcol.data(), hcol.size() * 4, hipMemcpyHostToDevice, h->stream));
    CREATE_HIP(hipMemsetAsync(w + lay.zll, 0, lay.pqll + 2 * (size_t)G.B * G.K * 16 - lay.zll, h->stream));
    CREATE_HIP(hipStreamSynchronize(h->stream));   // the host vectors go out of scope
  }
#undef CREATE_HIP
  h->last_status.assign(G.B, HPCG_SYS_RUNNING);
  *out = h;
  return HPCG_OK;
}

hpcg_status hpcg_set_values(hpcg_handle h, const float* d_val) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (h->nnz > 0 && !d_val) return fail(h, HPCG_ERR_INVALID_ARG, "d_val is NULL");
  if (h->nnz > 0)
    HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.val, d_val, (size_t)h->nnz * 4, hipMemcpyDeviceToDevice, h->stream));
  const int N = h->G.B * h->G.n;
  hipLaunchKernelGGL(k_diag_inv, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, h->stream, h->B.row_ptr, h->B.col,
                     h->B.val, reinterpret_cast<double*>(h->ws + h->lay.dinv), N, h->G.n);
  return check_launch(h, "diagonal launch");
}

namespace {
// The block apply's operands as fp16 pairs, formed from U and the slabs in the
// workspace (stream-ordered after their copies).
BlockFactors16 block_factors16(const hpcg_ctx* h) {
  const char* w = h->ws;
  auto p = [&](size_t o) { return reinterpret_cast<const _Float16*>(w + o); };
  BlockFactors16 f;
  f.Fh = p(h->lay.Fh); f.Fl = p(h->lay.Fl); f.Fe = reinterpret_cast<const int*>(w + h->lay.Fe);
  f.Wh = p(h->lay.Wh); f.Wl = p(h->lay.Wl); f.Th = p(h->lay.Th); f.Tl = p(h->lay.Tl);
  f.We = reinterpret_cast<const int*>(w + h->lay.We);
  return f;
}
void block_factor_pairs(hpcg_ctx* h) {
  char* w = h->ws;
  const Geom& G = h->G;
  hipLaunchKernelGGL(k_leaf_blocks, dim3(G.B * G.K), dim3(BNT), 0, h->stream, h->B.U,
                     reinterpret_cast<_Float16*>(w + h->lay.Fh), reinterpret_cast<_Float16*>(w + h->lay.Fl),
                     reinterpret_cast<int*>(w + h->lay.Fe));
  if (G.levels > 0)
    hipLaunchKernelGGL(k_split_slabs, dim3(G.B * G.levels * G.K), dim3(BNT), 0, h->stream, h->B.W,
                       reinterpret_cast<_Float16*>(w + h->lay.Wh), reinterpret_cast<_Float16*>(w + h->lay.Wl),
                       reinterpret_cast<_Float16*>(w + h->lay.Th), reinterpret_cast<_Float16*>(w + h->lay.Tl),
                       reinterpret_cast<int*>(w + h->lay.We));
}
}  // namespace

hpcg_status hpcg_set_factors(hpcg_handle h, const float* d_leafU, const float* d_tileW, const float* d_gate) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  const Geom& G = h->G;
  if (!d_leafU || !d_gate || (G.levels > 0 && !d_tileW)) return fail(h, HPCG_ERR_INVALID_ARG, "factor pointer is NULL");
  HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.U, d_leafU, (size_t)G.B * G.K * LEAF * LEAF * 4,
                                hipMemcpyDeviceToDevice, h->stream));
  if (G.levels > 0)
    HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.W, d_tileW, (size_t)G.B * G.levels * G.K * LEAF * RANK * 4,
                                  hipMemcpyDeviceToDevice, h->stream));
  HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.g, d_gate, (size_t)G.B * G.n * 4, hipMemcpyDeviceToDevice, h->stream));
  block_factor_pairs(h);
  hpcg_status s = check_launch(h, "leaf block launch");
  if (s != HPCG_OK) return s;
  h->factors_set = true;
  h->bridge_set = false;
  return HPCG_OK;
}

const void* fused_apply_kernel(int levels) {
  switch (levels) {
    case 0: return reinterpret_cast<const void*>(&k_apply_fused<0>);
    case 1: return reinterpret_cast<const void*>(&k_apply_fused<1>);
    case 2: return reinterpret_cast<const void*>(&k_apply_fused<2>);
    case 3: return reinterpret_cast<const void*>(&k_apply_fused<3>);
    case 4: return reinterpret_cast<const void*>(&k_apply_fused<4>);
    case 5: return reinterpret_cast<const void*>(&k_apply_fused<5>);
    case 6: return reinterpret_cast<const void*>(&k_apply_fused<6>);
    case 7: return reinterpret_cast<const void*>(&k_apply_fused<7>);
    case 8: return reinterpret_cast<const void*>(&k_apply_fused<8>);
    default: return nullptr;
  }
}

// Single launch of the apply when every leaf gets its own CU (one 512-thread
// workgroup per leaf, the occupancy query confirming that all of them fit at
// once); ran = false when it does not fit (the caller then uses the two
// launches).  An ordinary launch: the one device-wide barrier inside waits for
// workgroups that the hardware dispatches as soon as resources free up, and
// its wait is bounded.
const void* split_apply_kernel(int levels) {
  switch (levels) {
    case 1: return reinterpret_cast<const void*>(&k_apply_split<1>);
    case 2: return reinterpret_cast<const void*>(&k_apply_split<2>);
    case 3: return reinterpret_cast<const void*>(&k_apply_split<3>);
    case 4: return reinterpret_cast<const void*>(&k_apply_split<4>);
    case 5: return reinterpret_cast<const void*>(&k_apply_split<5>);
    case 6: return reinterpret_cast<const void*>(&k_apply_split<6>);
    case 7: return reinterpret_cast<const void*>(&k_apply_split<7>);
    case 8: return reinterpret_cast<const void*>(&k_apply_split<8>);
    default: return nullptr;
  }
}

#define HPCG_BRIDGE_KERNEL(LV)                                                                          \
  case LV:                                                                                              \
    return split ? reinterpret_cast<const void*>(&k_apply_bridge<LV, true>)                            \
                 : reinterpret_cast<const void*>(&k_apply_bridge<LV, false>);
const void* bridge_apply_kernel(int levels, bool split) {
  switch (levels) {
    HPCG_BRIDGE_KERNEL(1) HPCG_BRIDGE_KERNEL(2) HPCG_BRIDGE_KERNEL(3) HPCG_BRIDGE_KERNEL(4)
    HPCG_BRIDGE_KERNEL(5) HPCG_BRIDGE_KERNEL(6) HPCG_BRIDGE_KERNEL(7) HPCG_BRIDGE_KERNEL(8)
    default: return nullptr;
  }
}
#undef HPCG_BRIDGE_KERNEL

// The native bridge-format apply (factors from hpcg_set_factors_bridge): one
// launch per group of whole systems whose leaves all get a compute unit, two
// workgroups per leaf while the batch has at most half as many leaves as the
// device has CUs (as the slab apply; N16k 6.92 -> 6.81 us).  ran = false when
// it does not fit.
hpcg_status run_bridge_apply(hpcg_ctx* h, const float* d_r, float* d_y, bool& ran) {
  ran = false;
  const Geom G = h->G;
  const int items = G.B * G.K;
  if (G.levels < 1 || !h->bridge_set || G.K > h->num_cu) return HPCG_OK;
  const size_t dyn = (size_t)G.levels * RANK * CSTRIDE * sizeof(float);   // the leaf's tiles' cores
  if (dyn + sizeof(RSmem<float>) > kMaxLds) return HPCG_OK;
  const bool split = h->split_apply && 2 * (int64_t)items <= h->num_cu;
  const void* fn = bridge_apply_kernel(G.levels, split);
  if (!fn) return HPCG_OK;
  hpcg_status s = allow_lds(h, fn, dyn);
  if (s != HPCG_OK) return s;
  int& per_cu = split ? h->bridge_split_per_cu : h->bridge_per_cu;
  if (per_cu < 0) HIP_OR_FAIL(h, hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NTR, dyn));
  const int wg_per_leaf = split ? 2 : 1;
  const int64_t cap = (int64_t)per_cu * h->num_cu / wg_per_leaf;
  const int per_launch = (int)std::min<int64_t>(G.B, cap / G.K);
  if (per_launch < 1) return HPCG_OK;
  Geom Ga = G;
  Bufs Ba = h->B;
  const float* ra = d_r;
  float* ya = d_y;
  int item0 = 0;
  void* args[] = {&Ga, &Ba, &ra, &ya, &item0};
  for (int s0 = 0; s0 < G.B; s0 += per_launch) {
    item0 = s0 * G.K;
    const int nsys = std::min(per_launch, G.B - s0);
    HIP_OR_FAIL(h, hipLaunchKernel(fn, dim3(wg_per_leaf * nsys * G.K), dim3(NTR), args, (unsigned)dyn, h->stream));
  }
  ran = true;
  return HPCG_OK;
}

hpcg_status run_fused_apply(hpcg_ctx* h, const float* d_r, float* d_y, bool& ran) {
  ran = false;
  const Geom G = h->G;
  const int items = G.B * G.K;
  if (G.K > h->num_cu) return HPCG_OK;
  Geom Ga = G;
  Bufs Ba = h->B;
  const float* ra = d_r;
  float* ya = d_y;
  void* args[] = {&Ga, &Ba, &ra, &ya};
  const size_t dyn = 0;   // the partner words are summed as they land: no stage in LDS
  // two workgroups per leaf (diagonal / off-diagonal roles) while the batch
  // has at most half as many leaves as the device has compute units and
  // every workgroup can be resident at once.  Measured: n = 1,024 / 4,096 /
  // 8,192 gain 9 / 4 / 3%; at 128 leaves (n = 16,384), with the off-diagonal
  // workgroup's short wait before its first poll, 6.57 -> 6.16 us warm and
  // 9.66 -> 9.39 us with the factors in HBM (without the wait it gained
  // nothing warm and lost 4% cold).
  const bool split = h->split_apply && 2 * (int64_t)items <= h->num_cu;
  if (const void* fs = split ? split_apply_kernel(G.levels) : nullptr) {
    hpcg_status s = allow_lds(h, fs, dyn);
    if (s != HPCG_OK) return s;
    if (h->split_per_cu < 0)
      HIP_OR_FAIL(h, hipOccupancyMaxActiveBlocksPerMultiprocessor(&h->split_per_cu, fs, NTR, dyn));
    if (dyn + sizeof(RSmem<float>) <= kMaxLds && (int64_t)h->split_per_cu * h->num_cu >= 2 * (int64_t)items) {
      HIP_OR_FAIL(h, hipLaunchKernel(fs, dim3(2 * items), dim3(NTR), args, (unsigned)dyn, h->stream));
      ran = true;
      return HPCG_OK;
    }
  }
  const void* fn = fused_apply_kernel(G.levels);
  if (!fn) return HPCG_OK;
  if (dyn + sizeof(RSmem<float>) > kMaxLds) return HPCG_OK;
  hpcg_status s = allow_lds(h, fn, dyn);
  if (s != HPCG_OK) return s;
  if (h->fused_per_cu < 0)
    HIP_OR_FAIL(h, hipOccupancyMaxActiveBlocksPerMultiprocessor(&h->fused_per_cu, fn, NTR, dyn));
  // a leaf waits only for leaves of its own system: a batch larger than the
  // co-resident workgroups runs as launches over as many whole systems as fit
  const int64_t cap = (int64_t)h->fused_per_cu * h->num_cu;
  const int per_launch = (int)std::min<int64_t>(G.B, cap / G.K);
  if (per_launch < 1) return HPCG_OK;
  int item0 = 0;
  void* fargs[] = {&Ga, &Ba, &ra, &ya, &item0};
  for (int s0 = 0; s0 < G.B; s0 += per_launch) {
    item0 = s0 * G.K;
    const int nsys = std::min(per_launch, G.B - s0);
    HIP_OR_FAIL(h, hipLaunchKernel(fn, dim3(nsys * G.K), dim3(NTR), fargs, (unsigned)dyn, h->stream));
  }
  ran = true;
  return HPCG_OK;
}

hpcg_status hpcg_set_factors_bridge(hpcg_handle h, const float* d_leafF, const float* d_bridgeU,
                                    const float* d_bridgeV, const float* d_cores, const float* d_gate) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  const Geom& G = h->G;
  if (!d_leafF || !d_gate || (G.levels > 0 && (!d_bridgeU || !d_bridgeV || !d_cores)))
    return fail(h, HPCG_ERR_INVALID_ARG, "factor pointer is NULL");
  HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.U, d_leafF, (size_t)G.B * G.K * LEAF * LEAF * 4,
                                hipMemcpyDeviceToDevice, h->stream));
  if (G.levels > 0)
    hipLaunchKernelGGL(k_expand_bridge, dim3(G.B * G.levels * G.K), dim3(NT), 0, h->stream, G, d_bridgeU, d_bridgeV,
                       d_cores, reinterpret_cast<float*>(h->ws + h->lay.W));
  HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.g, d_gate, (size_t)G.B * G.n * 4, hipMemcpyDeviceToDevice, h->stream));
  if (G.levels > 0) {
    // the format as given, for the native bridge apply
    const size_t bridge = (size_t)G.B * G.K * LEAF * RANK * 4;
    HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.Ub, d_bridgeU, bridge, hipMemcpyDeviceToDevice, h->stream));
    HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.Vb, d_bridgeV, bridge, hipMemcpyDeviceToDevice, h->stream));
    HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.Bc, d_cores, (size_t)G.B * h->B.ncores * RANK * RANK * 4,
                                  hipMemcpyDeviceToDevice, h->stream));
  }
  block_factor_pairs(h);
  hpcg_status s = check_launch(h, "bridge expansion launch");
  if (s != HPCG_OK) return s;
  h->factors_set = true;
  h->bridge_set = G.levels > 0;
  return HPCG_OK;
}

namespace {
hpcg_status apply_H(hpcg_ctx* h, const float* d_r, float* d_y);
}

hpcg_status hpcg_apply_M(hpcg_handle h, const float* d_r, float* d_y) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_r || !d_y) return fail(h, HPCG_ERR_INVALID_ARG, "vector pointer is NULL");
  if (d_r == d_y) return fail(h, HPCG_ERR_INVALID_ARG, "d_r and d_y must not alias");
  if (h->B.form == FORM_JACOBI) {
    const int N = h->G.B * h->G.n;
    hipLaunchKernelGGL(k_jacobi_apply, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, h->stream, d_r, h->B.dinv,
                       d_y, N);
    return check_launch(h, "hpcg_apply_M launch");
  }
  if (!h->factors_set) return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  if (h->B.form == FORM_SQUARED) {
    float* tmp = reinterpret_cast<float*>(h->ws + h->lay.ftmp);
    hpcg_status s = apply_H(h, d_r, tmp);
    if (s != HPCG_OK) return s;
    return apply_H(h, tmp, d_y);
  }
  return apply_H(h, d_r, d_y);
}

namespace {
// y = H r with the H-matrix factors (the apply paths of hpcg_apply_M).
hpcg_status apply_H(hpcg_ctx* h, const float* d_r, float* d_y) {
  if (h->apply_path == HPCG_APPLY_BRIDGE || (h->apply_path == HPCG_APPLY_AUTO && h->bridge_set)) {
    bool ran = false;
    hpcg_status s = run_bridge_apply(h, d_r, d_y, ran);
    if (s != HPCG_OK) return s;
    if (ran) {
      h->last_apply_path = HPCG_APPLY_BRIDGE;
      return HPCG_OK;
    }
    if (h->apply_path == HPCG_APPLY_BRIDGE)
      return fail(h, HPCG_ERR_STATE, h->bridge_set ? "bridge apply: a system has more leaves than compute units"
                                                   : "bridge apply: factors were not set with hpcg_set_factors_bridge");
  }
  if (h->apply_path != HPCG_APPLY_STREAMING) {
    bool ran = false;
    hpcg_status s = run_fused_apply(h, d_r, d_y, ran);
    if (s != HPCG_OK) return s;
    if (ran) {
      h->last_apply_path = HPCG_APPLY_FUSED;
      return HPCG_OK;
    }
    if (h->apply_path == HPCG_APPLY_FUSED)
      return fail(h, HPCG_ERR_SHAPE, "fused apply: a system has more leaves than co-resident workgroups");
  }
  h->last_apply_path = HPCG_APPLY_STREAMING;
  const Geom& G = h->Gapply;
  const size_t lds_r = restrict_lds_bytes(G), lds_p = prolong_lds_bytes<float>(G);
  hpcg_status s = allow_lds(h, reinterpret_cast<const void*>(&k_apply_restrict), lds_r);
  if (s == HPCG_OK) s = allow_lds(h, reinterpret_cast<const void*>(&k_apply_prolong), lds_p);
  if (s != HPCG_OK) return s;
  hipLaunchKernelGGL(k_apply_restrict, dim3(G.nblk), dim3(NT), lds_r, h->stream, G, h->B, d_r);
  hipLaunchKernelGGL(k_apply_prolong, dim3(G.nblk), dim3(NT), lds_p, h->stream, G, h->B, d_r, d_y);
  return check_launch(h, "hpcg_apply_M launch");
}
}  // namespace

hpcg_status hpcg_read_probe(const void* d_src, size_t bytes, float* d_sink, int32_t workgroups, void* stream) {
  if (!d_src || !d_sink) return fail(nullptr, HPCG_ERR_INVALID_ARG, "read probe: pointer is NULL");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(d_src) % 16)
    return fail(nullptr, HPCG_ERR_INVALID_ARG, "read probe: bytes and d_src must be positive multiples of 16");
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(nullptr, HPCG_ERR_INVALID_ARG, "read probe: bad grid");
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)workgroups), dim3(PROBE_NT), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const float4*>(d_src), bytes / 16,
                     d_sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(nullptr, e, "read probe launch");
  return HPCG_OK;
}

hpcg_status hpcg_trace_read(uint64_t* h_out, size_t count, int32_t clear) {
#ifdef HPCG_TRACE
  const size_t total = (size_t)kTraceItems * kTraceSlots;
  if (count > total) return fail(nullptr, HPCG_ERR_INVALID_ARG, "trace: count exceeds the table");
  if (count > 0) {
    if (!h_out) return fail(nullptr, HPCG_ERR_INVALID_ARG, "trace: h_out is NULL");
    hipError_t e = hipMemcpyFromSymbol(h_out, HIP_SYMBOL(trace_table), count * sizeof(uint64_t), 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(nullptr, e, "trace: hipMemcpyFromSymbol");
  }
  if (clear) {
    std::vector<uint64_t> zero(total, 0);
    hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(trace_table), zero.data(), total * sizeof(uint64_t), 0,
                                     hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(nullptr, e, "trace: hipMemcpyToSymbol");
  }
  return HPCG_OK;
#else
  (void)h_out;
  (void)count;
  (void)clear;
  return fail(nullptr, HPCG_ERR_STATE, "this build has no timeline (compile with HPCG_TRACE)");
#endif
}

hpcg_status hpcg_apply_status(hpcg_handle h) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  HIP_OR_FAIL(h, hipMemcpyAsync(h->h_ctl + 1, h->B.apply_abort, sizeof(int), hipMemcpyDeviceToHost, h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  if (h->h_ctl[1]) return apply_timed_out(h);
  return HPCG_OK;
}

hpcg_status hpcg_spmv(hpcg_handle h, const float* d_x, float* d_y) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_x || !d_y) return fail(h, HPCG_ERR_INVALID_ARG, "vector pointer is NULL");
  if (d_x == d_y) return fail(h, HPCG_ERR_INVALID_ARG, "d_x and d_y must not alias");
  const int N = h->G.B * h->G.n;
  const int grid = (N + SPMV_ROWS - 1) / SPMV_ROWS;
  hipLaunchKernelGGL(k_spmv, dim3(grid), dim3(NT), 0, h->stream, h->B.row_ptr, h->B.col, h->B.val, d_x, d_y, N);
  return check_launch(h, "hpcg_spmv launch");
}

namespace {

bool block_nrhs_ok(int32_t nrhs) { return nrhs >= BNC && nrhs <= 1024 && nrhs % BNC == 0; }

// 16-column tiles per workgroup of the block apply (1, 2 or 4): doubled while
// they divide nrhs and the grid would still hold more workgroups than the
// device has compute units, so that each factor operand a workgroup loads
// feeds more products without leaving compute units idle.
int block_nct(const hpcg_ctx* h, int32_t nrhs) {
  const int64_t leaves = (int64_t)h->G.B * h->G.K;
  int nct = 1;
  while (nct < 4 && nrhs % (2 * nct * BNC) == 0 && leaves * (nrhs / (nct * BNC)) > h->num_cu) nct *= 2;
  return nct;
}

BlockGeom block_geom(const hpcg_ctx* h, int32_t nrhs) {
  BlockGeom bg;
  bg.n = h->G.n;
  bg.K = h->G.K;
  bg.levels = h->G.levels;
  bg.B = h->G.B;
  bg.nrhs = nrhs;
  bg.tiles = nrhs / (BNC * block_nct(h, nrhs));
  return bg;
}

// Leaf stage and restriction in workgroups of their own: with tile levels and
// at most two column tiles per workgroup (four would not fit two workgroups'
// registers on a compute unit), when asked, or (automatic) while the items
// leave compute units idle.
bool block_split(const hpcg_ctx* h, int32_t nrhs) {
  if (h->G.levels == 0 || h->block_split == 1 || block_nct(h, nrhs) > 2) return false;
  if (h->block_split == 2) return true;
  const BlockGeom bg = block_geom(h, nrhs);
  return (int64_t)h->G.B * h->G.K * bg.tiles < h->num_cu;
}

size_t block_half_bytes(const hpcg_ctx* h, int32_t nrhs) {
  return align_up((size_t)h->G.B * h->G.levels * h->G.K * RANK * nrhs * 4);
}

// The three launches of Y = M R for a block (scratch Q and H of
// block_half_bytes each; unused without tile levels).
// The block solve passes upd (the leaf stage takes its residual update) and,
// with tile levels, dot (the prolongation leaves its r.z partials); the plain
// block apply passes neither.
hpcg_status launch_block_apply(hpcg_ctx* h, int32_t nrhs, const float* d_R, float* d_Y, float* Q, float* H,
                               hipStream_t stream, const BlockUpd* upd = nullptr, const BlockDot* dot = nullptr) {
  const BlockGeom bg = block_geom(h, nrhs);
  const int nct = block_nct(h, nrhs);
  const int grid = h->G.B * h->G.K * bg.tiles;
  const BlockUpd up = upd ? *upd : BlockUpd{};
  const BlockDot dt = dot ? *dot : BlockDot{};
  const bool sp = block_split(h, nrhs);
  const BlockFactors16 f16 = block_factors16(h);
  // (block_split() holds only where a split instantiation exists: LV > 0, N < 4)
#define HPCG_BLOCK_RESTRICT_UPD(LV, N, UP)                                                               \
  do {                                                                                                   \
    if (sp && LV > 0 && N < 4)                                                                           \
      hipLaunchKernelGGL((k_block_restrict<LV, N, UP, (LV > 0 && N < 4)>), dim3(2 * grid), dim3(BNT), 0, \
                         stream, bg, f16, h->B.g, d_R, d_Y, Q, up);                                      \
    else                                                                                                 \
      hipLaunchKernelGGL((k_block_restrict<LV, N, UP, false>), dim3(grid), dim3(BNT), 0, stream, bg,      \
                         f16, h->B.g, d_R, d_Y, Q, up);                                                  \
  } while (0)
#define HPCG_BLOCK_RESTRICT_N(LV, N)                                                                     \
  do {                                                                                                   \
    if (upd) HPCG_BLOCK_RESTRICT_UPD(LV, N, true);                                                       \
    else HPCG_BLOCK_RESTRICT_UPD(LV, N, false);                                                          \
  } while (0)
  switch (h->G.levels) {
#define HPCG_BLOCK_RESTRICT(LV)                                                                          \
    case LV:                                                                                             \
      if (nct == 4) HPCG_BLOCK_RESTRICT_N(LV, 4);                                                        \
      else if (nct == 2) HPCG_BLOCK_RESTRICT_N(LV, 2);                                                   \
      else HPCG_BLOCK_RESTRICT_N(LV, 1);                                                                 \
      break;
    HPCG_BLOCK_RESTRICT(0) HPCG_BLOCK_RESTRICT(1) HPCG_BLOCK_RESTRICT(2) HPCG_BLOCK_RESTRICT(3)
    HPCG_BLOCK_RESTRICT(4) HPCG_BLOCK_RESTRICT(5) HPCG_BLOCK_RESTRICT(6) HPCG_BLOCK_RESTRICT(7)
    HPCG_BLOCK_RESTRICT(8)
#undef HPCG_BLOCK_RESTRICT
#undef HPCG_BLOCK_RESTRICT_N
#undef HPCG_BLOCK_RESTRICT_UPD
    default: return fail(h, HPCG_ERR_SHAPE, "levels out of range");
  }
  if (h->G.levels > 0) {
    size_t sys_total = 0;   // level 0 needs no half sums
    for (int l = 1; l < h->G.levels; ++l) sys_total += (size_t)(h->G.K >> l) * RANK * nrhs * halfsum_runs(l);
    if (sys_total > 0)
      hipLaunchKernelGGL(k_block_halfsum, dim3((unsigned)((sys_total + 255) / 256), (unsigned)std::min(h->G.B, 65535)),
                         dim3(256), 0, stream, bg, Q, H);
#define HPCG_BLOCK_PROLONG_N(LV, N)                                                                     \
  do {                                                                                                  \
    if (dot)                                                                                            \
      hipLaunchKernelGGL((k_block_prolong<LV, N, true>), dim3(grid), dim3(BNT), 0, stream, bg, f16, Q, H, \
                         d_Y, dt);                                                                      \
    else                                                                                                \
      hipLaunchKernelGGL((k_block_prolong<LV, N, false>), dim3(grid), dim3(BNT), 0, stream, bg, f16, Q,   \
                         H, d_Y, dt);                                                                   \
  } while (0)
    switch (h->G.levels) {
#define HPCG_BLOCK_PROLONG(LV)                                                                          \
      case LV:                                                                                          \
        if (nct == 4) HPCG_BLOCK_PROLONG_N(LV, 4);                                                      \
        else if (nct == 2) HPCG_BLOCK_PROLONG_N(LV, 2);                                                 \
        else HPCG_BLOCK_PROLONG_N(LV, 1);                                                               \
        break;
      HPCG_BLOCK_PROLONG(1) HPCG_BLOCK_PROLONG(2) HPCG_BLOCK_PROLONG(3) HPCG_BLOCK_PROLONG(4)
      HPCG_BLOCK_PROLONG(5) HPCG_BLOCK_PROLONG(6) HPCG_BLOCK_PROLONG(7) HPCG_BLOCK_PROLONG(8)
#undef HPCG_BLOCK_PROLONG
#undef HPCG_BLOCK_PROLONG_N
      default: return fail(h, HPCG_ERR_SHAPE, "levels out of range");
    }
  }
  return HPCG_OK;
}

}  // namespace

size_t hpcg_block_workspace_bytes(hpcg_handle h, int32_t nrhs) {
  if (!h || !block_nrhs_ok(nrhs)) return 0;
  return 2 * block_half_bytes(h, nrhs) + kAlign;
}

hpcg_status hpcg_apply_M_block(hpcg_handle h, const float* d_R, float* d_Y, int32_t nrhs, void* d_work,
                               size_t work_bytes) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_R || !d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "block pointer is NULL");
  if (d_R == d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "d_R and d_Y must not alias");
  if (!block_nrhs_ok(nrhs)) return fail(h, HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]");
  if ((reinterpret_cast<uintptr_t>(d_R) | reinterpret_cast<uintptr_t>(d_Y)) % 16)
    return fail(h, HPCG_ERR_INVALID_ARG, "d_R and d_Y must be 16-byte aligned");
  if (!h->factors_set) return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  if (h->B.form != FORM_DIRECT) return fail(h, HPCG_ERR_STATE, "the block apply runs the direct form (M = H) only");
  const size_t half = block_half_bytes(h, nrhs);
  if (h->G.levels > 0) {
    if (!d_work) return fail(h, HPCG_ERR_INVALID_ARG, "d_work is NULL");
    if (work_bytes < hpcg_block_workspace_bytes(h, nrhs)) return fail(h, HPCG_ERR_WORKSPACE, "block workspace too small");
  }
  char* wk = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(d_work)));
  hpcg_status s = launch_block_apply(h, nrhs, d_R, d_Y, reinterpret_cast<float*>(wk),
                                     reinterpret_cast<float*>(wk + half), h->stream);
  if (s != HPCG_OK) return s;
  return check_launch(h, "hpcg_apply_M_block launch");
}

hpcg_status hpcg_apply_M_block_noalloc(hpcg_handle h, const float* d_R, float* d_Y, int32_t nrhs) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_R || !d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "block pointer is NULL");
  if (d_R == d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "d_R and d_Y must not alias");
  if (!block_nrhs_ok(nrhs)) return fail(h, HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]");
  if ((reinterpret_cast<uintptr_t>(d_R) | reinterpret_cast<uintptr_t>(d_Y)) % 16)
    return fail(h, HPCG_ERR_INVALID_ARG, "d_R and d_Y must be 16-byte aligned");
  if (!h->factors_set) return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  if (h->B.form != FORM_DIRECT) return fail(h, HPCG_ERR_STATE, "the block apply runs the direct form (M = H) only");
  const size_t half = block_half_bytes(h, nrhs);
  if (h->G.levels > 0 && 2 * half > kNoAllocScratchBytes)
    return fail(h, HPCG_ERR_WORKSPACE,
                "allocation-free block apply: batch * levels * K * 32 * nrhs * 4 bytes, twice, exceed its fixed "
                "32 MiB scratch; use hpcg_apply_M_block with a caller workspace");
  if (!h->d_scratch) return fail(h, HPCG_ERR_STATE, "scratch address unknown");
  hpcg_status s = launch_block_apply(h, nrhs, d_R, d_Y, reinterpret_cast<float*>(h->d_scratch),
                                     reinterpret_cast<float*>(h->d_scratch + half), h->stream);
  if (s != HPCG_OK) return s;
  return check_launch(h, "hpcg_apply_M_block_noalloc launch");
}

hpcg_status hpcg_spmv_block(hpcg_handle h, const float* d_X, float* d_Y, int32_t nrhs) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_X || !d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "block pointer is NULL");
  if (d_X == d_Y) return fail(h, HPCG_ERR_INVALID_ARG, "d_X and d_Y must not alias");
  if (!block_nrhs_ok(nrhs)) return fail(h, HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]");
  if ((reinterpret_cast<uintptr_t>(d_X) | reinterpret_cast<uintptr_t>(d_Y)) % 16)
    return fail(h, HPCG_ERR_INVALID_ARG, "d_X and d_Y must be 16-byte aligned");
  const size_t threads = (size_t)h->G.B * h->G.n * (nrhs / 4);
  hipLaunchKernelGGL(k_spmv_block, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, h->stream, h->B.row_ptr,
                     h->B.col, h->B.val, d_X, d_Y, h->G.B * h->G.n, nrhs);
  return check_launch(h, "hpcg_spmv_block launch");
}

namespace {

// Sub-buffers of the block solve's caller-provided work buffer.
struct BlockSolveLayout {
  size_t R, Z, P, Q, scratchQ, scratchH, part, part2, cs, ctr, total;
};

BlockSolveLayout block_solve_layout(const hpcg_ctx* h, int32_t nrhs) {
  BlockSolveLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const size_t vec = (size_t)h->G.B * h->G.n * nrhs * 4;
  L.R = take(vec);
  L.Z = take(vec);
  L.P = take(vec);
  L.Q = take(vec);
  const size_t half = h->G.levels > 0 ? block_half_bytes(h, nrhs) : 0;
  L.scratchQ = take(half);
  L.scratchH = take(half);
  L.part = take((size_t)h->G.B * (h->G.n / BS_ROWS) * nrhs * 8);
  L.part2 = take((size_t)h->G.B * (h->G.n / BS_ROWS) * nrhs * 8);
  L.cs = take((size_t)h->G.B * nrhs * sizeof(ColState));
  L.ctr = take(256);
  L.total = off;
  return L;
}

// One block-PCG iteration (the steps of hpcg_bsolve.hpp) on `stream`.
hpcg_status block_iteration(hpcg_ctx* h, int32_t nrhs, char* wk, const BlockSolveLayout& L, double* d_X,
                            double tol, int32_t maxit, hipStream_t stream) {
  const Geom& G = h->G;
  float* R = reinterpret_cast<float*>(wk + L.R);
  float* Z = reinterpret_cast<float*>(wk + L.Z);
  float* P = reinterpret_cast<float*>(wk + L.P);
  float* Q = reinterpret_cast<float*>(wk + L.Q);
  double* part = reinterpret_cast<double*>(wk + L.part);
  double* part2 = reinterpret_cast<double*>(wk + L.part2);
  ColState* cs = reinterpret_cast<ColState*>(wk + L.cs);
  const int rblocks = G.n / BS_ROWS;   // row blocks per system
  const dim3 rows_grid((unsigned)(G.B * rblocks), (unsigned)((nrhs + BS_COLS - 1) / BS_COLS));
  const dim3 spmv_grid((unsigned)(G.B * G.K), (unsigned)((nrhs + BS_SPMV_COLS - 1) / BS_SPMV_COLS));
  const dim3 dir_grid((unsigned)(G.B * G.K), (unsigned)((nrhs + BS_DIR_COLS - 1) / BS_DIR_COLS));
  // Q = A P and the p.q partials per leaf
  hipLaunchKernelGGL(k_bs_spmv_dot, spmv_grid, dim3(BS_SPMV_NT), 0, stream, h->B.row_ptr, h->B.col, h->B.val, P, Q,
                     part, nrhs);
  // the PQ step, R -= alpha Q and the r.r partials in the leaf stage; the r.z
  // partials in the prolongation (per leaf), or, without tile levels, by a pass
  // of their own
  const BlockUpd upd{cs, part, Q, R, part2};
  const BlockDot dot{R, part};
  hpcg_status s = launch_block_apply(h, nrhs, R, Z, reinterpret_cast<float*>(wk + L.scratchQ),
                                     reinterpret_cast<float*>(wk + L.scratchH), stream, &upd, &dot);
  if (s != HPCG_OK) return s;
  int rz_blocks = G.K;
  if (G.levels == 0) {
    hipLaunchKernelGGL(k_bs_dot, rows_grid, dim3(BS_NT), 0, stream, R, Z, part, nrhs);
    rz_blocks = rblocks;
  }
  // the RRZ step, X += alpha P and P = Z + beta P
  const BsRrz rrz{part, rz_blocks, part2, G.K, tol, maxit};
  hipLaunchKernelGGL(k_bs_direction<true>, dir_grid, dim3(BS_DIR_NT), 0, stream, cs, Z, P, d_X, nrhs, G.K, rrz);
  return HPCG_OK;
}

}  // namespace

size_t hpcg_block_solve_workspace_bytes(hpcg_handle h, int32_t nrhs) {
  if (!h || !block_nrhs_ok(nrhs)) return 0;
  return block_solve_layout(h, nrhs).total + kAlign;
}

hpcg_status hpcg_solve_block(hpcg_handle h, const float* d_B, double* d_X, int32_t nrhs, double tol, int32_t maxit,
                             void* d_work, size_t work_bytes, int32_t* h_iters, double* h_relres) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_B || !d_X || !d_work) return fail(h, HPCG_ERR_INVALID_ARG, "block or work pointer is NULL");
  if (!block_nrhs_ok(nrhs)) return fail(h, HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]");
  if ((reinterpret_cast<uintptr_t>(d_B) | reinterpret_cast<uintptr_t>(d_X)) % 16)
    return fail(h, HPCG_ERR_INVALID_ARG, "d_B and d_X must be 16-byte aligned");
  if (!(tol > 0.0) || !(tol < 1.0)) return fail(h, HPCG_ERR_INVALID_ARG, "tol must lie in (0, 1)");
  if (maxit < 1) return fail(h, HPCG_ERR_INVALID_ARG, "maxit must be >= 1");
  if (!h->factors_set) return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  if (h->B.form != FORM_DIRECT) return fail(h, HPCG_ERR_STATE, "the block solve runs the direct form (M = H) only");
  if (work_bytes < hpcg_block_solve_workspace_bytes(h, nrhs)) return fail(h, HPCG_ERR_WORKSPACE, "block work buffer too small");
  const Geom& G = h->G;
  const BlockSolveLayout L = block_solve_layout(h, nrhs);
  char* wk = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(d_work)));
  float* R = reinterpret_cast<float*>(wk + L.R);
  float* Z = reinterpret_cast<float*>(wk + L.Z);
  float* P = reinterpret_cast<float*>(wk + L.P);
  double* part = reinterpret_cast<double*>(wk + L.part);
  ColState* cs = reinterpret_cast<ColState*>(wk + L.cs);
  int* ctr = reinterpret_cast<int*>(wk + L.ctr);
  int* hflag = h->h_flag + 16;
  int* dflag = h->d_flag + 16;
  const int rblocks = G.n / BS_ROWS;   // row blocks per system
  const dim3 rows_grid((unsigned)(G.B * rblocks), (unsigned)((nrhs + BS_COLS - 1) / BS_COLS));
  const int ncol = G.B * nrhs;
  const dim3 sc_grid((unsigned)(G.B * (nrhs / BS_SC_C)));

  // the recorded iterations depend on the buffers, nrhs, tol, maxit, the unroll
  // and the block split
  if (!h->bs_gexec || h->bs_key[0] != d_X || h->bs_key[1] != wk || h->bs_nrhs != nrhs || h->bs_tol != tol ||
      h->bs_maxit != maxit || h->bs_unroll != h->unroll || h->bs_split != h->block_split) {
    if (h->bs_gexec) (void)hipGraphExecDestroy(h->bs_gexec);
    if (h->bs_graph) (void)hipGraphDestroy(h->bs_graph);
    h->bs_gexec = nullptr;
    h->bs_graph = nullptr;
    HIP_OR_FAIL(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
    hpcg_status s = HPCG_OK;
    for (int j = 0; j < h->unroll && s == HPCG_OK; ++j) s = block_iteration(h, nrhs, wk, L, d_X, tol, maxit, h->cap_stream);
    if (s == HPCG_OK)
      hipLaunchKernelGGL(k_bs_progress, dim3(1), dim3(256), 0, h->cap_stream, cs, ncol, ctr, dflag);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(h->cap_stream, &g);
    if (s != HPCG_OK) { if (g) (void)hipGraphDestroy(g); return s; }
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamEndCapture (block solve)");
    h->bs_graph = g;
    const hipError_t e2 = hipGraphInstantiate(&h->bs_gexec, h->bs_graph, nullptr, nullptr, 0);
    if (e2 != hipSuccess) return hip_fail(h, e2, "hipGraphInstantiate (block solve)");
    h->bs_key[0] = d_X;
    h->bs_key[1] = wk;
    h->bs_nrhs = nrhs;
    h->bs_tol = tol;
    h->bs_maxit = maxit;
    h->bs_unroll = h->unroll;
    h->bs_split = h->block_split;
  }

  // R = B, X = 0, ||B_j||, Z = M R, rz, P = Z
  __atomic_store_n(hflag, 0, __ATOMIC_RELEASE);
  hipLaunchKernelGGL(k_bs_reset, dim3(1), dim3(64), 0, h->stream, ctr, dflag);
  hipLaunchKernelGGL(k_bs_init, rows_grid, dim3(BS_NT), 0, h->stream, d_B, R, d_X, part, nrhs);
  hipLaunchKernelGGL(k_bs_scalars<BS_INIT>, sc_grid, dim3(BS_SC_C * BS_SC_G), 0, h->stream, cs, part, G.B, nrhs, rblocks);
  hpcg_status s = launch_block_apply(h, nrhs, R, Z, reinterpret_cast<float*>(wk + L.scratchQ),
                                     reinterpret_cast<float*>(wk + L.scratchH), h->stream);
  if (s != HPCG_OK) return s;
  hipLaunchKernelGGL(k_bs_dot, rows_grid, dim3(BS_NT), 0, h->stream, R, Z, part, nrhs);
  hipLaunchKernelGGL(k_bs_scalars<BS_RZ0>, sc_grid, dim3(BS_SC_C * BS_SC_G), 0, h->stream, cs, part, G.B, nrhs, rblocks);
  const dim3 dir_grid((unsigned)(G.B * G.K), (unsigned)((nrhs + BS_DIR_COLS - 1) / BS_DIR_COLS));
  hipLaunchKernelGGL(k_bs_direction<false>, dir_grid, dim3(BS_DIR_NT), 0, h->stream, cs, Z, P, d_X, nrhs, G.K, BsRrz{});
  s = check_launch(h, "block solve setup launch");
  if (s != HPCG_OK) return s;

  // replays, two in flight, until no column is running (or maxit is spent)
  const int max_replays = (maxit + h->unroll - 1) / h->unroll;
  int launched = 0, seen = 0;
  bool done = false;
  while (!done) {
    while (launched < max_replays && launched - seen < 2) {
      HIP_OR_FAIL(h, hipGraphLaunch(h->bs_gexec, h->stream));
      ++launched;
    }
    unsigned spins = 0;
    for (;;) {
      const int f = __atomic_load_n(hflag, __ATOMIC_ACQUIRE);
      if ((f >> 1) > seen) {
        seen = f >> 1;
        done = (f & 1) != 0 || seen >= max_replays;
        break;
      }
      if ((++spins & 1023u) == 0) {
        const hipError_t q = hipStreamQuery(h->stream);
        if (q == hipSuccess) {
          const int f2 = __atomic_load_n(hflag, __ATOMIC_ACQUIRE);
          if ((f2 >> 1) <= seen) return fail(h, HPCG_ERR_HIP, "block solve: stream drained without progress flag");
        } else if (q != hipErrorNotReady) {
          return hip_fail(h, q, "hipStreamQuery");
        }
      }
    }
  }
  std::vector<ColState> host((size_t)ncol);
  HIP_OR_FAIL(h, hipMemcpyAsync(host.data(), cs, host.size() * sizeof(ColState), hipMemcpyDeviceToHost, h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  bool any_break = false, any_nc = false;
  for (int i = 0; i < ncol; ++i) {
    if (h_iters) h_iters[i] = host[i].iters;
    if (h_relres) h_relres[i] = host[i].relres;
    if (host[i].status == ST_BREAKDOWN) any_break = true;
    else if (host[i].status != ST_CONVERGED) any_nc = true;
  }
  if (any_break) return fail(h, HPCG_ERR_BREAKDOWN, "breakdown in some column: p.Ap or r.Mr not positive and finite");
  if (any_nc) return fail(h, HPCG_ERR_NOT_CONVERGED, "maxit reached before the tolerance in some column");
  return HPCG_OK;
}

namespace {

// One PCG solve with the configured engine; fills the per-system state copy
// h->h_st (status, iterations, recursive residual) and returns the call status.
hpcg_status solve_core(hpcg_ctx* h, const float* d_b, double* d_x, double tol, int32_t maxit) {
  const Geom G = h->G;
  const size_t N = (size_t)G.B * G.n;
  h->B.tol = tol;
  h->B.maxit = maxit;
  HIP_OR_FAIL(h, hipMemcpyAsync(h->ws + h->lay.b, d_b, N * 4, hipMemcpyDeviceToDevice, h->stream));
  hpcg_status s = HPCG_OK;
  bool ran = false;
  const bool f32 = (h->prec == HPCG_PREC_VEC32);
  // AUTO runs the register-resident persistent engine when every leaf of a
  // system gets its own CU (K <= #CUs; a larger batch runs in groups of whole
  // systems, one launch each): the factors then never leave VGPRs and an
  // iteration costs two barriers among the system's workgroups.  Otherwise
  // (and for the Jacobi form) the graph engine runs: a kernel boundary inside
  // a graph (about 2 us) is cheaper than an agent-scope barrier over a full
  // grid of streaming workgroups (about 10 us at 256 workgroups, dominated by
  // the per-workgroup L2 writeback and invalidate of the release/acquire
  // fences).
  if (h->engine_opt == HPCG_ENGINE_PERSISTENT || h->engine_opt == HPCG_ENGINE_AUTO) {
    s = f32 ? run_resident<float>(h, ran) : run_resident<double>(h, ran);
    if (s != HPCG_OK) return s;
    if (!ran && h->engine_opt == HPCG_ENGINE_PERSISTENT)
      s = f32 ? run_persistent<float>(h, ran) : run_persistent<double>(h, ran);
    if (s != HPCG_OK) return s;
    if (!ran && h->engine_opt == HPCG_ENGINE_PERSISTENT)
      return fail(h, HPCG_ERR_SHAPE, h->B.form != FORM_DIRECT
                                         ? "the streaming persistent engine runs the direct form only"
                                         : "persistent engine: device does not support a co-resident grid for this partition");
    if (ran) h->last_engine = HPCG_ENGINE_PERSISTENT;
  }
  if (!ran) {
    s = f32 ? run_graph<float>(h) : run_graph<double>(h);
    if (s != HPCG_OK) return s;
    h->last_engine = HPCG_ENGINE_GRAPH;
  }
  hipLaunchKernelGGL(k_copy_x, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, h->stream, h->B.x, d_x, (int)N);
  s = check_launch(h, "copy-out launch");
  if (s != HPCG_OK) return s;
  HIP_OR_FAIL(h, hipMemcpyAsync(h->h_st, h->B.st, (size_t)G.B * sizeof(SysState), hipMemcpyDeviceToHost, h->stream));
  HIP_OR_FAIL(h, hipMemcpyAsync(h->h_ctl, h->B.abort_flag, 2 * sizeof(int), hipMemcpyDeviceToHost, h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  if (h->h_ctl[0])
    return fail(h, HPCG_ERR_HIP, "a bounded wait of the persistent solve ran out (workgroups not co-resident, "
                                 "or HPCG_OPT_POLL_LIMIT below the exchange latency)");
  if (h->h_ctl[1]) return apply_timed_out(h);
  return HPCG_OK;
}

hpcg_status check_solve_args(hpcg_ctx* h, const float* d_b, double* d_x, double tol, int32_t maxit) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!d_b || !d_x) return fail(h, HPCG_ERR_INVALID_ARG, "vector pointer is NULL");
  if (!(tol > 0.0) || !(tol < 1e300)) return fail(h, HPCG_ERR_INVALID_ARG, "tol must be positive and finite");
  if (maxit < 1) return fail(h, HPCG_ERR_INVALID_ARG, "maxit must be >= 1");
  if (!h->factors_set && h->B.form != FORM_JACOBI)
    return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  return HPCG_OK;
}

}  // namespace

hpcg_status hpcg_solve(hpcg_handle h, const float* d_b, double* d_x, double tol, int32_t maxit,
                       int32_t* h_iters, double* h_relres) {
  hpcg_status s = check_solve_args(h, d_b, d_x, tol, maxit);
  if (s != HPCG_OK) return s;
  h->last_fallback = 0;
  s = solve_core(h, d_b, d_x, tol, maxit);
  if (s != HPCG_OK) return s;
  if (h->fallback && h->B.form != FORM_JACOBI) {
    bool broke = false;
    for (int i = 0; i < h->G.B; ++i) broke |= (h->h_st[i].status == ST_BREAKDOWN);
    if (broke) {
      // the preconditioner is not SPD for some system: solve again with Jacobi
      // (the streaming persistent engine runs the direct form only)
      const int form = h->B.form, engine = h->engine_opt;
      h->B.form = FORM_JACOBI;
      if (engine == HPCG_ENGINE_PERSISTENT) h->engine_opt = HPCG_ENGINE_AUTO;
      s = solve_core(h, d_b, d_x, tol, maxit);
      h->B.form = form;
      h->engine_opt = engine;
      if (s != HPCG_OK) return s;
      h->last_fallback = 1;
    }
  }
  bool any_break = false, any_nc = false;
  for (int i = 0; i < h->G.B; ++i) {
    const SysState& st = h->h_st[i];
    h->last_status[i] = st.status;
    if (h_iters) h_iters[i] = st.iters;
    if (h_relres) h_relres[i] = st.relres;
    if (st.status == ST_BREAKDOWN) any_break = true;
    else if (st.status != ST_CONVERGED) any_nc = true;
  }
  if (any_break) return fail(h, HPCG_ERR_BREAKDOWN, "breakdown: p.Ap or r.Mr not positive and finite");
  if (any_nc) return fail(h, HPCG_ERR_NOT_CONVERGED, "maxit reached before the tolerance");
  return HPCG_OK;
}

hpcg_status hpcg_solve_refined(hpcg_handle h, const float* d_b, double* d_x, double tol, int32_t maxit,
                               double inner_tol, int32_t max_outer, int32_t* h_iters, int32_t* h_outer,
                               double* h_relres) {
  hpcg_status s = check_solve_args(h, d_b, d_x, tol, maxit);
  if (s != HPCG_OK) return s;
  if (!(inner_tol > 0.0) || !(inner_tol < 1.0)) return fail(h, HPCG_ERR_INVALID_ARG, "inner_tol must lie in (0, 1)");
  if (max_outer < 1) return fail(h, HPCG_ERR_INVALID_ARG, "max_outer must be >= 1");
  const Geom G = h->G;
  const int N = G.B * G.n;
  const unsigned grid = (unsigned)((N + 255) / 256);
  double* r = reinterpret_cast<double*>(h->ws + h->lay.fr);
  double* d = reinterpret_cast<double*>(h->ws + h->lay.fd);
  float* rhs = reinterpret_cast<float*>(h->ws + h->lay.frhs);
  double* sumsq = reinterpret_cast<double*>(h->ws + h->lay.fsc);
  double* inv = sumsq + G.B;
  double* scale = inv + G.B;
  std::vector<double> hs(G.B), bn2(G.B), hinv(G.B), hscale(G.B), rel(G.B, 1.0);
  std::vector<int> its(G.B, 0), outer(G.B, 0), status(G.B, ST_RUNNING);
  const Bufs& B = h->B;
  HIP_OR_FAIL(h, hipMemsetAsync(d_x, 0, (size_t)N * 8, h->stream));
  bool any_break = false;
  for (int o = 0;; ++o) {
    // true residual of the current x, in fp64
    hipLaunchKernelGGL(k_residual64, dim3(grid), dim3(256), 0, h->stream, B.row_ptr, B.col, B.val, d_b, d_x, r, N);
    hipLaunchKernelGGL(k_sys_sumsq, dim3(G.B), dim3(NT), 0, h->stream, r, G.n, sumsq);
    s = check_launch(h, "refinement residual launch");
    if (s != HPCG_OK) return s;
    HIP_OR_FAIL(h, hipMemcpyAsync(hs.data(), sumsq, (size_t)G.B * 8, hipMemcpyDeviceToHost, h->stream));
    HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
    if (o == 0) bn2 = hs;
    bool all_done = true;
    for (int i = 0; i < G.B; ++i) {
      if (status[i] != ST_RUNNING) { hinv[i] = 0.0; continue; }
      rel[i] = bn2[i] > 0.0 ? std::sqrt(hs[i] / bn2[i]) : 0.0;
      if (rel[i] <= tol) { status[i] = ST_CONVERGED; hinv[i] = 0.0; continue; }
      if (o >= max_outer || its[i] >= maxit) { status[i] = ST_NOT_CONVERGED; hinv[i] = 0.0; continue; }
      all_done = false;
      hscale[i] = std::sqrt(hs[i]);
      hinv[i] = 1.0 / hscale[i];
    }
    if (all_done) break;
    // inner solve of A d = r / ||r|| with the configured engine and precision
    HIP_OR_FAIL(h, hipMemcpyAsync(inv, hinv.data(), (size_t)G.B * 8, hipMemcpyHostToDevice, h->stream));
    hipLaunchKernelGGL(k_scale_rhs, dim3(grid), dim3(256), 0, h->stream, r, inv, rhs, G.n, N);
    int budget = 0;
    for (int i = 0; i < G.B; ++i)
      if (status[i] == ST_RUNNING) budget = std::max(budget, maxit - its[i]);
    s = solve_core(h, rhs, d, inner_tol, std::max(budget, 1));
    if (s != HPCG_OK) return s;
    for (int i = 0; i < G.B; ++i) {
      if (status[i] != ST_RUNNING) { hscale[i] = 0.0; continue; }
      const SysState& st = h->h_st[i];
      its[i] += st.iters;
      outer[i] = o + 1;
      if (st.status == ST_BREAKDOWN) { status[i] = ST_BREAKDOWN; any_break = true; hscale[i] = 0.0; }
    }
    HIP_OR_FAIL(h, hipMemcpyAsync(scale, hscale.data(), (size_t)G.B * 8, hipMemcpyHostToDevice, h->stream));
    hipLaunchKernelGGL(k_add_scaled, dim3(grid), dim3(256), 0, h->stream, d_x, d, scale, G.n, N);
    s = check_launch(h, "refinement update launch");
    if (s != HPCG_OK) return s;
  }
  bool any_nc = false;
  for (int i = 0; i < G.B; ++i) {
    h->last_status[i] = status[i];
    if (h_iters) h_iters[i] = its[i];
    if (h_outer) h_outer[i] = outer[i];
    if (h_relres) h_relres[i] = rel[i];
    if (status[i] == ST_NOT_CONVERGED) any_nc = true;
  }
  if (any_break) return fail(h, HPCG_ERR_BREAKDOWN, "breakdown in an inner solve");
  if (any_nc) return fail(h, HPCG_ERR_NOT_CONVERGED, "outer or inner iteration budget reached before the tolerance");
  return HPCG_OK;
}

namespace {

// Number of eigenvalues below x of the symmetric tridiagonal matrix with
// diagonal a and off-diagonal b (Sturm sequence of the LDL^T pivots).
int sturm_count(const std::vector<double>& a, const std::vector<double>& b, double x) {
  int count = 0;
  double d = 1.0;
  for (size_t i = 0; i < a.size(); ++i) {
    const double off = i ? b[i - 1] * b[i - 1] : 0.0;
    d = a[i] - x - (i ? off / d : 0.0);
    if (d == 0.0) d = -1e-300;
    if (d < 0.0) ++count;
  }
  return count;
}

// k-th smallest eigenvalue (0-based) by bisection inside the Gershgorin interval.
double tridiag_eig(const std::vector<double>& a, const std::vector<double>& b, int k) {
  double lo = 0.0, hi = 0.0;
  for (size_t i = 0; i < a.size(); ++i) {
    const double r = (i ? std::fabs(b[i - 1]) : 0.0) + (i + 1 < a.size() ? std::fabs(b[i]) : 0.0);
    lo = i ? std::min(lo, a[i] - r) : a[i] - r;
    hi = i ? std::max(hi, a[i] + r) : a[i] + r;
  }
  for (int iter = 0; iter < 200 && hi - lo > 1e-15 * std::max(std::fabs(lo), std::fabs(hi)); ++iter) {
    const double mid = 0.5 * (lo + hi);
    if (sturm_count(a, b, mid) > k) hi = mid;
    else lo = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

hpcg_status hpcg_estimate_spectrum(hpcg_handle h, int32_t steps, double* h_lmin, double* h_lmax) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (steps < 2 || steps > 200) return fail(h, HPCG_ERR_INVALID_ARG, "steps must lie in [2, 200]");
  if (!h->factors_set) return fail(h, HPCG_ERR_STATE, "hpcg_set_factors has not been called");
  const size_t N = (size_t)h->G.B * h->G.n;
  float* d_in = reinterpret_cast<float*>(h->ws + h->lay.frhs);
  float* d_out = reinterpret_cast<float*>(h->ws + h->lay.w);
  std::vector<std::vector<double>> V;
  std::vector<double> alpha, beta, v(N), w(N);
  std::vector<float> buf(N);
  // seeded start vector (xorshift, uniform in [-1, 1))
  uint64_t st = 0x9e3779b97f4a7c15ULL;
  double nrm = 0.0;
  for (size_t i = 0; i < N; ++i) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    v[i] = (double)(st >> 11) * (1.0 / 4503599627370496.0) - 1.0;
    nrm += v[i] * v[i];
  }
  nrm = std::sqrt(nrm);
  for (auto& e : v) e /= nrm;
  for (int j = 0; j < steps; ++j) {
    V.push_back(v);
    for (size_t i = 0; i < N; ++i) buf[i] = (float)v[i];
    HIP_OR_FAIL(h, hipMemcpyAsync(d_in, buf.data(), N * 4, hipMemcpyHostToDevice, h->stream));
    hpcg_status s = apply_H(h, d_in, d_out);
    if (s != HPCG_OK) return s;
    HIP_OR_FAIL(h, hipMemcpyAsync(buf.data(), d_out, N * 4, hipMemcpyDeviceToHost, h->stream));
    HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
    for (size_t i = 0; i < N; ++i) w[i] = buf[i];
    double a = 0.0;
    for (size_t i = 0; i < N; ++i) a += w[i] * v[i];
    alpha.push_back(a);
    // full reorthogonalization against every Lanczos vector, twice
    for (int pass = 0; pass < 2; ++pass)
      for (const auto& u : V) {
        double c = 0.0;
        for (size_t i = 0; i < N; ++i) c += w[i] * u[i];
        for (size_t i = 0; i < N; ++i) w[i] -= c * u[i];
      }
    double bn = 0.0;
    for (size_t i = 0; i < N; ++i) bn += w[i] * w[i];
    bn = std::sqrt(bn);
    if (j + 1 == steps || bn <= 1e-12 * std::fabs(a)) break;
    beta.push_back(bn);
    for (size_t i = 0; i < N; ++i) v[i] = w[i] / bn;
  }
  {
    hpcg_status s = hpcg_apply_status(h);   // every apply above waited within its bound
    if (s != HPCG_OK) return s;
  }
  beta.resize(alpha.size() > 0 ? alpha.size() - 1 : 0);
  if (h_lmin) *h_lmin = tridiag_eig(alpha, beta, 0);
  if (h_lmax) *h_lmax = tridiag_eig(alpha, beta, (int)alpha.size() - 1);
  return HPCG_OK;
}

hpcg_status hpcg_last_solve_status(hpcg_handle h, int32_t* h_status) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (!h_status) return fail(h, HPCG_ERR_INVALID_ARG, "h_status is NULL");
  for (int i = 0; i < h->G.B; ++i) h_status[i] = h->last_status[i];
  return HPCG_OK;
}

hpcg_status hpcg_set_option(hpcg_handle h, int32_t option, int32_t value) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  switch (option) {
    case HPCG_OPT_ENGINE:
      if (value < HPCG_ENGINE_AUTO || value > HPCG_ENGINE_PERSISTENT) return fail(h, HPCG_ERR_INVALID_ARG, "bad engine");
      h->engine_opt = value;
      return HPCG_OK;
    case HPCG_OPT_GRAPH_UNROLL:
      if (value < 1 || value > 64) return fail(h, HPCG_ERR_INVALID_ARG, "graph unroll must lie in [1, 64]");
      h->unroll = value;
      return HPCG_OK;
    case HPCG_OPT_PRECISION:
      if (value != HPCG_PREC_VEC64 && value != HPCG_PREC_VEC32) return fail(h, HPCG_ERR_INVALID_ARG, "bad precision");
      h->prec = value;
      return HPCG_OK;
    case HPCG_OPT_POLL_LIMIT:
      if (value < 0 || value > (1 << 30)) return fail(h, HPCG_ERR_INVALID_ARG, "poll limit must be 0 .. 2^30");
      h->B.poll_limit = value == 0 ? kPollLimitDefault : (unsigned)value;
      return HPCG_OK;
    case HPCG_OPT_APPLY_POLL_LIMIT:
      if (value < 0 || value > (1 << 30)) return fail(h, HPCG_ERR_INVALID_ARG, "apply poll limit must be 0 .. 2^30");
      h->B.apply_poll_limit = value == 0 ? kApplyPollDefault : (unsigned)value;
      return HPCG_OK;
    case HPCG_OPT_FALLBACK:
      if (value != 0 && value != 1) return fail(h, HPCG_ERR_INVALID_ARG, "fallback must be 0 or 1");
      h->fallback = value;
      return HPCG_OK;
    case HPCG_OPT_FORM:
      if (value < HPCG_FORM_DIRECT || value > HPCG_FORM_JACOBI) return fail(h, HPCG_ERR_INVALID_ARG, "bad form");
      h->B.form = value;
      return HPCG_OK;
    case HPCG_OPT_APPLY_PATH:
      if (value < HPCG_APPLY_AUTO || value > HPCG_APPLY_BRIDGE) return fail(h, HPCG_ERR_INVALID_ARG, "bad apply path");
      h->apply_path = value;
      return HPCG_OK;
    case HPCG_OPT_BLOCK_SPLIT:
      if (value < 0 || value > 2) return fail(h, HPCG_ERR_INVALID_ARG, "block split must be 0 (automatic), 1 or 2");
      h->block_split = value;
      return HPCG_OK;
    case HPCG_OPT_LEAF_SPLIT: {
      if (value != 0 && value != 1 && value != 2 && value != 4 && value != 8)
        return fail(h, HPCG_ERR_INVALID_ARG, "leaf split must be 0 (automatic), 1, 2, 4 or 8");
      Geom G;
      std::string why;
      if (!make_geom(&h->part, G, why, value)) return fail(h, HPCG_ERR_SHAPE, why);
      h->G = G;
      h->split = value;
      h->Gapply = apply_geom(&h->part, G, value);
      return HPCG_OK;
    }
    default:
      return fail(h, HPCG_ERR_INVALID_ARG, "unknown option");
  }
}

int32_t hpcg_last_engine(hpcg_handle h) { return h ? h->last_engine : 0; }

int32_t hpcg_last_apply_path(hpcg_handle h) { return h ? h->last_apply_path : 0; }

int32_t hpcg_last_fallback(hpcg_handle h) { return h ? h->last_fallback : 0; }

hpcg_status hpcg_last_launch_info(hpcg_handle h, int32_t* grid, int32_t* lds_bytes) {
  if (!h) return fail(nullptr, HPCG_ERR_INVALID_ARG, "handle is NULL");
  if (grid) *grid = h->last_grid;
  if (lds_bytes) *lds_bytes = h->last_lds;
  return HPCG_OK;
}

const char* hpcg_status_string(hpcg_status s) {
  switch (s) {
    case HPCG_OK: return "ok";
    case HPCG_ERR_INVALID_ARG: return "invalid argument";
    case HPCG_ERR_SHAPE: return "unsupported shape";
    case HPCG_ERR_HIP: return "HIP runtime error";
    case HPCG_ERR_BREAKDOWN: return "PCG breakdown";
    case HPCG_ERR_NOT_CONVERGED: return "not converged";
    case HPCG_ERR_WORKSPACE: return "workspace error";
    case HPCG_ERR_STATE: return "call order error";
  }
  return "unknown status";
}

const char* hpcg_last_error(hpcg_handle h) {
  if (!h) return g_create_error.c_str();
  return h->err.c_str();
}

void hpcg_destroy(hpcg_handle h) {
  if (!h) return;
  destroy_graph(h);
  if (h->bs_gexec) (void)hipGraphExecDestroy(h->bs_gexec);
  if (h->bs_graph) (void)hipGraphDestroy(h->bs_graph);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  if (h->h_flag) (void)hipHostFree(h->h_flag);
  if (h->h_st) (void)hipHostFree(h->h_st);
  if (h->h_ctl) (void)hipHostFree(h->h_ctl);
  delete h;
}

}  // extern "C"
