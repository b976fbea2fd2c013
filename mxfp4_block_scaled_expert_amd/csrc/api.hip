// C ABI of libmxq (declared and documented in include/mxq.h): host-side
// argument validation, workspace carving, per-class grid bounds, and the kernel
// sequences of each entry point.
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/mxq.h"
#include "kernels.hpp"

using namespace mxq;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

mxq_status check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXQ_ERR_ARCH;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXQ_ERR_ARCH;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MXQ_OK : MXQ_ERR_ARCH;
}

mxq_status launch_status() { return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_LAUNCH; }

// Scratch of mxq_block_fp8_linear_noalloc: the bf16 input's quantised codes and scales.  Every
// GPU the library runs on holds one copy until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device memory: the device address of each GPU's copy comes
// from hipGetSymbolAddress, taken once per device (mxq_init, else the entry point's first call
// on that device) and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MXQ_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mxq_status scratch_ptr_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXQ_ERR_ARCH;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXQ_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MXQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MXQ_TRY(expr)                \
  do {                               \
    const mxq_status _s = (expr);    \
    if (_s != MXQ_OK) return _s;     \
  } while (0)

constexpr size_t kSkinnyMaxLds = 64 * 1024;
// Expert-streaming path: routing tables and two activation buffers per workgroup in LDS, at
// most kStreamMaxLds so that two or more workgroups share a compute unit.
constexpr int64_t kStreamMaxRows = 4096;
constexpr int32_t kStreamMaxExperts = 512;
constexpr size_t kStreamMaxLds = 80 * 1024;
#ifndef MXQ_DENSE_BIG_SHAPE
#define MXQ_DENSE_BIG_SHAPE (-1)
#endif
// tile shape of the large dense W8A8 GEMM: -1 picks it from the grid (dense_big_shape)
constexpr int kDenseBigShape = MXQ_DENSE_BIG_SHAPE;

#ifndef MXQ_DENSE_RING
#define MXQ_DENSE_RING 1
#endif
constexpr bool kDenseRing = MXQ_DENSE_RING != 0;

constexpr int kMoeBlockM = 128;
#ifndef MXQ_SELF_ROUTE
#define MXQ_SELF_ROUTE 1
#endif
constexpr bool kSelfRoute = MXQ_SELF_ROUTE != 0;
// routing ids held in each tile's LDS; past 2048 routed rows every workgroup's lookup (a pass
// over all ids) costs more than the sort it saves (4096 rows over 128 experts: 323 us sorted,
// 341 us self-routed; 2048 rows: 182 -> 156 us, MXFP4 523 -> 345 us)
constexpr int64_t kSelfRouteMaxRows = 2048;
constexpr int32_t kSelfRouteMaxExperts = 512;  // one expert per thread of the ring-fed tile
// Self-routed tiles cut each expert's rows into blocks of 64 (interleaved A/B against 128 and
// 32: W8A16 E = 8 with blocks of 4, 5, 33, 12, 1, 73 rows 30.6 against 34.6 / 36.7 us; 256
// tokens top-2 over 8 experts 40.7 against 48.4 / 56.1 us; 256 tokens top-4 over 64 experts
// 124 against 131 / 133 us; MXFP4 256 tokens top-4 over 32 experts 223 against 224 / 281 us):
// an expert's rows run on twice the workgroups of 128-row blocks, each with shorter K steps.
// A stage whose grid still fits the GPU with smaller blocks takes them instead of a K split
// (self_fill_block_m).
constexpr int32_t kSelfRouteBlockM = 64;
static_assert(kSelfRouteBlockM <= 128, "the self-routed tile keeps a block's row ids in 128 LDS slots");
constexpr int kNumClasses = 5;  // tiny-block kernel, 16-, 32-, 64-, 128-row MFMA tiles
constexpr int kClassTile[kNumClasses] = {-1, 3, 2, 1, 0};  // launcher tile index per class
constexpr int kClassRows[kNumClasses] = {16, 16, 32, 64, 128};  // [0] is set at run time

// The dispatch a call runs with: the caller's mxq_moe_dispatch, or the defaults for NULL.
mxq_status read_dispatch(const mxq_moe_dispatch* d, mxq_moe_dispatch& out) {
  out = mxq_moe_dispatch{MXQ_DISPATCH_PER_BLOCK, 0, MXQ_TINY_ROWS_AUTO, MXQ_TINY_MFMA, MXQ_K_SPLIT_AUTO, MXQ_SORT_AUTO,
                         MXQ_FUSE_AUTO};
  if (!d) return MXQ_OK;
  if (d->mode < MXQ_DISPATCH_PER_BLOCK || d->mode > MXQ_DISPATCH_LAYER_AVERAGE) return MXQ_ERR_ARG;
  if (d->tiny_kernel != MXQ_TINY_MFMA && d->tiny_kernel != MXQ_TINY_GEMV) return MXQ_ERR_ARG;
  if (d->forced_class < 0 || d->forced_class >= kNumClasses) return MXQ_ERR_ARG;
  if (d->tiny_max_rows < MXQ_TINY_ROWS_AUTO || d->tiny_max_rows > 16) return MXQ_ERR_ARG;
  if (d->k_split != MXQ_K_SPLIT_AUTO && d->k_split != 1 && d->k_split != 2 && d->k_split != 4 && d->k_split != 8)
    return MXQ_ERR_ARG;
  if (d->sort != MXQ_SORT_AUTO && d->sort != MXQ_SORT_ALWAYS) return MXQ_ERR_ARG;
  if (d->fuse != MXQ_FUSE_AUTO && d->fuse != MXQ_FUSE_NONE) return MXQ_ERR_ARG;
  out = *d;
  return MXQ_OK;
}

// Operands the 128 x 256 direct-to-LDS tile addresses with 32-bit byte offsets: the
// activation rows of both stages (x / ic1 rows) and one expert's weights.
bool big_tile_offsets_fit(int64_t M, int64_t R, int64_t H, int64_t I) {
  constexpr int64_t k4G = int64_t(1) << 32;
  return M * H < k4G && R * I < k4G && 2 * I * H < k4G;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The column-width half of the tile choice: the 256-wide direct-to-LDS W8A8 tile takes the
// column tiles of width 256; a last column tile of n_size <= 128 (where the wide tile would
// leave at least half of its products unused) takes the 128-wide tile instead.  Returns the
// columns the wide tile covers.
constexpr int64_t kWideTileN = 256;
int64_t wide_tile_columns(int64_t N) {
  const int64_t tail = N % kWideTileN;
  return (tail != 0 && tail <= kWideTileN / 2) ? N - tail : N;
}

// Tile shape of the dense direct-to-LDS W8A8 GEMM from the grid it gives: each tile runs its K
// range as one serial chain, so until the 256 compute units are full, more and smaller tiles
// finish sooner -- the 128 x 128 three-stage tile when its tiles fit one round, else the
// 128 x 256 three-stage tile when its tiles do, else the 256 x 256 two-stage tile (interleaved
// on the box, K = 7168: M = 2048, N = 2048 92 -> 48 us; M = 4096, N = 2048 93 -> 68 us; M = 512,
// N = 7168, K = 2048 31 -> 19 us; 2048 x 7168 x 2048 stays on the 256 x 256 tile, 34 us against
// 41 on 128 x 256).  Shapes as launch_gemm_w8a8_big numbers them.
int dense_big_shape(int64_t M, int64_t N) {
  if (kDenseBigShape >= 0) return kDenseBigShape;
  if (cdiv(M, int64_t(128)) * cdiv(N, int64_t(128)) <= 256) return 3;
  if (cdiv(M, int64_t(128)) * cdiv(N, int64_t(256)) <= 256) return 1;
  return 0;
}

// Columns [n0, N) of a GEMM as a problem of their own: weights, weight-scale grid rows, bias
// and output shifted by n0 columns (n0 a multiple of 256: of every weight-scale block width
// and of the tiled layout's 16-row groups).
GemmArgs column_slice(const GemmArgs& g, int64_t n0, bool out_f32) {
  GemmArgs t = g;
  t.W = g.W + (g.w_tiled ? (n0 / 16) * tiled_steps(g.ldw) * 2048 : n0 * g.ldw);
  t.ws = static_cast<const float*>(g.ws) + (n0 / (g.block_n > 0 ? g.block_n : 128)) * g.ws_s0;
  if (g.bias) t.bias = static_cast<const uint8_t*>(g.bias) + n0 * (g.bias_bf16 ? 2 : 4);
  t.out = static_cast<uint8_t*>(g.out) + n0 * (out_f32 ? 4 : 2);
  t.N = g.N - n0;
  return t;
}

// K split of the routed stages with bf16 activations.  A stage with few expert blocks runs too
// few workgroups to stream its weights at HBM speed (each holds a bounded number of loads in
// flight), so each tile's K range is cut into chunks that run as separate workgroups; they
// write fp32 partial sums to slices of the workspace, summed in slice order by the kernel after
// the stage (the SiLU-and-mul after stage 1, the combine after stage 2).  Chunks are whole
// multiples of 256 columns of K.  The workspace holds split_cap(R) slices per stage.
constexpr int64_t kSplitMaxRows = 1024;    // more routed rows: no split (workspace bound)
constexpr int64_t kSplitRowSlices = 2048;  // slices x routed rows the workspace holds at most
constexpr int kSplitMax = 8;
// Automatic choice, from measurements of the ring-fed tiles (W8A16 E = 8 with the 128-token
// small-block routing, 256 tokens top-2, MXFP4 40 tokens top-4): a split pays only while the
// stage's tiles stay at most one per compute unit and the partial sums are small (at most
// 256 routed rows); beyond that the partial-sum traffic and the extra tile prologues cost more
// than the shorter K loops save.
constexpr int64_t kSplitAutoMaxRows = 256;
constexpr int64_t kSplitTargetTiles = 256;

int split_cap(int64_t R) {
  if (R > kSplitMaxRows) return 1;
  int s = 1;
  while (s < kSplitMax && int64_t(2 * s) * R <= kSplitRowSlices) s *= 2;
  return s;
}

struct KSplit {
  int n;          // chunks (1: no split)
  int64_t chunk;  // K elements per chunk
};

// `requested`: MXQ_K_SPLIT_AUTO, or the caller's upper bound (1 = off).  Automatic: with at
// most kSplitAutoMaxRows routed rows, the most chunks that keep an estimate of the stage's
// tiles (at most min(E, R) blocks of 128-column tiles) within kSplitTargetTiles.
KSplit pick_split(int64_t R, int32_t E, int64_t N, int64_t K, int requested) {
  const int cap = split_cap(R);
  int s = 1;
  if (requested > 1) {
    s = std::min(requested, cap);
  } else if (requested == MXQ_K_SPLIT_AUTO) {
    const int64_t tiles = std::min<int64_t>(E, R) * cdiv(N, int64_t(128));
    if (R <= kSplitAutoMaxRows)
      while (s < cap && tiles * s * 2 <= kSplitTargetTiles) s *= 2;
  }
  if (s <= 1) return {1, 0};
  const int64_t chunk = cdiv(cdiv(K, int64_t(s)), int64_t(256)) * 256;
  const int n = int(cdiv(K, chunk));
  return n > 1 ? KSplit{n, chunk} : KSplit{1, 0};
}

struct MoeWorkspace {
  int32_t *sorted_ids, *expert_ids, *offsets, *num_blocks, *class_lists, *class_counts;
  float* partial;  // K-split partial slices (bf16 activations, R <= kSplitMaxRows)
  int32_t* align_scratch;  // per-chunk counts of the multi-workgroup sort (many routed rows)
  uint8_t* qx;
  float* sx;
  uint16_t* ic0;
  uint16_t* ic1;
  uint8_t* ic1_q;
  float* ic1_s;
  float* y;
  size_t bytes;
};

MoeWorkspace carve_moe(void* base, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, bool act_quant) {
  const int64_t R = M * topk;
  const int64_t mbk = mxq_moe_max_blocks(M, topk, E, kMoeBlockM);
  MoeWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    uint8_t* p = base ? static_cast<uint8_t*>(base) + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.sorted_ids = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * mbk * kMoeBlockM));
  w.expert_ids = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * mbk));
  w.offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (mbk + 1)));
  w.num_blocks = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  w.class_lists = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 4 * mbk * kNumClasses));
  w.class_counts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * kNumClasses));
  if (act_quant) {
    w.qx = take(size_t(M) * H);
    w.sx = reinterpret_cast<float*>(take(sizeof(float) * M * (H / 128)));
  }
  w.ic0 = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * R * 2 * I));
  if (act_quant) {
    w.ic1_q = take(size_t(R) * I);
    w.ic1_s = reinterpret_cast<float*>(take(sizeof(float) * R * (I / 128)));
  } else {
    w.ic1 = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * R * I));
  }
  w.y = reinterpret_cast<float*>(take(sizeof(float) * R * H));
  if (!act_quant && split_cap(R) > 1)
    w.partial = reinterpret_cast<float*>(take(sizeof(float) * split_cap(R) * R * std::max(2 * I, H)));
  if (align_multi_scratch_ints(R, E) > 0)
    w.align_scratch = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * align_multi_scratch_ints(R, E)));
  w.bytes = off;
  return w;
}

// Largest number of blocks that can fall in class c (no host sync: from sizes only).
int64_t class_bound(int c, int64_t R, int32_t E, int64_t max_blocks, const ClassPolicy& pol) {
  if (pol.forced >= 0) return c == pol.forced ? max_blocks : 0;
  if (c >= pol.n_live) return 0;
  const int lo = c == 0 ? 0 : pol.bound[c - 1];
  const bool top = c == pol.n_live - 1;  // also takes every block past the launched bounds
  const int hi = top ? kMoeBlockM : pol.bound[c];
  if (hi <= lo) return 0;
  int64_t ub = std::min<int64_t>(max_blocks, R / (lo + 1));
  if (hi < kMoeBlockM) ub = std::min<int64_t>(ub, E);  // only an expert's last block is partial
  return std::max<int64_t>(ub, 0);
}

// Self-routed stages: the smallest block size (16, 32 or 64 rows) whose largest possible grid
// (blocks x column tiles) fits the GPU's compute units -- the stage's rows alone then fill the
// GPU and it runs without a K split; 0 when no size fits (64-row blocks and the K-split rule).
// Interleaved A/B: W8A16 E = 8 with blocks of 4, 5, 33, 12, 1, 73 rows 30.6 -> 26.2 us (16-row
// blocks, no split, the SiLU-and-mul in the stage-1 epilogue), 64 tokens top-2 over 8 experts
// 29.2 -> 26.3 us; larger routings keep 64-row blocks (no change).
int32_t self_fill_block_m(int64_t M, int32_t topk, int32_t E, int64_t n_tiles) {
  for (int32_t bm : {16, 32, 64})
    if (mxq_moe_max_blocks(M, topk, E, bm) * n_tiles <= kSplitTargetTiles) return bm;
  return 0;
}

// Per-block tile-class policy (page [A], implementation items 1-2: each block's kernel from its
// own row count).  The bounds come from the class sweep (`bench.py --only classes`: E experts
// each holding exactly m rows, every class forced in turn, on the GPT-OSS MXFP4, DeepSeek W8A8
// and small W8A16 expert shapes):
//  * the tiny-block kernel is the fastest class up to 4 rows per block with e4m3 activations,
//    8 with bf16 activations and e4m3 weights, 4 with e2m1 weights (it streams an expert's
//    weights once per pass of 4-8 rows, the tiles pay a fixed cost per block); then the 16-,
//    32-, 64- and 128-row tiles each win in their own range;
//  * with bf16 activations on the ring-fed tiles, when the routing averages more rows per
//    expert than the tiny bound the tile classes are launched anyway: the tiny blocks then
//    take 16-row tiles in that launch, beside the taller blocks, instead of a launch of their
//    own after it (W8A16 E = 8 with blocks of 4, 5, 33, 12, 1 and 73 rows: 40 against 54 us;
//    256 tokens top-2: 54 against 58 us; MXFP4 40 tokens top-4: 73 against 77 us);
//  * the tiny class takes every block when M <= 32 or R <= 2 E: an expert holds at most M rows,
//    and with at most two routed rows per expert on average (decode batches) an odd taller
//    block's extra passes run beside the many tiny blocks, while a tile-class launch would run
//    mostly empty workgroups;
//  * with the 128 x 256 direct-to-LDS W8A8 tile and R > 4096 routed rows every class folds
//    into the 128-row one: with many blocks one launch of that tile keeps the GPU full, where
//    separate class launches each leave it partly idle (DeepSeek prefill, 4096 tokens: 4-5 %
//    faster than separate classes; equal at 512 tokens, and slower than the 32- and 64-row
//    tiles with 32 experts of 8-64 rows).
// M also caps the classes launched: those whose lower bound reaches M get no blocks when every
// token names distinct experts (a block beyond that, from repeated ids, lands in the largest
// launched class).
int tiny_rows_auto(int wfmt, bool act_quant) { return act_quant ? 4 : (wfmt == W_E2M1_MX ? 4 : 8); }

ClassPolicy make_policy(int64_t M, int64_t R, int32_t E, bool big_tile, bool ring, int wfmt, bool act_quant,
                        const mxq_moe_dispatch& dc) {
  const int tiny = dc.tiny_max_rows < 0 ? tiny_rows_auto(wfmt, act_quant) : dc.tiny_max_rows;
  ClassPolicy pol{};
  pol.n_classes = kNumClasses;
  pol.forced = -1;
  pol.bound[0] = tiny;
  for (int c = 1; c < kNumClasses; ++c) pol.bound[c] = std::max(tiny, kClassRows[c]);
  if (tiny > 0 && (M <= 32 || R <= 2 * int64_t(E))) {
    pol.bound[0] = int(std::max<int64_t>(tiny, M));
  } else if (ring && dc.tiny_max_rows < 0 && R > int64_t(tiny) * E) {
    // bf16 activations on the ring-fed tiles: unless the routing averages at most the tiny
    // bound per expert, the tile classes are launched anyway and the tiny blocks take 16-row
    // tiles in the same launch (running beside the taller blocks instead of in a launch of
    // their own)
    pol.bound[0] = 0;
  } else if (big_tile && R > 4096) {
    if (dc.tiny_kernel == MXQ_TINY_MFMA) pol.bound[0] = 0;
    for (int c = 1; c < kNumClasses - 1; ++c) pol.bound[c] = pol.bound[0];
  }
  pol.n_live = kNumClasses;
  for (int c = 1; c < kNumClasses; ++c)
    if (pol.bound[c - 1] >= M) {
      pol.n_live = c;
      break;
    }
  if (dc.mode == MXQ_DISPATCH_FORCED) {
    pol.forced = dc.forced_class;
    pol.n_live = kNumClasses;
  } else if (dc.mode == MXQ_DISPATCH_LAYER_AVERAGE) {
    // the per-layer rule maps the average onto the plain class bounds (no folding)
    const int64_t avg = std::max<int64_t>(1, R / std::max<int32_t>(E, 1));
    int c = kNumClasses - 1;
    for (int i = 0; i < kNumClasses - 1; ++i)
      if (avg <= (i == 0 ? tiny : kClassRows[i])) { c = i; break; }
    pol.forced = c;
    pol.n_live = kNumClasses;
  }
  return pol;
}

// The two stage GEMMs of a fused-MoE call over the carved workspace w (stage 1: ic0 = x @ w1^T
// + b1 by compact row; stage 2: y = ic1 @ w2^T, rows scattered back to flat ids).
void moe_stage_args(GemmArgs& g1, GemmArgs& g2, const MoeWorkspace& w, const void* x, const void* w1,
                    const void* w1s, const void* w2, const void* w2s, const float* b1, int64_t M, int64_t H,
                    int64_t I, int32_t topk, int wfmt, bool act_quant, bool tiled) {
  const int64_t R = M * topk;
  const bool mx = wfmt == W_E2M1_MX;
  BlockRouting rt{w.sorted_ids, w.expert_ids, w.offsets, nullptr, nullptr, kMoeBlockM, topk};

  // stage 1: ic0 = x @ w1^T (+ b1), compact rows
  g1 = GemmArgs{};
  g1.A = act_quant ? static_cast<const void*>(w.qx) : x;
  g1.lda = H;
  g1.sa = w.sx;
  g1.lds = H / 128;
  g1.W = static_cast<const uint8_t*>(w1);
  g1.ldw = mx ? H / 2 : H;
  g1.w_tiled = tiled;
  g1.w_estride = tiled ? 2 * I * tiled_steps(g1.ldw) * 128 : g1.ldw * 2 * I;
  g1.ws = w1s;
  if (mx) {
    g1.ws_s0 = H / 32;
    g1.ws_estride = tiled ? 2 * I * tiled_scale_steps(H / 32) * 8 : 2 * I * (H / 32);
  } else {
    g1.ws_s0 = H / 128;
    g1.ws_s1 = 1;
    g1.ws_estride = cdiv(2 * I, 128) * (H / 128);
  }
  g1.block_n = 128;
  g1.bias = b1;
  g1.bias_bf16 = 0;
  g1.bias_estride = 2 * I;
  g1.out = w.ic0;
  g1.ldo = 2 * I;
  g1.M = R;
  g1.N = 2 * I;
  g1.K = H;
  g1.rt = rt;

  // stage 2: y = ic1 @ w2^T, rows scattered back to flat ids
  g2 = GemmArgs{};
  g2.A = act_quant ? static_cast<const void*>(w.ic1_q) : static_cast<const void*>(w.ic1);
  g2.lda = I;
  g2.sa = w.ic1_s;
  g2.lds = I / 128;
  g2.W = static_cast<const uint8_t*>(w2);
  g2.ldw = mx ? I / 2 : I;
  g2.w_tiled = tiled;
  g2.w_estride = tiled ? H * tiled_steps(g2.ldw) * 128 : g2.ldw * H;
  g2.ws = w2s;
  if (mx) {
    g2.ws_s0 = I / 32;
    g2.ws_estride = tiled ? H * tiled_scale_steps(I / 32) * 8 : H * (I / 32);
  } else {
    g2.ws_s0 = I / 128;
    g2.ws_s1 = 1;
    g2.ws_estride = cdiv(H, 128) * (I / 128);
  }
  g2.block_n = 128;
  g2.out = w.y;
  g2.ldo = H;
  g2.M = R;
  g2.N = H;
  g2.K = I;
  g2.rt = rt;

}

// Every host-side decision of a fused-MoE call, from sizes, the dispatch and the stage
// arguments' layout and alignment (no device state is read).
struct MoePlan {
  bool big_tile;            // W8A8: the 128 x 256 direct-to-LDS tile takes the 65..128-row blocks
  bool ring_shape, ring;    // bf16 activations: the ring-fed tiles (shape only / and alignment)
  ClassPolicy pol;
  bool expert_stream;       // every block tiny: the two expert-streaming kernels, no sort
  bool self_routable, self_route;  // small routing the tiles can route themselves (and do)
  int32_t bm1, bm2;         // self-routed block rows per stage
  int64_t mbk1, mbk2;       // their largest block counts
  bool fill1, fill2;        // a stage whose self-routed grid fits the GPU (no K split)
  KSplit sp1, sp2;
  bool fuse_silu;           // SiLU-and-mul in the tiny kernel's stage-2 row staging
  bool pair_silu;           // SiLU-and-mul in the stage-1 epilogue of the ring-fed tiles
  bool fold_top1;           // top-1 combine in the self-routed stage-2 epilogue
};

MoePlan plan_moe(const GemmArgs& g1, const GemmArgs& g2, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                 int wfmt, bool act_quant, bool tiled, const mxq_moe_dispatch& dc) {
  MoePlan p{};
  const int64_t R = M * topk;
  const int64_t mbk = mxq_moe_max_blocks(M, topk, E, kMoeBlockM);
  const int wfmt_w16 = wfmt == W_E2M1_MX ? W_E2M1_MX : W_E4M3_BLOCK;
  // the 128 x 256 W8A8 tile: K <= 16384 on both stages and operand offsets below 4 GiB
  p.big_tile = act_quant && H <= 16384 && I <= 16384 && big_tile_offsets_fit(M, R, H, I);
  // bf16 activations: both stages take the ring-fed tiles (the class policy looks only at the
  // layout-independent part, so that plain and tiled weights run the same classes)
  p.ring_shape = !act_quant && w16_ring_shape_ok(g1, wfmt_w16) && w16_ring_shape_ok(g2, wfmt_w16);
  p.ring = p.ring_shape && w16_ring_supported(g1, wfmt_w16) && w16_ring_supported(g2, wfmt_w16);
  p.pol = make_policy(M, R, E, p.big_tile, p.ring_shape, wfmt, act_quant, dc);
  const int tiny = dc.tiny_kernel;
  // Every block of the routing is tiny and the activations stay bf16: the expert-streaming
  // kernels group the routed rows by expert themselves (no sort, no block tables), stage 1 ends
  // in the SiLU-and-mul, and rows are indexed by flat routed id up to the combine.
  // (Such a routing runs without a K split whatever the sort and fuse knobs say, so that the
  // sorted path they select computes the same sums.)
  const bool streamable = !act_quant && p.pol.forced < 0 && p.pol.n_live == 1 && tiny == MXQ_TINY_MFMA &&
                          R <= kStreamMaxRows && E <= kStreamMaxExperts && I % 16 == 0 &&
                          expert_stream_lds_bytes(wfmt_w16, 1, 2 * I, H, E, R) <= kStreamMaxLds &&
                          expert_stream_lds_bytes(wfmt_w16, 2, H, I, E, R) <= kStreamMaxLds;
  p.expert_stream = streamable && dc.sort == MXQ_SORT_AUTO && dc.fuse == MXQ_FUSE_AUTO;
  if (p.expert_stream) return p;
  // Small bf16 routings on the ring-fed tiles with no tiny-class launch: every workgroup finds
  // its block from the routing ids itself (the expert-ordered blocks the sort would lay out,
  // cut at 16, 32 or 64 rows, each with the class the policy picks for its row count) and no
  // sort kernel runs; every row's products are those of the sorted path, so the outputs are the
  // same bits.  A stage whose self-routed rows alone fill the GPU runs without a K split.  The
  // split follows from the routing's size whether or not the sort runs (MXQ_SORT_ALWAYS), so the
  // two paths compute the same sums.
  p.self_routable = kSelfRoute && p.ring && R <= kSelfRouteMaxRows && E <= kSelfRouteMaxExperts &&
                    class_bound(0, R, E, mbk, p.pol) == 0;
  p.self_route = p.self_routable && dc.sort == MXQ_SORT_AUTO;
  const int32_t f1 = p.self_routable ? self_fill_block_m(M, topk, E, cdiv(2 * I, int64_t(128))) : 0;
  const int32_t f2 = p.self_routable ? self_fill_block_m(M, topk, E, cdiv(H, int64_t(128))) : 0;
  p.fill1 = f1 > 0;
  p.fill2 = f2 > 0;
  p.bm1 = p.fill1 ? f1 : kSelfRouteBlockM;
  p.bm2 = p.fill2 ? f2 : kSelfRouteBlockM;
  p.mbk1 = mxq_moe_max_blocks(M, topk, E, p.bm1);
  p.mbk2 = mxq_moe_max_blocks(M, topk, E, p.bm2);
  // K split (bf16 activations; not with the GEMV tiny kernel): partial slices in the workspace
  const bool gemv_runs = tiny == MXQ_TINY_GEMV && !tiled;  // the GEMV kernel writes whole sums only
  const bool can_split = !act_quant && !gemv_runs && split_cap(R) > 1;
  const bool auto_split = dc.k_split == MXQ_K_SPLIT_AUTO;
  p.sp1 = can_split && !(auto_split && (p.fill1 || streamable)) ? pick_split(R, E, 2 * I, H, dc.k_split)
                                                                 : KSplit{1, 0};
  p.sp2 = can_split && !(auto_split && (p.fill2 || streamable)) ? pick_split(R, E, H, I, dc.k_split)
                                                                 : KSplit{1, 0};
  // With bf16 activations and only the tiny-block class launched, stage 2 computes the
  // SiLU-and-mul while staging its rows (no ic1 round trip, one launch fewer).
  p.fuse_silu = !act_quant && dc.fuse == MXQ_FUSE_AUTO && p.pol.forced < 0 && p.pol.n_live == 1 &&
                tiny == MXQ_TINY_MFMA && p.sp1.n == 1 && skinny_lds_bytes(wfmt_w16, false, I) <= kSkinnyMaxLds;
  // With bf16 activations, stage 1 wholly on the ring-fed tiles (no tiny-class launch) and
  // whole K ranges, each stage-1 tile pairs 64 gate with the matching 64 up columns and ends in
  // the SiLU-and-mul: ic1 comes straight out of stage 1, one launch fewer.
  p.pair_silu = !act_quant && dc.fuse == MXQ_FUSE_AUTO && p.ring && p.sp1.n == 1 && I % 64 == 0 &&
                class_bound(0, R, E, mbk, p.pol) == 0;
  // Self-routed stage 2 with top-1 routing and whole K ranges: the combine (one weighted row per
  // token) folds into the stage-2 epilogue, which writes out directly.
  p.fold_top1 = p.self_route && topk == 1 && p.sp2.n == 1 && dc.fuse == MXQ_FUSE_AUTO;
  return p;
}

mxq_status run_moe(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, const int32_t* ids,
                   const float* wts, const void* w1, const void* w1s, const void* w2, const void* w2s,
                   const float* b1, int wfmt, bool act_quant, bool tiled, const mxq_moe_dispatch& dc, void* out,
                   void* ws, size_t ws_bytes, hipStream_t st) {
  const int64_t R = M * topk;
  if (R == 0) return MXQ_OK;
  const int64_t mbk = mxq_moe_max_blocks(M, topk, E, kMoeBlockM);
  MoeWorkspace w = carve_moe(ws, M, H, I, E, topk, act_quant);
  if (!ws || ws_bytes < w.bytes) return MXQ_ERR_WORKSPACE;
  const bool mx = wfmt == W_E2M1_MX;
  const int wfmt_w16 = mx ? W_E2M1_MX : W_E4M3_BLOCK;
  GemmArgs g1, g2;
  moe_stage_args(g1, g2, w, x, w1, w1s, w2, w2s, b1, M, H, I, topk, wfmt, act_quant, tiled);
  const MoePlan plan = plan_moe(g1, g2, M, H, I, E, topk, wfmt, act_quant, tiled, dc);
  const bool big_tile = plan.big_tile, ring = plan.ring;
  const ClassPolicy pol = plan.pol;
  const int tiny = dc.tiny_kernel;

  if (plan.expert_stream) {
    const EsRoute er{ids, int32_t(R), E, topk};
    GemmArgs s1{};
    s1.A = x;
    s1.lda = H;
    s1.W = static_cast<const uint8_t*>(w1);
    s1.ldw = mx ? H / 2 : H;
    s1.w_tiled = tiled;
    s1.w_estride = tiled ? 2 * I * tiled_steps(s1.ldw) * 128 : s1.ldw * 2 * I;
    s1.ws = w1s;
    s1.ws_s0 = mx ? H / 32 : H / 128;
    s1.ws_s1 = 1;
    s1.ws_estride = mx ? (tiled ? 2 * I * tiled_scale_steps(H / 32) * 8 : 2 * I * (H / 32)) : cdiv(2 * I, 128) * (H / 128);
    s1.bias = b1;
    s1.bias_estride = 2 * I;
    s1.out = w.ic1;
    s1.ldo = I;
    s1.M = R;
    s1.N = 2 * I;
    s1.K = H;
    GemmArgs s2{};
    s2.A = w.ic1;
    s2.lda = I;
    s2.W = static_cast<const uint8_t*>(w2);
    s2.ldw = mx ? I / 2 : I;
    s2.w_tiled = tiled;
    s2.w_estride = tiled ? H * tiled_steps(s2.ldw) * 128 : s2.ldw * H;
    s2.ws = w2s;
    s2.ws_s0 = mx ? I / 32 : I / 128;
    s2.ws_s1 = 1;
    s2.ws_estride = mx ? (tiled ? H * tiled_scale_steps(I / 32) * 8 : H * (I / 32)) : cdiv(H, 128) * (I / 128);
    s2.out = w.y;
    s2.ldo = H;
    s2.M = R;
    s2.N = H;
    s2.K = I;
    launch_expert_stream(s1, wfmt_w16, 1, er, st);
    launch_expert_stream(s2, wfmt_w16, 2, er, st);
    launch_combine(w.y, 1, 0, wts, ids, E, M, topk, H, static_cast<uint16_t*>(out), st);
    return launch_status();
  }

  const bool self_route = plan.self_route;
  const int64_t self_mbk1 = plan.mbk1, self_mbk2 = plan.mbk2;
  if (self_route) {
    for (GemmArgs* g : {&g1, &g2}) {
      g->rt.block_m = g == &g1 ? plan.bm1 : plan.bm2;
      g->rt.route_ids = ids;
      g->rt.route_R = int32_t(R);
      g->rt.route_E = E;
      g->rt.route_pol = pol;
    }
  } else {
    launch_moe_align(ids, M, topk, E, kMoeBlockM, w.sorted_ids, w.expert_ids, w.offsets, w.num_blocks, mbk, pol,
                     w.class_lists, mbk, w.class_counts, false, w.align_scratch, st);
  }
  if (act_quant) launch_quant_1x128(static_cast<const uint16_t*>(x), M, H, H, w.qx, H, w.sx, st);

  // K split: partial slices in the workspace
  const KSplit sp1 = plan.sp1, sp2 = plan.sp2;
  if (sp1.n > 1) {
    g1.k_split = sp1.n;
    g1.k_chunk = sp1.chunk;
    g1.split_stride = R * 2 * I;
    g1.out = w.partial;
  }
  if (sp2.n > 1) {
    g2.k_split = sp2.n;
    g2.k_chunk = sp2.chunk;
    g2.split_stride = R * H;
    g2.out = w.partial;
  }

  const bool fuse_silu = plan.fuse_silu, pair_silu = plan.pair_silu, fold_top1 = plan.fold_top1;
  if (fuse_silu) {
    g2.A = w.ic0;
    g2.lda = 2 * I;
    g2.a_silu = 1;
  }
  if (pair_silu) {
    g1.silu_pair = 1;
    g1.out = w.ic1;
    g1.ldo = I;
  }
  if (fold_top1) {
    g2.out = out;
    g2.ldo = H;
    g2.top1_w = wts;
  }
  for (int stage = 0; stage < 2; ++stage) {
    if (stage == 1 && sp1.n > 1)
      launch_split_silu_mul(w.partial, sp1.n, R * 2 * I, R, I, w.ic1, st);
    else if (stage == 1 && !fuse_silu && !pair_silu)
      launch_silu_mul(w.ic0, R, I, 2 * I, w.ic1, w.ic1_q, w.ic1_s, st);
    GemmArgs& g = stage == 0 ? g1 : g2;
    const int mode = stage == 0 ? ROWS_GATHER_TOK : ROWS_COMPACT_IN;
    const bool out_f32 = (stage == 1 && !fold_top1) || (stage == 0 && sp1.n > 1);
    // bf16 activations: the 16/32/64/128-row tile classes go out together in one grouped launch
    GemmArgs grp[4] = {g, g, g, g};
    int64_t grp_ub[4] = {0, 0, 0, 0};
    for (int c = 0; c < kNumClasses; ++c) {
      const int64_t ub = class_bound(c, R, E, mbk, pol);
      if (ub <= 0) continue;
      g.rt.work_desc = w.class_lists + int64_t(c) * mbk * 4;
      g.rt.work_count = w.class_counts + c;
      // Tiny blocks: the weight-streaming MFMA kernel keeps a pass of activation rows over the
      // whole K in LDS; past its LDS cap they take the 16-row MFMA tile.  The vector-ALU GEMV
      // alternative reads the plain weight layout only.
      const bool skinny_fits = skinny_lds_bytes(wfmt_w16, act_quant, g.K) <= kSkinnyMaxLds;
      const bool use_gemv = tiny == MXQ_TINY_GEMV && !tiled;
      const int tile = c == 0 ? kClassTile[1] : kClassTile[c];
      if (c == 0 && use_gemv)
        launch_gemv(g, wfmt_w16, act_quant, mode, out_f32, ub, st);
      else if (c == 0 && skinny_fits)
        launch_skinny(g, wfmt_w16, act_quant, mode, out_f32, ub, st);
      else if (big_tile && c == kNumClasses - 1) {
        // blocks of 65..128 rows: the 128 x 256 three-stage direct-to-LDS tile, and for a
        // narrow last column tile the 128 x 128 tile
        const int64_t nw = wide_tile_columns(g.N);
        if (nw > 0) {
          GemmArgs gw = g;
          gw.N = nw;
          launch_gemm_w8a8_big(gw, mode, 1, out_f32, ub, st);
        }
        if (nw < g.N) launch_gemm_w8a8(column_slice(g, nw, out_f32), mode, 0, out_f32, ub, st);
      }
      else if (act_quant)
        launch_gemm_w8a8(g, mode, tile, out_f32, ub, st);
      else if (c == 0)
        launch_gemm_w16(g, wfmt_w16, mode, tile, out_f32, ub, st);
      else {
        grp[3 - tile] = g;  // tile 3 (16 rows) .. tile 0 (128 rows)
        grp_ub[3 - tile] = ub;
      }
    }
    if (self_route) {
      const bool live[4] = {grp_ub[0] > 0, grp_ub[1] > 0, grp_ub[2] > 0, grp_ub[3] > 0};
      launch_gemm_w16_ring_routed(g, stage == 0 ? self_mbk1 : self_mbk2, live, wfmt_w16, mode, out_f32, st);
    } else if (!act_quant) {
      if (ring)
        launch_gemm_w16_ring(grp, grp_ub, wfmt_w16, mode, out_f32, st);
      else
        launch_gemm_w16_grouped(grp, grp_ub, wfmt_w16, mode, out_f32, st);
    }
  }
  if (sp2.n > 1)
    launch_combine(w.partial, sp2.n, R * H, wts, ids, E, M, topk, H, static_cast<uint16_t*>(out), st);
  else if (!fold_top1)
    launch_combine(w.y, 1, 0, wts, ids, E, M, topk, H, static_cast<uint16_t*>(out), st);
  return launch_status();
}

int dense_tile_for(int64_t M) { return M <= 16 ? 3 : M <= 32 ? 2 : M <= 64 ? 1 : 0; }

int64_t tile_rows(int tile) { return tile == 0 ? 128 : tile == 1 ? 64 : tile == 2 ? 32 : 16; }

// Dense bf16-activation tiles: the smallest tile that holds M rows, then smaller row tiles
// while the grid (row tiles x 128-column tiles x batch) stays under one workgroup per compute
// unit -- a small product is bound by the latency of its K steps, which shorter row tiles
// take in less time, and more workgroups overlap (per-tensor 97 x 576 x 224: 15.0 -> 8.7 us;
// 128 heads of [64, 512] x [128, 512]^T: 11.4 -> 9.8 us).
int dense_w16_tile(int64_t M, int64_t N, int64_t batch) {
  int tile = dense_tile_for(M);
  while (tile < 3 && cdiv(M, tile_rows(tile)) * cdiv(N, int64_t(128)) * batch < 256) ++tile;
  return tile;
}

// Dense per-tensor products take the ring-fed tiles when the grid holds at most one workgroup
// per compute unit and K spans two or more 128-wide steps: such a product is bound by the
// latency of its K steps, and the ring keeps three of them in flight (per-tensor 97 x 576 x
// 224: 8.7 -> 6.8 us; 128 heads of [64, 512] x [128, 512]^T: 9.8 -> 8.8 us).  Larger grids keep
// the register-staged tiles, two or more workgroups per compute unit (128 heads of [1024, 128]
// x [512, 128]^T: 64 against 84 us on the ring).  Both give the same bits (same products in
// the same order, the scale and bias applied after the last one).
bool dense_ring(const GemmArgs& g, int tile, int64_t batch) {
  return kDenseRing && g.K > 128 && cdiv(g.M, tile_rows(tile)) * cdiv(g.N, int64_t(128)) * batch <= 256 &&
         w16_ring_dense_supported(g, batch);
}

// Dense W8A8 GEMMs of few rows stream their weights through the tiny-block kernel (tiles of 4
// or 8 rows and 64 or 128 columns) rather than the 16..128-row tiles: they are bound by reading
// W once, which the tiles do on far fewer workgroups, each over a long serial K chain.  Used
// for M <= kSkDenseMaxRows while the tiles' grid would hold at most kSkDenseTileGrid workgroups
// (kSkDenseTileGrid8 for up to 8 rows), and for up to kSkDenseLongKRows rows whenever
// K >= kSkDenseLongK (interleaved on the box: 1 x 2048 x 7168 52.2 -> 12.4 us, 13 x 2048 x 4096
// 24.0 -> 13.6, 16 x 2048 x 7168 53.6 -> 16.9, 64 x 2048 x 7168 62.0 -> 27.9, 8 x 7168 x 2048
// 19.2 -> 14.9, 1 x 7168 x 16384 110.6 -> 38.4; with long K on wide grids 1 x 16384 x 7168
// 54.6 -> 33.2, 4 x 16384 x 4096 34.3 -> 23.6, 16 x 8192 x 7168 54.5 -> 34.9, 32 x 7168 x 7168
// 56.4 -> 52.9; the tiles stay with short K on wide grids: 8 x 24576 x 1536 16.7 against
// 19.9, 1 x 32768 x 2048 20.3 against 21.8, 16 x 7168 x 2048 19.3 against 20.4, 64 x 7168 x
// 2048 22.3 against 27.4; the bound 96 sits between a measured 56-workgroup win and
// 128-workgroup loss at K = 2048).  K is cut into S chunks (whole 128-column steps, at least four per
// chunk) until the grid reaches kSkDenseWorkgroups; the chunks' fp32 partial sums sit in the
// workspace and one more kernel adds them in chunk order.
#ifndef MXQ_SK_DENSE_MAX
#define MXQ_SK_DENSE_MAX 64
#endif
constexpr int64_t kSkDenseTileGrid = 32, kSkDenseTileGrid8 = 96;
constexpr int64_t kSkDenseLongK = 4096, kSkDenseLongKRows = 32;
#ifndef MXQ_SK_DENSE_WG
#define MXQ_SK_DENSE_WG 512
#endif
constexpr int64_t kSkDenseMaxRows = MXQ_SK_DENSE_MAX;
constexpr int64_t kSkDenseWorkgroups = MXQ_SK_DENSE_WG;
constexpr size_t kSkDenseMaxPartial = size_t(8) << 20;  // partial-sum bytes at most

struct DenseSkinny {
  bool on;
  int32_t rows;        // rows per tile (8, or 4 when eight rows of the K chunk pass the LDS cap)
  int32_t split;       // S
  int64_t chunk;       // K elements per chunk
  size_t partial_bytes;
};

// (swcol: 1 x 128 weight blocks, whose per-column scales of a K chunk also sit in LDS)
DenseSkinny dense_skinny_plan(int64_t M, int64_t N, int64_t K, bool a_e4m3, bool swcol = false) {
  DenseSkinny p{false, 8, 1, K, 0};
  if (kSkDenseMaxRows <= 0 || M < 1 || M > kSkDenseMaxRows || N < 1 || K < 128 || K % 128 != 0 ||
      N * K >= (int64_t(1) << 32))
    return p;
  const bool long_k = K >= kSkDenseLongK && M <= kSkDenseLongKRows;
  if (!long_k &&
      cdiv(M, tile_rows(dense_tile_for(M))) * cdiv(N, int64_t(128)) > (M <= 8 ? kSkDenseTileGrid8 : kSkDenseTileGrid))
    return p;
  const int64_t steps = K / 128;
  // eight rows per tile while their K chunk stays within 32 KB of LDS (several workgroups per
  // compute unit), else four within 64 KB
  for (const int ar : {8, 4}) {
    int32_t S = 1;
    const int64_t wgs = cdiv(M, int64_t(ar)) * skinny_dense_col_tiles(N);
    while (S < 8 && wgs * S * 2 <= kSkDenseWorkgroups && steps >= 8 * S && size_t(4) * 2 * S * M * N <= kSkDenseMaxPartial)
      S *= 2;
    const int64_t chunk = cdiv(steps, int64_t(S)) * 128;
    if (skinny_dense_lds(N, K, ar, S > 1 ? chunk : 0, a_e4m3, swcol) > (ar == 8 ? size_t(32) << 10 : kSkinnyMaxLds))
      continue;
    p.on = true;
    p.rows = ar;
    p.split = S;
    p.chunk = chunk;
    p.partial_bytes = S > 1 ? align256(sizeof(float) * S * M * N) : 0;
    break;
  }
  return p;
}

// Dense W8A8 GEMMs of 65..1024 rows whose 128 x 128 tiles leave the GPU mostly idle (few tiles,
// K >= 4096): each tile's K range is cut into S chunks that run as workgroups of their own (the
// launch's second grid dimension), writing fp32 partial sums to the workspace, and the split-sum
// kernel adds them in chunk order.  S doubles while the grid stays within 256 workgroups and a
// chunk keeps at least four K blocks; the partial sums stay within 16 MiB and M * K within 8 M
// (so that, with the quantised activations, the allocation-free entry point's array still holds
// every input it took before).  Interleaved on the box: 128 x 2048 x 7168 75.1 -> 20.3 us,
// 96 x 2048 x 7168 70.9 -> 18.5, 300 x 520 x 4096 28.5 -> 15.2, 512 x 2048 x 7168 47.7 -> 25.9,
// 1024 x 2048 x 7168 47.4 -> 35.8; with K = 2048 it loses (1000 x 1024 x 2048 17.5 against 20.3).
#ifndef MXQ_BIG_SPLIT
#define MXQ_BIG_SPLIT 1
#endif
struct BigSplit {
  int32_t split;
  int64_t chunk;  // K elements per chunk
  size_t partial_bytes;
};

BigSplit dense_big_split(int64_t M, int64_t N, int64_t K) {
  BigSplit p{1, K, 0};
  if (!MXQ_BIG_SPLIT || M <= 64 || M > 1024 || M * K > (int64_t(8) << 20) || K % 128 != 0 || K < 4096 || K > 16384 ||
      N < 1 || N * K >= (int64_t(1) << 32) || dense_big_shape(M, N) != 3)
    return p;
  const int64_t tiles = cdiv(M, int64_t(128)) * cdiv(N, int64_t(128)), kb = K / 128;
  while (p.split < 8 && tiles * p.split * 2 <= 256 && kb >= 8 * p.split &&
         size_t(4) * 2 * p.split * M * N <= (size_t(16) << 20))
    p.split *= 2;
  p.chunk = cdiv(kb, int64_t(p.split)) * 128;
  p.partial_bytes = p.split > 1 ? align256(sizeof(float) * p.split * M * N) : 0;
  return p;
}

size_t block_linear_quant_bytes(int64_t M, int64_t K, int32_t a_dtype) {
  if (a_dtype != MXQ_DTYPE_BF16 || M <= 0 || K <= 0) return 0;
  return align256(size_t(M) * K) + align256(sizeof(float) * M * (K / 128));
}

// Per-tensor W8A16 GEMMs of few rows stream their weights the same way (the per-tensor scale
// read as a 128 x 128 block grid with strides 0), in a narrower range than W8A8: with bf16
// activations each weight byte costs a decode and two bf16 MFMAs, and the ring-fed tiles are
// stronger -- up to 16 rows, K >= 4096 (a multiple of 128), the tiles' grid at most 32
// workgroups (interleaved on the box: 1 x 2048 x 7168 35.2 -> 22.4 us, 16 x 2048 x 7168 35.3 ->
// 21.2; the tiles stay at 1 x 7168 x 2048 19.6 against 22.3, 8 x 7168 x 2048 19.6 against 22.1,
// 32 x 7168 x 7168 35.6 against 79.0, 64 x 2048 x 7168 35.2 against 41.6, and tie at
// 4 x 16384 x 4096).
#ifndef MXQ_SK_W16
#define MXQ_SK_W16 1
#endif
DenseSkinny per_tensor_skinny_plan(int64_t M, int64_t N, int64_t K) {
  if (!MXQ_SK_W16 || M > 16 || K < 4096 || cdiv(M, int64_t(16)) * cdiv(N, int64_t(128)) > 32)
    return DenseSkinny{false, 8, 1, K, 0};
  return dense_skinny_plan(M, N, K, false);
}

// Per-tensor W8A16 GEMMs on the ring-fed tiles whose grid holds at most 128 workgroups and
// K >= 6144 (N a multiple of 8): each tile's K range runs as S chunks (the launch's third grid
// dimension), fp32 partial sums to the workspace, added in chunk order by the split-sum kernel;
// S doubles while the grid stays within 256 workgroups and a chunk keeps at least four 128-wide
// steps, partial sums within 16 MiB.  Not where the weight-streaming path runs.  Interleaved
// through the Python op: 64 x 2048 x 7168 35.4 -> 23.8 us, 128 x 2048 x 7168 35.9 -> 24.7,
// 1 x 2048 x 7136 36.2 -> 22.6; at K = 4096 no gain (300 x 520 x 4096 22.1 against 22.9,
// 16 x 7168 x 4096 22.1 against 22.7).
#ifndef MXQ_RING_SPLIT
#define MXQ_RING_SPLIT 1
#endif
struct RingSplit {
  int32_t split;
  int64_t chunk;
  size_t partial_bytes;
};

RingSplit per_tensor_ring_split(int64_t M, int64_t N, int64_t K) {
  RingSplit p{1, K, 0};
  if (!MXQ_RING_SPLIT || M < 1 || N < 8 || N % 8 != 0 || K < 6144 || K % 32 != 0 || per_tensor_skinny_plan(M, N, K).on)
    return p;
  const int64_t grid = cdiv(M, tile_rows(dense_w16_tile(M, N, 1))) * cdiv(N, int64_t(128)), steps = cdiv(K, int64_t(128));
  if (!kDenseRing || grid > 128) return p;
  while (p.split < 8 && grid * p.split * 2 <= 256 && steps >= 8 * p.split &&
         size_t(4) * 2 * p.split * M * N <= (size_t(16) << 20))
    p.split *= 2;
  p.chunk = cdiv(steps, int64_t(p.split)) * 128;
  p.partial_bytes = p.split > 1 ? align256(sizeof(float) * p.split * M * N) : 0;
  return p;
}

// MX linears whose tiles (128 or 256 rows as launch_gemm_mx picks them, 256 columns) number at
// most 128 and K >= 3072 (at K = 2048 mixed through the Python op: MXFP4 1 x 7168 x 2048 22.0
// against 24.5 us split, MXFP8 256 x 2048 x 2048 25.8 -> 22.9; at 3072 32 x 4096 x 3072 27.6 ->
// 23.6 / 33.0 -> 23.5 with MXFP4 / MXFP8 weights): each tile's K range runs as S chunks (the launch's second grid
// dimension), fp32 partial sums to the workspace after the quantised activations, added in
// chunk order by the split-sum kernel; S doubles while the grid stays within 256 workgroups and a
// chunk keeps at least four 128-wide steps, partial sums within 16 MiB.
#ifndef MXQ_MX_SPLIT
#define MXQ_MX_SPLIT 1
#endif
RingSplit mx_split(int64_t M, int64_t N, int64_t K) {
  RingSplit p{1, K, 0};
  if (!MXQ_MX_SPLIT || M < 1 || N < 1 || K < 3072 || K % 128 != 0) return p;
  const int64_t nt = cdiv(N, int64_t(256)), t128 = cdiv(M, int64_t(128)) * nt;
  const int64_t tiles = (M <= 128 || t128 <= 256) ? t128 : cdiv(M, int64_t(256)) * nt, kb = K / 128;
  if (tiles > 128) return p;
  while (p.split < 8 && tiles * p.split * 2 <= 256 && kb >= 8 * p.split &&
         size_t(4) * 2 * p.split * M * N <= (size_t(16) << 20))
    p.split *= 2;
  p.chunk = cdiv(kb, int64_t(p.split)) * 128;
  p.partial_bytes = p.split > 1 ? align256(sizeof(float) * p.split * M * N) : 0;
  return p;
}

size_t mx_quant_bytes(int64_t M, int64_t K, int32_t a_dtype) {
  if (a_dtype != MXQ_DTYPE_BF16 || M <= 0 || K <= 0) return 0;
  return align256(size_t(M) * K) + align256(size_t(M) * (K / 32));
}

}  // namespace

extern "C" {

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "unsupported sizes, strides or alignment";
    case MXQ_ERR_BLOCK: return "block size must be [1,128] or [128,128] (group 128)";
    case MXQ_ERR_DTYPE: return "unsupported dtype";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERR_ARCH: return "the current device is not gfx950 (MI355X)";
    case MXQ_ERR_LAUNCH: return "kernel launch failed";
    case MXQ_ERR_ARG: return "invalid argument";
    case MXQ_ERR_SCRATCH:
      return "the quantised input exceeds the static scratch of the allocation-free entry point "
             "(MXQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t mxq_abi_version(void) { return 14; }

mxq_status mxq_init(int32_t device) {
  if (hipSetDevice(device) != hipSuccess) return MXQ_ERR_ARCH;
  MXQ_TRY(check_arch());
  void* p = nullptr;
  return scratch_ptr_current_device(&p);
}

mxq_status mxq_per_token_group_quant_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group, void* q,
                                         float* s, void* stream) {
  if (group != 128) return MXQ_ERR_BLOCK;
  if (M < 0 || K < 0 || K % 128 != 0 || ldx < K || ldx % 8 != 0) return MXQ_ERR_SHAPE;
  if (M == 0 || K == 0) return MXQ_OK;
  if (!x || !q || !s) return MXQ_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  launch_quant_1x128(static_cast<const uint16_t*>(x), M, K, ldx, static_cast<uint8_t*>(q), K, s,
                     static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t mxq_fp8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return std::max(per_tensor_skinny_plan(M, N, K).partial_bytes, per_tensor_ring_split(M, N, K).partial_bytes);
}

mxq_status mxq_fp8_scaled_mm(const void* A, int64_t M, int64_t K, int64_t lda, const void* W, int64_t N,
                             const float* scale, const void* bias, int32_t bias_dtype, void* out, int64_t ldo,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || lda < K || lda % 8 != 0 || ldo < N) return MXQ_ERR_SHAPE;
  if (bias && bias_dtype != MXQ_DTYPE_F32 && bias_dtype != MXQ_DTYPE_BF16) return MXQ_ERR_DTYPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!A || !W || !scale || !out) return MXQ_ERR_NULL;
  if (!aligned16(A) || !aligned16(W)) return MXQ_ERR_SHAPE;
  const size_t need = mxq_fp8_scaled_mm_workspace_size(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MXQ_ERR_WORKSPACE;
  MXQ_TRY(check_arch());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const DenseSkinny sk = per_tensor_skinny_plan(M, N, K);
  if (sk.on) {
    GemmArgs gs{};
    gs.A = A;
    gs.lda = lda;
    gs.W = static_cast<const uint8_t*>(W);
    gs.ldw = K;
    gs.ws = scale;  // every (column block, K block) reads the one scale
    gs.ws_s0 = 0;
    gs.ws_s1 = 0;
    gs.bias = bias;
    gs.bias_bf16 = bias_dtype == MXQ_DTYPE_BF16;
    gs.M = M;
    gs.N = N;
    gs.K = K;
    if (sk.split > 1) {
      float* part = static_cast<float*>(workspace);
      gs.out = part;
      gs.ldo = N;
      gs.k_split = sk.split;
      gs.k_chunk = sk.chunk;
      gs.split_stride = M * N;
      launch_skinny_dense(gs, sk.rows, false, true, st);
      launch_dense_split_sum(part, sk.split, M, N, static_cast<uint16_t*>(out), ldo, st);
    } else {
      gs.out = out;
      gs.ldo = ldo;
      launch_skinny_dense(gs, sk.rows, false, false, st);
    }
    return launch_status();
  }
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.W = static_cast<const uint8_t*>(W);
  g.ldw = K;
  g.ws = scale;
  g.bias = bias;
  g.bias_bf16 = bias_dtype == MXQ_DTYPE_BF16;
  g.out = out;
  g.ldo = ldo;
  g.M = M;
  g.N = N;
  g.K = K;
  const int tile = dense_w16_tile(M, N, 1);
  if (const RingSplit rs = per_tensor_ring_split(M, N, K); rs.split > 1) {
    // few ring-fed tiles over a long K: chunks of K as workgroups of their own, then the sum
    float* part = static_cast<float*>(workspace);
    GemmArgs gs = g;
    gs.out = part;
    gs.ldo = N;
    gs.k_split = rs.split;
    gs.k_chunk = rs.chunk;
    gs.split_stride = M * N;
    if (w16_ring_dense_supported(gs, 1)) {
      launch_gemm_w16_ring_dense(gs, tile, 1, st);
      launch_dense_split_sum(part, rs.split, M, N, static_cast<uint16_t*>(out), ldo, st);
      return launch_status();
    }
  }
  if (dense_ring(g, tile, 1))
    launch_gemm_w16_ring_dense(g, tile, 1, static_cast<hipStream_t>(stream));
  else
    launch_gemm_w16(g, W_E4M3_TENSOR, ROWS_DENSE, tile, false, cdiv(M, tile_rows(tile)),
                    static_cast<hipStream_t>(stream));
  return launch_status();
}

mxq_status mxq_fp8_scaled_bmm(const void* A, int64_t batch, int64_t M, int64_t K, int64_t lda, int64_t a_bstride,
                              const void* W, int64_t N, int64_t w_bstride, const float* scale,
                              int64_t scale_bstride, const void* bias, int32_t bias_dtype, int64_t bias_bstride,
                              void* out, int64_t ldo, int64_t o_bstride, void* stream) {
  if (batch < 0 || batch > 65535 || M < 0 || N < 0 || K < 0 || K % 32 != 0 || lda < K || lda % 8 != 0 ||
      ldo < N)
    return MXQ_ERR_SHAPE;
  if (bias && bias_dtype != MXQ_DTYPE_F32 && bias_dtype != MXQ_DTYPE_BF16) return MXQ_ERR_DTYPE;
  if (batch == 0 || M == 0 || N == 0) return MXQ_OK;
  // inputs may be shared between entries (stride 0 included); outputs may not overlap
  if (a_bstride < 0 || a_bstride % 8 != 0 || w_bstride < 0 || w_bstride % 16 != 0 || scale_bstride < 0 ||
      bias_bstride < 0 || o_bstride < 0 || (batch > 1 && o_bstride < (M - 1) * ldo + N))
    return MXQ_ERR_SHAPE;
  if (!A || !W || !scale || !out) return MXQ_ERR_NULL;
  if (!aligned16(A) || !aligned16(W)) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.a_bstride = a_bstride;
  g.W = static_cast<const uint8_t*>(W);
  g.ldw = K;
  g.w_estride = w_bstride;
  g.ws = scale;
  g.ws_estride = scale_bstride;
  g.bias = bias;
  g.bias_bf16 = bias_dtype == MXQ_DTYPE_BF16;
  g.bias_estride = bias_bstride;
  g.out = out;
  g.ldo = ldo;
  g.o_bstride = o_bstride;
  g.M = M;
  g.N = N;
  g.K = K;
  const int tile = dense_w16_tile(M, N, batch);
  if (dense_ring(g, tile, batch))
    launch_gemm_w16_ring_dense(g, tile, batch, static_cast<hipStream_t>(stream));
  else
    launch_gemm_w16_batched(g, tile, batch, static_cast<hipStream_t>(stream));
  return launch_status();
}


size_t mxq_block_fp8_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t a_dtype) {
  if (M <= 0 || N <= 0 || K <= 0 || (a_dtype != MXQ_DTYPE_BF16 && a_dtype != MXQ_DTYPE_E4M3)) return 0;
  // (the weight recipe is not an argument: room for whichever plan either recipe takes)
  return block_linear_quant_bytes(M, K, a_dtype) +
         std::max({dense_skinny_plan(M, N, K, true).partial_bytes, dense_skinny_plan(M, N, K, true, true).partial_bytes,
                   dense_big_split(M, N, K).partial_bytes});
}

mxq_status mxq_block_fp8_linear(const void* A, int32_t a_dtype, const float* a_scale, int64_t M, int64_t K,
                                int64_t lda, const void* W, int64_t N, const float* w_scale, int64_t ws_stride0,
                                int64_t ws_stride1, int32_t block_n, int32_t block_k, const void* bias,
                                int32_t bias_dtype, void* out, int32_t out_dtype, int64_t ldo, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (block_k != 128 || (block_n != 1 && block_n != 128)) return MXQ_ERR_BLOCK;
  if (a_dtype != MXQ_DTYPE_BF16 && a_dtype != MXQ_DTYPE_E4M3) return MXQ_ERR_DTYPE;
  if (out_dtype != MXQ_DTYPE_BF16) return MXQ_ERR_DTYPE;
  if (bias && bias_dtype != MXQ_DTYPE_F32 && bias_dtype != MXQ_DTYPE_BF16) return MXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || lda < K || ldo < N) return MXQ_ERR_SHAPE;
  if (a_dtype == MXQ_DTYPE_BF16 ? (lda % 8 != 0) : (lda % 16 != 0)) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!A || !W || !w_scale || !out) return MXQ_ERR_NULL;
  if (a_dtype == MXQ_DTYPE_E4M3 && !a_scale) return MXQ_ERR_NULL;
  if (!aligned16(A) || !aligned16(W)) return MXQ_ERR_SHAPE;
  if (K == 0) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* qa = static_cast<const uint8_t*>(A);
  const float* sa = a_scale;
  int64_t lqa = lda;
  const size_t need = mxq_block_fp8_linear_workspace_size(M, N, K, a_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MXQ_ERR_WORKSPACE;
  if (a_dtype == MXQ_DTYPE_BF16) {
    uint8_t* q = static_cast<uint8_t*>(workspace);
    float* s = reinterpret_cast<float*>(q + align256(size_t(M) * K));
    launch_quant_1x128(static_cast<const uint16_t*>(A), M, K, lda, q, K, s, st);
    qa = q;
    sa = s;
    lqa = K;
  }
  GemmArgs g{};
  g.A = qa;
  g.lda = lqa;
  g.sa = sa;
  g.lds = K / 128;
  g.W = static_cast<const uint8_t*>(W);
  g.ldw = K;
  g.ws = w_scale;
  g.ws_s0 = ws_stride0;
  g.ws_s1 = ws_stride1;
  g.block_n = block_n;
  g.bias = bias;
  g.bias_bf16 = bias_dtype == MXQ_DTYPE_BF16;
  g.out = out;
  g.ldo = ldo;
  g.M = M;
  g.N = N;
  g.K = K;
  const DenseSkinny sk = dense_skinny_plan(M, N, K, true, block_n == 1);
  if ((block_n == 128 || block_n == 1) && sk.on && int64_t(M) * lqa < (int64_t(1) << 32)) {
    if (sk.split > 1) {
      float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + block_linear_quant_bytes(M, K, a_dtype));
      GemmArgs gs = g;
      gs.out = part;
      gs.ldo = N;
      gs.k_split = sk.split;
      gs.k_chunk = sk.chunk;
      gs.split_stride = M * N;
      launch_skinny_dense(gs, sk.rows, true, true, st, block_n == 1);
      launch_dense_split_sum(part, sk.split, M, N, static_cast<uint16_t*>(out), ldo, st);
    } else {
      launch_skinny_dense(g, sk.rows, true, false, st, block_n == 1);
    }
  } else if (const BigSplit bs = dense_big_split(M, N, K);
             bs.split > 1 && (block_n == 128 || block_n == 1) && int64_t(M) * lqa < (int64_t(1) << 32)) {
    // few 128 x 128 tiles over a long K: chunks of K as workgroups of their own, then the sum
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + block_linear_quant_bytes(M, K, a_dtype));
    GemmArgs gs = g;
    gs.out = part;
    gs.ldo = N;
    gs.k_split = bs.split;
    gs.k_chunk = bs.chunk;
    gs.split_stride = M * N;
    launch_gemm_w8a8_big(gs, ROWS_DENSE, 3, true, cdiv(M, int64_t(128)), st);
    launch_dense_split_sum(part, bs.split, M, N, static_cast<uint16_t*>(out), ldo, st);
  } else if ((block_n == 128 || block_n == 1) && K <= 16384 && int64_t(M) * lqa < (int64_t(1) << 32) &&
      N * K < (int64_t(1) << 32)) {
    // The direct-to-LDS tiles at any row count: they beat the register-staged tiles at every
    // measured M with the same bits (interleaved: 128 x 7168 x 2048 27.2 -> 18.2 us, 64 x 7168 x
    // 2048 22.2 -> 18.0, 100 x 24576 x 1536 24.0 -> 16.5, 16 x 7168 x 2048 19.1 -> 17.3,
    // 1 x 24576 x 1536 16.2 -> 15.6); the register-staged tiles keep K > 16384 and operands past
    // 4 GiB.  A 256-wide tile for the column tiles of width 256 and the register-staged 128-wide tile
    // for a narrow last one; the 128 x 128 tile for all of N
    const int shape = dense_big_shape(M, N);
    const int64_t nw = shape >= 2 ? N : wide_tile_columns(N);
    if (nw > 0) {
      GemmArgs gw = g;
      gw.N = nw;
      launch_gemm_w8a8_big(gw, ROWS_DENSE, shape, false, cdiv(M, int64_t(big_tile_rows(shape))), st);
    }
    if (nw < N) launch_gemm_w8a8(column_slice(g, nw, false), ROWS_DENSE, 0, false, cdiv(M, int64_t(128)), st);
  } else {
    const int tile = dense_tile_for(M);
    launch_gemm_w8a8(g, ROWS_DENSE, tile, false, cdiv(M, tile_rows(tile)), st);
  }
  return launch_status();
}

mxq_status mxq_block_fp8_linear_noalloc(const void* A, int32_t a_dtype, const float* a_scale, int64_t M, int64_t K,
                                        int64_t lda, const void* W, int64_t N, const float* w_scale,
                                        int64_t ws_stride0, int64_t ws_stride1, int32_t block_n, int32_t block_k,
                                        const void* bias, int32_t bias_dtype, void* out, int32_t out_dtype,
                                        int64_t ldo, void* stream) {
  // the size checks of the allocating entry point first, so that a bad shape reports as such
  if (block_k != 128 || (block_n != 1 && block_n != 128)) return MXQ_ERR_BLOCK;
  if (a_dtype != MXQ_DTYPE_BF16 && a_dtype != MXQ_DTYPE_E4M3) return MXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return MXQ_ERR_SHAPE;
  const size_t need = mxq_block_fp8_linear_workspace_size(M, N, K, a_dtype);
  if (need > size_t(MXQ_NOALLOC_SCRATCH_BYTES)) return MXQ_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && M > 0 && N > 0) {
    if (!A || !W || !w_scale || !out) return MXQ_ERR_NULL;
    MXQ_TRY(check_arch());
    MXQ_TRY(scratch_ptr_current_device(&ws));
  }
  return mxq_block_fp8_linear(A, a_dtype, a_scale, M, K, lda, W, N, w_scale, ws_stride0, ws_stride1, block_n,
                              block_k, bias, bias_dtype, out, out_dtype, ldo, ws, need, stream);
}

mxq_status mxq_mxfp8_quant(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, void* s, void* stream) {
  if (M < 0 || K < 0 || K % 32 != 0 || ldx < K || ldx % 8 != 0) return MXQ_ERR_SHAPE;
  if (M == 0 || K == 0) return MXQ_OK;
  if (!x || !q || !s) return MXQ_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  launch_quant_mx(static_cast<const uint16_t*>(x), M, K, ldx, static_cast<uint8_t*>(q), static_cast<uint8_t*>(s),
                  static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t mxq_mx_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t a_dtype) {
  if (M <= 0 || N <= 0 || K <= 0 || (a_dtype != MXQ_DTYPE_BF16 && a_dtype != MXQ_DTYPE_E4M3)) return 0;
  return mx_quant_bytes(M, K, a_dtype) + mx_split(M, N, K).partial_bytes;
}

mxq_status mxq_mx_linear(const void* A, int32_t a_dtype, const void* a_scale, int64_t M, int64_t K, int64_t lda,
                         const void* W, int32_t w_dtype, int64_t N, const void* w_scale, const void* bias,
                         int32_t bias_dtype, void* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (a_dtype != MXQ_DTYPE_BF16 && a_dtype != MXQ_DTYPE_E4M3) return MXQ_ERR_DTYPE;
  if (w_dtype != MXQ_DTYPE_E4M3 && w_dtype != MXQ_DTYPE_E2M1) return MXQ_ERR_DTYPE;
  if (bias && bias_dtype != MXQ_DTYPE_F32 && bias_dtype != MXQ_DTYPE_BF16) return MXQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || lda < K || ldo < N) return MXQ_ERR_SHAPE;
  if (a_dtype == MXQ_DTYPE_BF16 ? (lda % 8 != 0) : (lda % 16 != 0)) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (K == 0) return MXQ_ERR_SHAPE;
  if (!A || !W || !w_scale || !out) return MXQ_ERR_NULL;
  if (a_dtype == MXQ_DTYPE_E4M3 && !a_scale) return MXQ_ERR_NULL;
  const int64_t wrow = w_dtype == MXQ_DTYPE_E2M1 ? K / 2 : K;
  // operands are addressed with 32-bit byte offsets inside the kernel
  constexpr int64_t k4G = int64_t(1) << 32;
  if (M * std::max<int64_t>(lda, K) >= k4G || N * wrow >= k4G || std::max(M, N) * (K / 32) >= k4G)
    return MXQ_ERR_SHAPE;
  if (!aligned16(A) || !aligned16(W) || (reinterpret_cast<uintptr_t>(w_scale) & 3u) ||
      (a_scale && (reinterpret_cast<uintptr_t>(a_scale) & 3u)))
    return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  hipStream_t st = static_cast<hipStream_t>(stream);
  MxArgs g{};
  g.A = A;
  g.lda = lda;
  g.sa = a_scale;
  g.lds_bytes = K / 32;
  const size_t need = mxq_mx_linear_workspace_size(M, N, K, a_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MXQ_ERR_WORKSPACE;
  if (a_dtype == MXQ_DTYPE_BF16) {
    uint8_t* q = static_cast<uint8_t*>(workspace);
    uint8_t* s = q + align256(size_t(M) * K);
    launch_quant_mx(static_cast<const uint16_t*>(A), M, K, lda, q, s, st);
    g.A = q;
    g.lda = K;
    g.sa = s;
  }
  g.W = W;
  g.ldw = wrow;
  g.sw = w_scale;
  g.ldws_bytes = K / 32;
  g.w_fmt = w_dtype == MXQ_DTYPE_E2M1 ? MX_W_E2M1 : MX_W_E4M3;
  g.bias = bias;
  g.bias_bf16 = bias_dtype == MXQ_DTYPE_BF16;
  g.out = out;
  g.ldo = ldo;
  g.M = M;
  g.N = N;
  g.K = K;
  if (const RingSplit sp = mx_split(M, N, K); sp.split > 1) {
    // few tiles over a long K: chunks of K as workgroups of their own, then the sum
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + mx_quant_bytes(M, K, a_dtype));
    MxArgs gs = g;
    gs.out = part;
    gs.ldo = N;
    gs.k_split = sp.split;
    gs.k_chunk = sp.chunk;
    gs.split_stride = M * N;
    launch_gemm_mx(gs, st);
    launch_dense_split_sum(part, sp.split, M, N, static_cast<uint16_t*>(out), ldo, st);
    return launch_status();
  }
  launch_gemm_mx(g, st);
  return launch_status();
}

int64_t mxq_moe_max_blocks(int64_t M, int32_t topk, int32_t E, int32_t block_m) {
  if (M < 0 || topk <= 0 || E <= 0 || block_m <= 0) return 0;
  const int64_t R = M * topk;
  return cdiv(R, block_m) + std::min<int64_t>(E, R);
}

mxq_status mxq_moe_align(const int32_t* topk_ids, int64_t M, int32_t topk, int32_t E, int32_t block_m,
                         int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, int32_t* num_blocks,
                         void* stream) {
  if (M < 0 || topk <= 0 || E <= 0 || E > 512 || block_m <= 0 || block_m > 1024) return MXQ_ERR_SHAPE;
  if (!offsets || !num_blocks || (M > 0 && (!topk_ids || !sorted_ids || !expert_ids))) return MXQ_ERR_NULL;
  MXQ_TRY(check_arch());
  ClassPolicy pol{};
  pol.n_classes = 0;
  pol.forced = -1;
  launch_moe_align(topk_ids, M, topk, E, block_m, sorted_ids, expert_ids, offsets, num_blocks,
                   mxq_moe_max_blocks(M, topk, E, block_m), pol, nullptr, 0, nullptr, true, nullptr,
                   static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t mxq_fused_moe_workspace_size(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                                    int32_t act_quant) {
  if (M <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  (void)weights;
  return carve_moe(nullptr, M, H, I, E, topk, act_quant != 0).bytes;
}

mxq_status mxq_fused_moe_workspace_layout(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                                          int32_t act_quant, int64_t* offsets) {
  if (M <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return MXQ_ERR_SHAPE;
  if (!offsets) return MXQ_ERR_NULL;
  const bool aq = act_quant != 0 && weights == MXQ_WEIGHTS_FP8_BLOCK;
  // carve from a fake non-null base so every used region gets its offset
  uint8_t* const base = reinterpret_cast<uint8_t*>(uintptr_t(1) << 20);
  const MoeWorkspace w = carve_moe(base, M, H, I, E, topk, aq);
  auto off = [&](const void* p) -> int64_t { return p ? int64_t(static_cast<const uint8_t*>(p) - base) : -1; };
  offsets[MXQ_MOE_WS_SORTED_IDS] = off(w.sorted_ids);
  offsets[MXQ_MOE_WS_EXPERT_IDS] = off(w.expert_ids);
  offsets[MXQ_MOE_WS_OFFSETS] = off(w.offsets);
  offsets[MXQ_MOE_WS_NUM_BLOCKS] = off(w.num_blocks);
  offsets[MXQ_MOE_WS_QX] = off(w.qx);
  offsets[MXQ_MOE_WS_SX] = off(w.sx);
  offsets[MXQ_MOE_WS_IC0] = off(w.ic0);
  offsets[MXQ_MOE_WS_IC1] = off(w.ic1);
  offsets[MXQ_MOE_WS_IC1_Q] = off(w.ic1_q);
  offsets[MXQ_MOE_WS_IC1_S] = off(w.ic1_s);
  offsets[MXQ_MOE_WS_Y] = off(w.y);
  offsets[MXQ_MOE_WS_BLOCK_M] = kMoeBlockM;
  offsets[MXQ_MOE_WS_PARTIAL] = off(w.partial);
  return MXQ_OK;
}

mxq_status mxq_fused_moe_plan(int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk, int32_t weights,
                              int32_t act_quant, int32_t weight_layout, const mxq_moe_dispatch* dispatch,
                              int32_t* plan) {
  if (weights != MXQ_WEIGHTS_FP8_BLOCK && weights != MXQ_WEIGHTS_MXFP4) return MXQ_ERR_ARG;
  if (act_quant != 0 && act_quant != 1) return MXQ_ERR_ARG;
  if (weights == MXQ_WEIGHTS_MXFP4 && act_quant) return MXQ_ERR_ARG;
  if (weight_layout != MXQ_LAYOUT_PLAIN && weight_layout != MXQ_LAYOUT_TILED) return MXQ_ERR_ARG;
  mxq_moe_dispatch dc;
  MXQ_TRY(read_dispatch(dispatch, dc));
  if (M <= 0 || H <= 0 || I <= 0 || E <= 0 || E > 512 || topk <= 0 || topk > E) return MXQ_ERR_SHAPE;
  const int64_t q = weights == MXQ_WEIGHTS_MXFP4 ? 32 : 128;
  if (H % q != 0 || I % q != 0) return MXQ_ERR_SHAPE;
  if (!plan) return MXQ_ERR_NULL;
  const bool mx = weights == MXQ_WEIGHTS_MXFP4, aq = act_quant != 0, tiled = weight_layout == MXQ_LAYOUT_TILED;
  // stage arguments over stand-in pointers (16-byte aligned, as every call's pointers are)
  auto fake = [](int i) { return reinterpret_cast<void*>(uintptr_t(i) << 24); };
  const MoeWorkspace w = carve_moe(fake(1), M, H, I, E, topk, aq);
  GemmArgs g1, g2;
  moe_stage_args(g1, g2, w, fake(2), fake(3), fake(4), fake(5), fake(6), nullptr, M, H, I, topk,
                 mx ? W_E2M1_MX : W_E4M3_BLOCK, aq, tiled);
  const MoePlan p = plan_moe(g1, g2, M, H, I, E, topk, mx ? W_E2M1_MX : W_E4M3_BLOCK, aq, tiled, dc);
  const int64_t R = M * topk, mbk = mxq_moe_max_blocks(M, topk, E, kMoeBlockM);
  for (int i = 0; i < MXQ_MOE_PLAN_FIELDS; ++i) plan[i] = 0;
  if (p.expert_stream) {
    plan[MXQ_MOE_PLAN_PATH] = MXQ_MOE_PATH_EXPERT_STREAM;
    plan[MXQ_MOE_PLAN_CLASSES] = 1;
    plan[MXQ_MOE_PLAN_K_SPLIT1] = plan[MXQ_MOE_PLAN_K_SPLIT2] = 1;
    plan[MXQ_MOE_PLAN_SILU] = MXQ_MOE_SILU_EXPERT_STREAM;
    plan[MXQ_MOE_PLAN_COMBINE] = MXQ_MOE_COMBINE_KERNEL;
    return MXQ_OK;
  }
  plan[MXQ_MOE_PLAN_PATH] = p.self_route ? MXQ_MOE_PATH_SELF_ROUTED : MXQ_MOE_PATH_SORTED;
  plan[MXQ_MOE_PLAN_TILES] = aq ? (p.big_tile ? MXQ_MOE_TILES_W8A8_WIDE : MXQ_MOE_TILES_W8A8)
                                : (p.ring ? MXQ_MOE_TILES_RING : MXQ_MOE_TILES_REGISTER);
  int32_t classes = 0;
  for (int c = 0; c < kNumClasses; ++c)
    if (class_bound(c, R, E, mbk, p.pol) > 0) classes |= 1 << c;
  plan[MXQ_MOE_PLAN_CLASSES] = classes;
  plan[MXQ_MOE_PLAN_BLOCK_M1] = p.self_route ? p.bm1 : kMoeBlockM;
  plan[MXQ_MOE_PLAN_BLOCK_M2] = p.self_route ? p.bm2 : kMoeBlockM;
  plan[MXQ_MOE_PLAN_K_SPLIT1] = p.sp1.n;
  plan[MXQ_MOE_PLAN_K_SPLIT2] = p.sp2.n;
  plan[MXQ_MOE_PLAN_SILU] = p.sp1.n > 1    ? MXQ_MOE_SILU_SPLIT_SUM
                            : p.pair_silu ? MXQ_MOE_SILU_STAGE1_EPILOGUE
                            : p.fuse_silu ? MXQ_MOE_SILU_STAGE2_STAGING
                                          : MXQ_MOE_SILU_KERNEL;
  plan[MXQ_MOE_PLAN_COMBINE] = p.fold_top1 ? MXQ_MOE_COMBINE_STAGE2_EPILOGUE : MXQ_MOE_COMBINE_KERNEL;
  return MXQ_OK;
}

mxq_status mxq_silu_and_mul(const void* ic0, int64_t rows, int64_t I, int64_t ld_in, void* out, void* q, float* s,
                            void* stream) {
  if (rows < 0 || I <= 0 || I % 8 != 0 || ld_in < 2 * I || ld_in % 8 != 0) return MXQ_ERR_SHAPE;
  if (q && I % 128 != 0) return MXQ_ERR_SHAPE;
  if (rows == 0) return MXQ_OK;
  if (!ic0 || (q ? !s : !out)) return MXQ_ERR_NULL;
  if (!aligned16(ic0) || (!q && !aligned16(out)) || (q && (reinterpret_cast<uintptr_t>(q) & 7u)))
    return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  launch_silu_mul(static_cast<const uint16_t*>(ic0), rows, I, ld_in, static_cast<uint16_t*>(q ? nullptr : out),
                  static_cast<uint8_t*>(q), s, static_cast<hipStream_t>(stream));
  return launch_status();
}

static mxq_status moe_common_checks(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                                    const int32_t* ids, const float* wts, const void* w1, const void* w1s,
                                    const void* w2, const void* w2s, void* out) {
  if (M < 0 || H <= 0 || I <= 0 || E <= 0 || E > 512 || topk <= 0 || topk > E) return MXQ_ERR_SHAPE;
  if (M == 0) return MXQ_OK;
  if (!x || !ids || !wts || !w1 || !w1s || !w2 || !w2s || !out) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(out)) return MXQ_ERR_SHAPE;
  return check_arch();
}

mxq_status mxq_fused_moe_fp8(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                             const int32_t* topk_ids, const float* topk_weights, const void* w1,
                             const float* w1_scale, const void* w2, const float* w2_scale, const float* w1_bias,
                             int32_t act_quant, int32_t weight_layout, const mxq_moe_dispatch* dispatch, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (H % 128 != 0 || I % 128 != 0) return MXQ_ERR_SHAPE;
  if (act_quant != 0 && act_quant != 1) return MXQ_ERR_ARG;
  if (weight_layout != MXQ_LAYOUT_PLAIN && weight_layout != MXQ_LAYOUT_TILED) return MXQ_ERR_ARG;
  mxq_moe_dispatch dc;
  MXQ_TRY(read_dispatch(dispatch, dc));
  MXQ_TRY(moe_common_checks(x, M, H, I, E, topk, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, out));
  if (M == 0) return MXQ_OK;
  return run_moe(x, M, H, I, E, topk, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias, W_E4M3_BLOCK,
                 act_quant != 0, weight_layout == MXQ_LAYOUT_TILED, dc, out, workspace, workspace_bytes,
                 static_cast<hipStream_t>(stream));
}

mxq_status mxq_fused_moe_mxfp4(const void* x, int64_t M, int64_t H, int64_t I, int32_t E, int32_t topk,
                               const int32_t* topk_ids, const float* topk_weights, const void* w1,
                               const void* w1_scale, const void* w2, const void* w2_scale, const float* w1_bias,
                               int32_t weight_layout, const mxq_moe_dispatch* dispatch, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (H % 32 != 0 || I % 32 != 0) return MXQ_ERR_SHAPE;
  if (weight_layout != MXQ_LAYOUT_PLAIN && weight_layout != MXQ_LAYOUT_TILED) return MXQ_ERR_ARG;
  mxq_moe_dispatch dc;
  MXQ_TRY(read_dispatch(dispatch, dc));
  MXQ_TRY(moe_common_checks(x, M, H, I, E, topk, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, out));
  if (M == 0) return MXQ_OK;
  return run_moe(x, M, H, I, E, topk, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias, W_E2M1_MX, false,
                 weight_layout == MXQ_LAYOUT_TILED, dc, out, workspace, workspace_bytes,
                 static_cast<hipStream_t>(stream));
}

size_t mxq_moe_prepack_size(int64_t E, int64_t N, int64_t row_bytes) {
  if (E <= 0 || N <= 0 || row_bytes <= 0 || N % 16 != 0 || row_bytes % 16 != 0) return 0;
  return size_t(E) * size_t(N) * size_t(tiled_steps(row_bytes)) * 128;
}

size_t mxq_moe_prepack_scales_size(int64_t E, int64_t N, int64_t groups) {
  if (E <= 0 || N <= 0 || groups <= 0 || N % 16 != 0) return 0;
  return size_t(E) * size_t(N) * size_t(tiled_scale_steps(groups)) * 8;
}

mxq_status mxq_moe_prepack(const void* w, int64_t E, int64_t N, int64_t row_bytes, void* out, void* stream) {
  if (E <= 0 || N <= 0 || row_bytes <= 0 || N % 16 != 0 || row_bytes % 16 != 0) return MXQ_ERR_SHAPE;
  if (!w || !out) return MXQ_ERR_NULL;
  if (!aligned16(w) || !aligned16(out)) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  launch_prepack_w(static_cast<const uint8_t*>(w), E, N, row_bytes, static_cast<uint8_t*>(out),
                   static_cast<hipStream_t>(stream));
  return launch_status();
}

mxq_status mxq_moe_prepack_scales(const void* s, int64_t E, int64_t N, int64_t groups, void* out, void* stream) {
  if (E <= 0 || N <= 0 || groups <= 0 || N % 16 != 0) return MXQ_ERR_SHAPE;
  if (!s || !out) return MXQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out) & 1u) return MXQ_ERR_SHAPE;
  MXQ_TRY(check_arch());
  launch_prepack_s(static_cast<const uint8_t*>(s), E, N, groups, static_cast<uint8_t*>(out),
                   static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"
