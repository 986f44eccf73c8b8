// Expert MLP launches (gfx950): act = silu(x W1^T) * (x W3^T), y = act W2^T.
//
// The gated-SiLU expert ("silu" activation and packed gate_up_proj (E, 2I, H) of
// recursive_replace on "vllm.model_executor.models.transformers.moe"; w13 / w2 of
// fused_experts in "ep_fused_moe_patch.py" _ep_forward Step 3). Kernel choice follows the
// number of rows per tile: the 16-row streaming kernel when few tokens reach each expert
// (weight-bandwidth bound), the 64/128-row LDS-tiled MFMA kernel otherwise.
#include <atomic>
#include <cmath>

#include "gemm.h"
#include "launch.h"

namespace moe {

namespace {

// Compute units of the current device (cached per device; callers on several host threads may
// fill an entry at once, with the same value).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The LDS tile with the weight hint of the launch (GemmArgs::b_nt) as a compile-time choice.
template <int BM, int BNR, int WM, int WN, int MODE, int NS, bool SKIP>
int launch_dma(const GemmArgs& a, int grid, int threads, size_t dyn, hipStream_t s) {
  if (a.b_nt) return launch(gemm_bf16_dma<BM, BNR, WM, WN, MODE, NS, SKIP, true>, grid, threads, dyn, s, a);
  return launch(gemm_bf16_dma<BM, BNR, WM, WN, MODE, NS, SKIP, false>, grid, threads, dyn, s, a);
}

template <int BM, int BNR, int WM, int WN, int MODE>
int launch_tile_only(GemmArgs a, int n_rows_b, int est_blocks, int tail_mode, hipStream_t s) {
  a.n_tiles = n_rows_b / BNR;
  a.tail_mode = tail_mode;
  a.n_cu = cu_count();
  constexpr size_t kLdsCu = 160 * 1024;
  constexpr size_t kStage = static_cast<size_t>(BM + BNR) * 128;
  constexpr int kThreads = 64 * WM * WN;
  if (tail_mode == 2) {
    // Quarter tiles of a tail, at most one per CU: three LDS stages (loads two K steps ahead)
    // where they fit, and more than half of the CU's LDS reserved (unused) so that the
    // dispatcher cannot stack two on one CU while others stay idle.
    constexpr int NS = 3 * kStage <= kLdsCu ? 3 : 2;
    constexpr size_t kStatic = NS * kStage;
    const size_t dyn = kStatic <= kLdsCu / 2 ? kLdsCu / 2 + 1024 - kStatic : 0;
    const int grid = (a.n_cu + kXcds - 1) / kXcds * kXcds;
    if (a.valid_map) return launch_dma<BM, BNR, WM, WN, MODE, NS, true>(a, grid, kThreads, dyn, s);
    return launch_dma<BM, BNR, WM, WN, MODE, NS, false>(a, grid, kThreads, dyn, s);
  } else {
    // Three stages (one workgroup per CU) where two already take more than half of the CU's
    // LDS, or where the expected tiles fill at most two rounds of the CUs, so that latency and
    // not occupancy bounds them; otherwise two stages and two or more workgroups per CU.
    constexpr bool kFits3 = 3 * kStage <= kLdsCu;
    constexpr bool kBig = 2 * kStage > kLdsCu / 2;
    const bool few = static_cast<int64_t>(est_blocks) * a.n_tiles <= 2 * static_cast<int64_t>(a.n_cu);
    const int grid = tile_grid(a.m_blocks, a.n_tiles);
    constexpr int NS3 = kFits3 ? 3 : 2;
    const bool deep = kFits3 && (kBig || few);
    // sorted rows skip padding row groups; dense launches keep the branch-free loop
    if (a.valid_map) {
      if (deep) return launch_dma<BM, BNR, WM, WN, MODE, NS3, true>(a, grid, kThreads, 0, s);
      return launch_dma<BM, BNR, WM, WN, MODE, 2, true>(a, grid, kThreads, 0, s);
    }
    if (deep) return launch_dma<BM, BNR, WM, WN, MODE, NS3, false>(a, grid, kThreads, 0, s);
    return launch_dma<BM, BNR, WM, WN, MODE, 2, false>(a, grid, kThreads, 0, s);
  }
}

// Quarter tile (half BM, half BNR) and its wave grid for the tail launch; BM2 = 0: none.
template <int BM, int BNR, int MODE> struct Quarter { static constexpr int BM2 = 0, WM = 0, WN = 0; };
template <int MODE> struct Quarter<256, 256, MODE> { static constexpr int BM2 = 128, WM = 4, WN = 2; };
template <int MODE> struct Quarter<128, 256, MODE> { static constexpr int BM2 = 64, WM = 2, WN = 2; };
template <int MODE> struct Quarter<256, 128, MODE> { static constexpr int BM2 = 128, WM = 4, WN = 1; };
template <> struct Quarter<128, 128, kStore> { static constexpr int BM2 = 64, WM = 2, WN = 2; };

// A tile launch; when the shape has a quarter tile, the full-size launch leaves the tail of
// its last round (decided on the device from the row count) to a quarter-tile launch.
template <int BM, int BNR, int WM, int WN, int MODE>
int launch_tile(GemmArgs a, int n_rows_b, int est_blocks, hipStream_t s) {
  using Q = Quarter<BM, BNR, MODE>;
  if constexpr (Q::BM2 == 0) {
    return launch_tile_only<BM, BNR, WM, WN, MODE>(a, n_rows_b, est_blocks, 0, s);
  } else {
    const int n_cu = cu_count();
    if (n_cu <= 0) return launch_tile_only<BM, BNR, WM, WN, MODE>(a, n_rows_b, est_blocks, 0, s);
    if (a.num_padded == nullptr) {
      // dense rows: the tile count is known here, so is whether there is a tail to split
      const int total = ceil_div(a.M_rows, BM) * (n_rows_b / BNR);
      const int rem = total % n_cu;
      if (rem == 0 || 4 * rem > n_cu)
        return launch_tile_only<BM, BNR, WM, WN, MODE>(a, n_rows_b, est_blocks, 0, s);
    }
    if (int rc = launch_tile_only<BM, BNR, WM, WN, MODE>(a, n_rows_b, est_blocks, 1, s)) return rc;
    a.m_blocks = 0;  // unused in tail mode 2
    return launch_tile_only<Q::BM2, BNR / 2, Q::WM, Q::WN, MODE>(a, n_rows_b, 4 * est_blocks, 2, s);
  }
}

// Weight-row tile (BNR) for a launch: the widest of 256 / 128 / 64 that divides n_rows_b and
// still gives about two workgroups per CU for the expected number of row blocks.
inline int pick_bnr(int n_rows_b, int est_blocks, bool silu) {
  constexpr int kWant = 480;
  if (n_rows_b % 256 == 0 && est_blocks * (n_rows_b / 256) >= kWant) return 256;
  // gate/up tiles pair gate and up rows: 2I is a multiple of 128, and 128 keeps the pairs
  if (n_rows_b % 128 == 0 && (est_blocks * (n_rows_b / 128) >= kWant || silu)) return 128;
  return 64;
}

// BNR of a 256-row tile launch (one workgroup per CU): the width whose tiles are expected to
// finish first, counting rounds of one tile per CU (a tail of at most a quarter round goes to
// quarter tiles, about 0.6 of a round) times the time of one tile relative to a 128-wide one
// (measured on the sorted MoE GEMMs: 1.7 for 256, about 0.6 for 64). Ties go to the wider.
inline int pick_bnr256(int n_rows_b, int est_blocks, bool silu, int n_cu) {
  if (n_cu <= 0) return pick_bnr(n_rows_b, est_blocks, silu);
  struct Cand { int bnr; double w; bool quarter; };
  // 192 (three 64-row blocks) only for widths that 128 does not divide (e.g. 2880), where the
  // only other choice is the narrow 64 (its gate/up pairs need an even block count)
  constexpr Cand cands[4] = {{256, 1.7, true}, {192, 1.35, false}, {128, 1.0, true}, {64, 0.6, false}};
  int best = 0;
  double best_cost = 0.0;
  for (const Cand& c : cands) {
    if (n_rows_b % c.bnr != 0 || (silu && c.bnr < 128)) continue;
    if (c.bnr == 192 && (silu || n_rows_b % 128 == 0)) continue;
    const int64_t tiles = static_cast<int64_t>(est_blocks) * (n_rows_b / c.bnr);
    const int64_t full = tiles / n_cu;
    const int64_t rem = tiles % n_cu;
    const double tail = rem == 0 ? 0.0 : (c.quarter && 4 * rem <= n_cu) ? 0.6 : 1.0;
    const double cost = (static_cast<double>(full) + tail) * c.w;
    if (best == 0 || cost < best_cost) {
      best = c.bnr;
      best_cost = cost;
    }
  }
  return best;
}

// Wave grids: 8 waves (two per SIMD) wherever the tile splits into 8 blocks of whole MFMA
// tiles with gate/up pairs; measured faster than 4 on the 256-row tiles.
template <int MODE>
int launch_tile256(const GemmArgs& a, int n_rows_b, int bnr, int est, hipStream_t s) {
  if (bnr == 256) return launch_tile<256, 256, 2, 4, MODE>(a, n_rows_b, est, s);
  if constexpr (MODE == kStore) {
    if (bnr == 192) return launch_tile<256, 192, 4, 2, MODE>(a, n_rows_b, est, s);
  }
  if (bnr == 128) return launch_tile<256, 128, 4, 2, MODE>(a, n_rows_b, est, s);
  return launch_tile<256, 64, 8, 1, MODE>(a, n_rows_b, est, s);
}

template <int MODE>
int launch_tile128(const GemmArgs& a, int n_rows_b, int bnr, int est, hipStream_t s) {
  if (bnr == 256) return launch_tile<128, 256, 2, 4, MODE>(a, n_rows_b, est, s);
  if (bnr == 128) return launch_tile<128, 128, 4, 2, MODE>(a, n_rows_b, est, s);
  return launch_tile<128, 64, 4, 1, MODE>(a, n_rows_b, est, s);
}

template <int MODE>
int launch_tile64(const GemmArgs& a, int n_rows_b, int bnr, int est, hipStream_t s) {
  if (bnr == 256) return launch_tile<64, 256, 1, 4, MODE>(a, n_rows_b, est, s);
  if (bnr == 128) return launch_tile<64, 128, 2, 2, MODE>(a, n_rows_b, est, s);
  if constexpr (MODE != kSiluMul)  // 2I is always a multiple of 128
    return launch_tile<64, 64, 2, 2, MODE>(a, n_rows_b, est, s);
  return MOE_EINVAL;
}

}  // namespace

namespace {

// Kernel family and rows per row block of a launch. Expert-sorted rows follow the padding
// granule (each row block stays inside one expert); dense rows follow the row count.
//   stream MB=1/2   : 16/32 rows, weights streamed from global memory into MFMA operands
//   tile 64/128/256 : LDS-fed MFMA tile (measured faster from 64 rows up inside the MoE,
//                     where the row blocks of one expert share each weight tile in L2)
struct Plan {
  bool stream;
  int rows;  // rows per row block
};

// Dense rows: the tile height whose launch is expected to finish first, counting whole rounds
// of one tile per CU; a 256-row tile takes about 1.9x a 128-row one (dense MI355X timing:
// 1.40 vs 1.34 PFLOP/s).
int dense_tile_rows(int rows, int n_rows_b) {
  if (rows <= 1024) return 64;
  const int n_cu = cu_count() > 0 ? cu_count() : 256;
  const int64_t t128 = static_cast<int64_t>(ceil_div(rows, 128)) * (n_rows_b / 256);
  const int64_t t256 = static_cast<int64_t>(ceil_div(rows, 256)) * (n_rows_b / 256);
  const double r128 = static_cast<double>((t128 + n_cu - 1) / n_cu);
  const double r256 = 1.91 * static_cast<double>((t256 + n_cu - 1) / n_cu);
  return r256 < r128 ? 256 : 128;
}

Plan plan_rows(const moe_params& p, bool sorted, int block_m, int rows, int n_rows_b) {
  if (p.dtype == MOE_F32) return {false, 16};
  const int r = sorted ? block_m : rows;
  if (r <= 16) return {true, 16};
  if (r <= 32) return {true, 32};
  if (sorted) return {false, block_m};
  return {false, dense_tile_rows(rows, n_rows_b)};
}

// Expected share of padding rows in the expert-sorted row blocks of tr rows, with the same
// spread of per-expert loads as est_row_blocks (padding ends each expert's segment).
double est_padding(const moe_params& p, int T, int tr) {
  const double per = static_cast<double>(T) * p.top_k / p.num_experts;
  double pad = 0.0, all = 0.0;
  for (int i = 0; i < 8; ++i) {
    const double c = per * (0.825 + 0.05 * i);
    const double blocks = std::ceil((c > 1.0 ? c : 1.0) / tr) * tr;
    pad += blocks - c;
    all += blocks;
  }
  return all > 0.0 ? pad / all : 0.0;
}

// Under 512 rows per expert expected, one or two row blocks read each weight tile, so the
// weights stream from HBM rather than from L2.
bool stream_var_blocks(const moe_params& p, int T) {
  return static_cast<double>(T) * p.top_k < 512.0 * p.num_experts;
}

// Weights read by one or two row blocks (under 512 rows per expert expected, or a dense launch
// of at most 512 rows) stream through with the non-temporal hint; weight tiles that serve more
// row blocks from L2 load without it (measured, hint on every weight load: EP share T=8192
// 0.240 -> 0.218 ms, skewed T=256 0.272 -> 0.235 ms, but Mixtral-shaped T=4096 +4.6%,
// DeepSeek-V2-shaped (its dense 4096-row shared expert) +5.7%, skewed T=16384 +3.9%).
int weights_streamed(const moe_params& p, int T, bool sorted) {
  return sorted ? stream_var_blocks(p, T) : T <= 512;
}

// Row blocks a launch is expected to have: the dense row count, or for expert-sorted rows
// every local expert's expected blocks, with the expert's rows taken as the uniform-routing
// mean spread evenly over +-17.5% (eight points) and weighted by the chance that the expert is
// routed at all.
int est_row_blocks(const moe_params& p, int T, bool sorted, int tr, int rows) {
  const int cap = (rows + tr - 1) / tr;
  if (!sorted) return cap;
  const double per = static_cast<double>(T) * p.top_k / p.num_experts;
  double b = 0.0;
  for (int i = 0; i < 8; ++i) {
    const double c = per * (0.825 + 0.05 * i);
    b += std::ceil((c > 1.0 ? c : 1.0) / tr);
  }
  const double touched = 1.0 - std::exp(-per);
  const int blocks = static_cast<int>(std::ceil(p.num_local_experts * touched * b / 8.0));
  return blocks < cap ? blocks : cap;
}

// Streaming kernel with MB 16-row blocks per workgroup; 32 weight rows per workgroup when 64
// would leave CUs idle. m_blocks counts row blocks of 16*MB rows.
template <int MODE, int MB>
int launch_stream_mb(GemmArgs g, int n_rows_b, int est_blocks, hipStream_t s) {
  if (est_blocks * (n_rows_b / 64) >= 512 || n_rows_b % 32 != 0) {
    g.n_tiles = n_rows_b / 64;
    return launch(gemm_bf16_stream<4, MODE, MB>, tile_grid(g.m_blocks, g.n_tiles), 256, 0, s, g);
  }
  g.n_tiles = n_rows_b / 32;
  return launch(gemm_bf16_stream<2, MODE, MB>, tile_grid(g.m_blocks, g.n_tiles), 256, 0, s, g);
}

template <int MODE>
int launch_stream(GemmArgs g, int n_rows_b, int rows_per_block, int est_blocks, hipStream_t s) {
  if (rows_per_block == 16) return launch_stream_mb<MODE, 1>(g, n_rows_b, est_blocks, s);
  return launch_stream_mb<MODE, 2>(g, n_rows_b, est_blocks, s);
}

GemmArgs base_args(const moe_params& p, int T, const int32_t* num_padded,
                   const int32_t* block_expert, int block_m, int rows) {
  GemmArgs a{};
  a.b_packed = p.weight_layout == MOE_WEIGHTS_PACKED;
  a.row_div = p.top_k;
  a.M_pairs = T * p.top_k;
  a.M_rows = rows;
  a.num_padded = num_padded;
  a.block_expert = block_expert;
  a.block_m = block_m > 0 ? block_m : 1;
  return a;
}

// One thread per 16-byte chunk of the packed output, in output order: chunk q is row
// (q / 4) % 16 and column chunk q % 4 of block q / 64; consecutive threads write consecutive
// 16 bytes.
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int rows, int cols, int total) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= total) return;
  const int kblocks = cols / 32, panels = rows / 16;
  const int blk = q >> 6, w = q & 63;
  const int kb = blk % kblocks;
  const int rest = blk / kblocks;            // matrix * panels + panel
  const int row = (rest % panels) * 16 + (w >> 2);
  const int64_t m = rest / panels;
  const int64_t src_chunk = (m * rows + row) * (cols / 8) + kb * 4 + (w & 3);
  dst[q] = src[src_chunk];
}

}  // namespace

int launch_pack_weights(int64_t n, int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s) {
  const int total = static_cast<int>(n * rows * (cols / 8));
  return launch(pack_weights_kernel, ceil_div(total, 256), 256, 0, s, static_cast<const uint4*>(src),
                static_cast<uint4*>(dst), static_cast<int>(rows), static_cast<int>(cols), total);
}

int launch_gate_up(const moe_params& p, int T, const void* x, const void* w13, int inter,
                   const int32_t* row_map, const int32_t* num_padded,
                   const int32_t* block_expert, int block_m, int rows, void* act, hipStream_t s,
                   const float* b13) {
  const int H = p.hidden_size;
  const int I = inter;
  // act[r, :] = silu(x[src(r)] W1^T) * (x[src(r)] W3^T), B = w13 [2I, H] per slot.
  GemmArgs g = base_args(p, T, num_padded, block_expert, block_m, rows);
  g.A = x;
  g.row_map = row_map;
  // Padding-row skip (per 32-row block, from the sorted pair list): its per-block branches
  // cost about 2.5% on blocks of real rows, so it is used where more than 8% of the rows are
  // expected to be padding (measured: Mixtral-shaped prefill, 12% padding, gains 2.6%; skewed
  // T=16384, whose hot experts fill whole blocks, loses 2.5% with it).
  g.valid_map = row_map != nullptr && est_padding(p, T, block_m) > 0.08 ? row_map : nullptr;
  g.B = w13;
  g.b_stride = static_cast<int64_t>(2) * I * H;
  g.K = H;
  g.N = I;
  g.N_valid = I;
  g.C = act;
  g.ldc = I;
  g.bias = b13;
  g.bias_stride = static_cast<int64_t>(2) * I;
  g.act = p.activation;
  g.b_nt = weights_streamed(p, T, row_map != nullptr);
  if (block_m == 0 && num_padded != nullptr) {
    // variable row blocks of expert-sorted rows (block_m 0 with dense rows, num_padded NULL, is
    // the dense launch below): 320 x 256 tiles over the block table; at most rows / 256 + 1 +
    // E_l blocks (the grid's worst case; workgroups past the active tiles exit)
    if (block_expert == nullptr || row_map == nullptr) return MOE_EINVAL;
    g.valid_map = nullptr;
    g.n_tiles = 2 * I / 256;
    const int nbmax = rows / 256 + 1 + p.num_local_experts;
    if (g.b_nt) return launch(gemm_bf16_var4<kSiluMul, true>, tile_grid(nbmax, g.n_tiles), 512, 0, s, g);
    return launch(gemm_bf16_var4<kSiluMul, false>, tile_grid(nbmax, g.n_tiles), 512, 0, s, g);
  }
  const bool sorted = row_map != nullptr;
  const Plan pl = plan_rows(p, sorted, block_m, rows, 2 * I);
  const int tr = pl.rows;
  g.m_blocks = ceil_div(rows, tr);
  const int est = est_row_blocks(p, T, sorted, tr, rows);
  if (p.dtype == MOE_F32) return launch(gemm_f32_tile<kSiluMul>, g.m_blocks * (I / 32), 256, 0, s, g);
  if (pl.stream) return launch_stream<kSiluMul>(g, 2 * I, tr, est, s);
  if (tr == 64) return launch_tile64<kSiluMul>(g, 2 * I, pick_bnr(2 * I, est, true), est, s);
  if (tr == 128) return launch_tile128<kSiluMul>(g, 2 * I, pick_bnr(2 * I, est, true), est, s);
  return launch_tile256<kSiluMul>(g, 2 * I, pick_bnr256(2 * I, est, true, cu_count()), est, s);
}

int launch_down(const moe_params& p, int T, const void* act, const void* w2, int inter,
                const int32_t* num_padded, const int32_t* block_expert, int block_m, int rows,
                void* y, hipStream_t s, const float* b2, const int32_t* store_map) {
  const int H = p.hidden_size;
  const int I = inter;
  // y[r, :] = act[r] W2^T, B = w2 [H, I] per slot; act rows are already in order.
  GemmArgs g = base_args(p, T, num_padded, block_expert, block_m, rows);
  g.A = act;
  g.row_map = nullptr;
  // no padding-row skip here: measured slower on the long-K down projection (Mixtral-shaped
  // prefill: 931 us with it, 814 us without), unlike the gate/up projection
  g.valid_map = nullptr;
  // Padding rows of y (the combine reads real rows only) are left unwritten where more than
  // 20% of the rows are expected to be padding; below that the per-row check costs more than
  // the stores it saves.
  g.store_map = store_map != nullptr && est_padding(p, T, block_m) > 0.2 ? store_map : nullptr;
  g.B = w2;
  g.b_stride = static_cast<int64_t>(H) * I;
  g.K = I;
  g.N = H;
  g.N_valid = H;
  g.C = y;
  g.ldc = H;
  g.bias = b2;
  g.bias_stride = H;
  g.b_nt = weights_streamed(p, T, num_padded != nullptr);
  if (block_m == 0 && num_padded != nullptr) {
    // variable row blocks of expert-sorted rows (padding is under 32 rows per expert: every
    // row is stored); block_m 0 with dense rows (num_padded NULL) is the dense launch below
    if (block_expert == nullptr) return MOE_EINVAL;
    g.store_map = nullptr;
    g.n_tiles = H / 256;
    const int nbmax = rows / 256 + 1 + p.num_local_experts;
    if (g.b_nt) return launch(gemm_bf16_var4<kStore, true>, tile_grid(nbmax, g.n_tiles), 512, 0, s, g);
    return launch(gemm_bf16_var4<kStore, false>, tile_grid(nbmax, g.n_tiles), 512, 0, s, g);
  }
  const bool sorted = num_padded != nullptr;
  const Plan pl = plan_rows(p, sorted, block_m, rows, H);
  const int tr = pl.rows;
  g.m_blocks = ceil_div(rows, tr);
  const int est = est_row_blocks(p, T, sorted, tr, rows);
  if (p.dtype == MOE_F32) return launch(gemm_f32_tile<kStore>, g.m_blocks * (H / 64), 256, 0, s, g);
  if (pl.stream) return launch_stream<kStore>(g, H, tr, est, s);
  if (tr == 64) return launch_tile64<kStore>(g, H, pick_bnr(H, est, false), est, s);
  if (tr == 128) return launch_tile128<kStore>(g, H, pick_bnr(H, est, false), est, s);
  return launch_tile256<kStore>(g, H, pick_bnr256(H, est, false, cu_count()), est, s);
}

int device_cu_count() { return cu_count(); }

bool prefer_var_blocks(const moe_params& p, int64_t T) {
  // Expected row blocks with the 256 granule and with variable blocks. A local expert's rows
  // under an even router spread like a Poisson count: mean T k / E, standard deviation its
  // square root, taken at the eight octile midpoints of a normal distribution.
  // Variable blocks pay where they remove remainder blocks: measured on MI355X, Mixtral-shaped
  // T=4096 (36 -> 32 blocks) 2.72 -> 2.46 ms, EP share gate/up + down 0.18 -> 0.14 ms; with as
  // many blocks (skewed T=16384, 1% more rows in taller tiles) they lose 1.4%, and below a round
  // of 320 x 256 tiles (skewed T=256) 7%, where the 256-row launch picks narrower tiles.
  constexpr double z[8] = {-1.534, -0.887, -0.489, -0.157, 0.157, 0.489, 0.887, 1.534};
  const double per = static_cast<double>(T) * p.top_k / p.num_experts;
  double b256 = 0.0, bvar = 0.0;
  for (int i = 0; i < 8; ++i) {
    const double c = per + z[i] * std::sqrt(per);
    const int rows = static_cast<int>(std::ceil(c > 1.0 ? c : 1.0));
    b256 += (rows + 255) / 256;
    const int c32 = (rows + 31) / 32 * 32;
    const int q = c32 / 256, r = c32 - 256 * q;
    bvar += (q >= 1 && r <= 64) ? q : q + (r > 0 ? 1 : 0);
  }
  const double touched = 1.0 - std::exp(-per);
  const double tiles = p.num_local_experts * touched * bvar / 8.0 * (2.0 * p.intermediate_size / 256.0);
  const int n_cu = cu_count() > 0 ? cu_count() : 256;
  if (bvar <= 0.95 * b256 && tiles >= n_cu) return true;
  // As many blocks, 128 to 512 rows per expert: the variable blocks run a four-stage pipeline,
  // the 256 granule a two-stage one (DeepSeek-V2-shaped, 153 rows per expert: 0.636 -> 0.619
  // ms; skewed T=256 and T=16384, 32 and 2048 rows per expert, lose 8% and 7%, and again 7% and
  // 1-2% with the weight hint only where weights stream).
  return per >= 128.0 && stream_var_blocks(p, static_cast<int>(T)) && bvar <= b256;
}

int launch_mlp(const moe_params& p, int T, const void* x, const void* w13, const void* w2,
               int inter, const int32_t* row_map, const int32_t* num_padded,
               const int32_t* block_expert, int block_m, int rows, void* act, void* y,
               hipStream_t s, const float* b13, const float* b2) {
  int rc = launch_gate_up(p, T, x, w13, inter, row_map, num_padded, block_expert, block_m, rows,
                          act, s, b13);
  if (rc) return rc;
  return launch_down(p, T, act, w2, inter, num_padded, block_expert, block_m, rows, y, s, b2,
                     row_map);
}

}  // namespace moe
