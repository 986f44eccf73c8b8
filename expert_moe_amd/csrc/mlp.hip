// Expert MLP launches (gfx950): act = silu(x W1^T) * (x W3^T), y = act W2^T.
//
// The gated-SiLU expert ("silu" activation and packed gate_up_proj (E, 2I, H) of
// recursive_replace on "vllm.model_executor.models.transformers.moe"; w13 / w2 of
// fused_experts in "ep_fused_moe_patch.py" _ep_forward Step 3). Kernel choice follows the
// number of rows per tile: the 16-row streaming kernel when few tokens reach each expert
// (weight-bandwidth bound), the 64/128-row LDS-tiled MFMA kernel otherwise.
#include "gemm.h"
#include "launch.h"

namespace moe {

namespace {

template <int BM, int BNR, int WM, int WN, int MODE>
void launch_tile(GemmArgs a, int n_rows_b, hipStream_t s) {
  a.n_tiles = n_rows_b / BNR;
  gemm_bf16_dma<BM, BNR, WM, WN, MODE><<<tile_grid(a.m_blocks, a.n_tiles), 256, 0, s>>>(a);
}

template <int MODE>
void launch_tile256(const GemmArgs& a, int n_rows_b, hipStream_t s) {
  if (n_rows_b % 256 == 0)
    launch_tile<256, 256, 2, 2, MODE>(a, n_rows_b, s);
  else if (n_rows_b % 128 == 0)
    launch_tile<256, 128, 2, 2, MODE>(a, n_rows_b, s);
  else
    launch_tile<256, 64, 4, 1, MODE>(a, n_rows_b, s);
}

template <int MODE>
void launch_tile128(const GemmArgs& a, int n_rows_b, hipStream_t s) {
  // n_rows_b: B rows spanned by the whole output (2I for the silu GEMM, H for the store)
  if (n_rows_b % 256 == 0)
    launch_tile<128, 256, 2, 2, MODE>(a, n_rows_b, s);
  else if (n_rows_b % 128 == 0)
    launch_tile<128, 128, 2, 2, MODE>(a, n_rows_b, s);
  else
    launch_tile<128, 64, 4, 1, MODE>(a, n_rows_b, s);
}

template <int MODE>
void launch_tile64(const GemmArgs& a, int n_rows_b, hipStream_t s) {
  if (n_rows_b % 256 == 0)
    launch_tile<64, 256, 1, 4, MODE>(a, n_rows_b, s);
  else if (n_rows_b % 128 == 0)
    launch_tile<64, 128, 2, 2, MODE>(a, n_rows_b, s);
  else if constexpr (MODE != kSiluMul)  // 2I is always a multiple of 128
    launch_tile<64, 64, 2, 2, MODE>(a, n_rows_b, s);
}

}  // namespace

namespace {

// Rows per tile: the sorted granule when rows are expert-sorted, else by row count.
int tile_rows(const moe_params& p, bool sorted, int block_m, int rows) {
  if (p.dtype == MOE_F32) return 16;
  if (sorted) return block_m <= 32 ? 16 : block_m;
  return rows <= 64 ? 16 : 128;
}

GemmArgs base_args(const moe_params& p, int T, const int32_t* num_padded,
                   const int32_t* block_expert, int block_m, int rows) {
  GemmArgs a{};
  a.row_div = p.top_k;
  a.M_pairs = T * p.top_k;
  a.M_rows = rows;
  a.num_padded = num_padded;
  a.block_expert = block_expert;
  a.block_m = block_m > 0 ? block_m : 1;
  return a;
}

}  // namespace

int launch_gate_up(const moe_params& p, int T, const void* x, const void* w13, int inter,
                   const int32_t* row_map, const int32_t* num_padded,
                   const int32_t* block_expert, int block_m, int rows, void* act, hipStream_t s) {
  const int H = p.hidden_size;
  const int I = inter;
  // act[r, :] = silu(x[src(r)] W1^T) * (x[src(r)] W3^T), B = w13 [2I, H] per slot.
  GemmArgs g = base_args(p, T, num_padded, block_expert, block_m, rows);
  g.A = x;
  g.row_map = row_map;
  g.B = w13;
  g.b_stride = static_cast<int64_t>(2) * I * H;
  g.K = H;
  g.N = I;
  g.N_valid = I;
  g.C = act;
  g.ldc = I;
  const int tr = tile_rows(p, row_map != nullptr, block_m, rows);
  g.m_blocks = ceil_div(rows, tr);
  if (p.dtype == MOE_F32)
    gemm_f32_tile<kSiluMul><<<g.m_blocks * (I / 32), 256, 0, s>>>(g);
  else if (tr == 16)
    gemm_bf16_stream<4, kSiluMul><<<g.m_blocks * (I / 32), 256, 0, s>>>(g);
  else if (tr == 64)
    launch_tile64<kSiluMul>(g, 2 * I, s);
  else if (tr == 128)
    launch_tile128<kSiluMul>(g, 2 * I, s);
  else
    launch_tile256<kSiluMul>(g, 2 * I, s);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_down(const moe_params& p, int T, const void* act, const void* w2, int inter,
                const int32_t* num_padded, const int32_t* block_expert, int block_m, int rows,
                void* y, hipStream_t s) {
  const int H = p.hidden_size;
  const int I = inter;
  // y[r, :] = act[r] W2^T, B = w2 [H, I] per slot; act rows are already in order.
  GemmArgs g = base_args(p, T, num_padded, block_expert, block_m, rows);
  g.A = act;
  g.row_map = nullptr;
  g.B = w2;
  g.b_stride = static_cast<int64_t>(H) * I;
  g.K = I;
  g.N = H;
  g.N_valid = H;
  g.C = y;
  g.ldc = H;
  const int tr = tile_rows(p, num_padded != nullptr, block_m, rows);
  g.m_blocks = ceil_div(rows, tr);
  if (p.dtype == MOE_F32)
    gemm_f32_tile<kStore><<<g.m_blocks * (H / 64), 256, 0, s>>>(g);
  else if (tr == 16)
    gemm_bf16_stream<4, kStore><<<g.m_blocks * (H / 64), 256, 0, s>>>(g);
  else if (tr == 64)
    launch_tile64<kStore>(g, H, s);
  else if (tr == 128)
    launch_tile128<kStore>(g, H, s);
  else
    launch_tile256<kStore>(g, H, s);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_mlp(const moe_params& p, int T, const void* x, const void* w13, const void* w2,
               int inter, const int32_t* row_map, const int32_t* num_padded,
               const int32_t* block_expert, int block_m, int rows, void* act, void* y,
               hipStream_t s) {
  int rc = launch_gate_up(p, T, x, w13, inter, row_map, num_padded, block_expert, block_m, rows,
                          act, s);
  if (rc) return rc;
  return launch_down(p, T, act, w2, inter, num_padded, block_expert, block_m, rows, y, s);
}

}  // namespace moe
