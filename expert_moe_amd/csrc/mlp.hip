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

template <int MODE>
void launch_tile128(const GemmArgs& a, int n_rows_b, hipStream_t s) {
  // n_rows_b: B rows spanned by the whole output (2I for the silu GEMM, H for the store)
  if (n_rows_b % 256 == 0)
    gemm_bf16_tile<128, 256, 2, 2, MODE><<<a.m_blocks * (n_rows_b / 256), 256, 0, s>>>(a);
  else if (n_rows_b % 128 == 0)
    gemm_bf16_tile<128, 128, 2, 2, MODE><<<a.m_blocks * (n_rows_b / 128), 256, 0, s>>>(a);
  else
    gemm_bf16_tile<128, 64, 4, 1, MODE><<<a.m_blocks * (n_rows_b / 64), 256, 0, s>>>(a);
}

template <int MODE>
void launch_tile64(const GemmArgs& a, int n_rows_b, hipStream_t s) {
  if (n_rows_b % 256 == 0)
    gemm_bf16_tile<64, 256, 1, 4, MODE><<<a.m_blocks * (n_rows_b / 256), 256, 0, s>>>(a);
  else if (n_rows_b % 128 == 0)
    gemm_bf16_tile<64, 128, 2, 2, MODE><<<a.m_blocks * (n_rows_b / 128), 256, 0, s>>>(a);
  else if constexpr (MODE != kSiluMul)  // 2I is always a multiple of 128
    gemm_bf16_tile<64, 64, 2, 2, MODE><<<a.m_blocks * (n_rows_b / 64), 256, 0, s>>>(a);
}

}  // namespace

int launch_mlp(const moe_params& p, int T, const void* x, const void* w13, const void* w2,
               int inter, const int32_t* row_map, const int32_t* num_padded,
               const int32_t* block_expert, int block_m, int rows, void* act, void* y,
               hipStream_t s) {
  const int H = p.hidden_size;
  const int I = inter;
  // GEMM 1: act[r, :] = silu(x[src(r)] W1^T) * (x[src(r)] W3^T), B = w13 [2I, H] per slot.
  GemmArgs g1{};
  g1.A = x;
  g1.row_map = row_map;
  g1.row_div = p.top_k;
  g1.M_pairs = T * p.top_k;
  g1.M_rows = rows;
  g1.num_padded = num_padded;
  g1.block_expert = block_expert;
  g1.block_m = block_m > 0 ? block_m : 1;
  g1.B = w13;
  g1.b_stride = static_cast<int64_t>(2) * I * H;
  g1.K = H;
  g1.N = I;
  g1.N_valid = I;
  g1.C = act;
  g1.ldc = I;
  // GEMM 2: y[r, :] = act[r] W2^T, B = w2 [H, I] per slot; act rows are already in order.
  GemmArgs g2 = g1;
  g2.A = act;
  g2.row_map = nullptr;
  g2.B = w2;
  g2.b_stride = static_cast<int64_t>(H) * I;
  g2.K = I;
  g2.N = H;
  g2.N_valid = H;
  g2.C = y;
  g2.ldc = H;

  if (p.dtype == MOE_F32) {
    g1.m_blocks = g2.m_blocks = ceil_div(rows, 16);
    gemm_f32_tile<kSiluMul><<<g1.m_blocks * (I / 32), 256, 0, s>>>(g1);
    MOE_LAUNCH_CHECK();
    gemm_f32_tile<kStore><<<g2.m_blocks * (H / 64), 256, 0, s>>>(g2);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  // Rows per tile: the sorted granule when rows are expert-sorted, else by token count.
  const int tile_rows = row_map ? (block_m <= 32 ? 16 : block_m) : (rows <= 64 ? 16 : 128);
  if (tile_rows == 16) {
    g1.m_blocks = g2.m_blocks = ceil_div(rows, 16);
    gemm_bf16_stream<4, kSiluMul><<<g1.m_blocks * (I / 32), 256, 0, s>>>(g1);
    MOE_LAUNCH_CHECK();
    gemm_bf16_stream<4, kStore><<<g2.m_blocks * (H / 64), 256, 0, s>>>(g2);
    MOE_LAUNCH_CHECK();
  } else if (tile_rows == 64) {
    g1.m_blocks = g2.m_blocks = ceil_div(rows, 64);
    launch_tile64<kSiluMul>(g1, 2 * I, s);
    MOE_LAUNCH_CHECK();
    launch_tile64<kStore>(g2, H, s);
    MOE_LAUNCH_CHECK();
  } else {
    g1.m_blocks = g2.m_blocks = ceil_div(rows, 128);
    launch_tile128<kSiluMul>(g1, 2 * I, s);
    MOE_LAUNCH_CHECK();
    launch_tile128<kStore>(g2, H, s);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace moe
