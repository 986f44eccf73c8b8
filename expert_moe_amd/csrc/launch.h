// Internal launchers of the fused MoE forward. Arguments are already validated by the
// C-ABI layer; every launcher only enqueues kernels on `s` and returns MOE_OK or MOE_EHIP.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Tokens handled by one workgroup of the align count/scatter passes.
constexpr int kAlignChunk = 256;

inline int align_chunks(int64_t T) { return static_cast<int>((T + kAlignChunk - 1) / kAlignChunk); }

// Number of K splits of the router logits GEMM for T tokens (enough workgroups to fill the
// chip when T is small): powers of two whose K ranges stay multiples of 256, or for hidden
// sizes without such a split a divisor of H / (K step) with at least four K steps per range.
int router_splits(const moe_params& p, int T);

// Router logits: router_splits() partial sums [splits, T, E] fp32 of x . Wg^T.
int launch_router_logits(const moe_params& p, int T, const void* x, const void* w_gate,
                         float* logits, hipStream_t s);

// Replicated experts: logical expert e is served by the physical experts
// l2p[e * max_rep + i], i < cnt[e]; the expert map is then indexed by physical id (P entries).
struct EplbMap {
  const int32_t* l2p;
  const int32_t* cnt;
  int max_rep;
  int P;
};

// Sum of the logit partials (written back into partial 0), fp32 softmax or sigmoid, (grouped)
// top-k on the scores plus score_bias (when given), renormalise, scale, expert_map lookup
// (through the replica of token t, t mod cnt[e], when eplb is given).
int launch_topk(const moe_params& p, int T, float* logits, const float* bias,
                const float* score_bias, const int32_t* expert_map, int32_t* ids, float* w,
                int32_t* local, hipStream_t s, const EplbMap* eplb = nullptr);

// The whole router: the logits GEMM into `logits`, then launch_topk.
int launch_route(const moe_params& p, int T, const void* x, const void* w_gate, float* logits,
                 const float* bias, const float* score_bias, const int32_t* expert_map,
                 int32_t* ids, float* w, int32_t* local, hipStream_t s, const EplbMap* eplb = nullptr);

// Count / scan / scatter of the (token, slot) pairs by local expert (block_expert may be NULL).
// meta: [num_padded(1) | offsets(E_l+1) | counts(E_l)], chunk: [align_chunks(T) * E_l].
int launch_align(const moe_params& p, int T, const int32_t* topk_local, int block_m,
                 int32_t* sorted_pairs, int32_t* block_expert, int32_t* pair_row,
                 int32_t* num_padded, int32_t* meta, int32_t* chunk, hipStream_t s);

// The two GEMMs of the expert MLP (see launch_mlp for the row modes). b13: per-slot fp32
// [slots, 2 inter] gate then up biases, b2: [slots, H], each NULL = none.
int launch_gate_up(const moe_params& p, int T, const void* x, const void* w13, int inter,
                   const int32_t* row_map, const int32_t* num_padded,
                   const int32_t* block_expert, int block_m, int rows, void* act, hipStream_t s,
                   const float* b13 = nullptr);
int launch_down(const moe_params& p, int T, const void* act, const void* w2, int inter,
                const int32_t* num_padded, const int32_t* block_expert, int block_m, int rows,
                void* y, hipStream_t s, const float* b2 = nullptr,
                const int32_t* store_map = nullptr);

// Expert MLP over rows: act = act_fn(x W1^T + b1, x W3^T + b3) (p.activation: silu(g) * u or
// the clamped SwiGLU), y = act W2^T + b2 (biases optional).
//  sorted (row_map != NULL): rows of the expert-sorted pair list, capacity rows, block_m granule;
//  dense  (row_map == NULL): the first `rows` tokens with a single weight set.
int launch_mlp(const moe_params& p, int T, const void* x, const void* w13, const void* w2,
               int inter, const int32_t* row_map, const int32_t* num_padded,
               const int32_t* block_expert, int block_m, int rows, void* act, void* y,
               hipStream_t s, const float* b13 = nullptr, const float* b2 = nullptr);

// Packed weight layout (b_offset in gemm.h) of n row-major bf16 [rows, cols] matrices; the
// total number of 16-byte chunks is below 2^31.
int launch_pack_weights(int64_t n, int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s);

// Compute units of the current device (cached per device); 0 if the query fails.
int device_cu_count();

// Whether variable row blocks are expected to beat the 256-row granule for T tokens (fewer
// row blocks, and at least a round of gate/up tiles).
bool prefer_var_blocks(const moe_params& p, int64_t T);

// Scratch of the exchange dispatch: the owning rank of every pair [T*k], the rank-sorted pair
// list [T*k], the alignment's chunk counts.
struct EpScratch {
  int32_t* rank_of;
  int32_t* sorted_pairs;
  int32_t* chunk;
};

// Dispatch plan and send buffers of the expert-parallel exchange (one row per token and
// destination rank); rank_meta: [n_send | offsets (ep_size+1) | counts (ep_size)].
int launch_ep_dispatch(const moe_params& p, int T, int ep_size, const int32_t* ids, const float* w,
                       const void* x, int32_t* send_pos, int32_t* rank_meta, int32_t* send_token,
                       void* send_x, int32_t* send_local, float* send_w, const EpScratch& ws,
                       hipStream_t s);

// out[t] = sum_j w[t,j] * y[pair_row[t,j]] (+ shared_y[t]); w = NULL: weight 1.
int launch_combine(const moe_params& p, int T, const void* y, const int32_t* pair_row,
                   const float* topk_w, const void* shared_y, void* out, hipStream_t s);

}  // namespace moe
