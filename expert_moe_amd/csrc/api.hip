// C ABI of the fused MoE forward: argument checks, workspace layout, launch order.
// Declarations and the contract of every entry point are in include/moe.h.
#include <initializer_list>
#include <math.h>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"

namespace {

using moe::align_chunks;

constexpr size_t kAlign = 256;
constexpr int kMaxPhysical = 4096;  // physical experts of a replicated placement

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline size_t elt_bytes(const moe_params& p) { return p.dtype == MOE_F32 ? 4 : 2; }

inline bool mult64(int32_t v) { return v > 0 && v % 64 == 0; }

int check_params(const moe_params* p) {
  if (!p) return MOE_EINVAL;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (p->scoring_func != MOE_SCORE_SOFTMAX && p->scoring_func != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (p->activation != MOE_ACT_SILU && p->activation != MOE_ACT_SWIGLUOAI) return MOE_EINVAL;
  if (p->weight_layout != MOE_WEIGHTS_ROW_MAJOR && p->weight_layout != MOE_WEIGHTS_PACKED) return MOE_EINVAL;
  if (p->weight_layout == MOE_WEIGHTS_PACKED && p->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  const int E = p->num_experts;
  if (E < 1 || p->top_k < 1 || p->top_k > E) return MOE_EINVAL;
  if (!mult64(p->hidden_size) || !mult64(p->intermediate_size)) return MOE_EINVAL;
  if (p->renormalize != 0 && p->renormalize != 1) return MOE_EINVAL;
  if (p->use_grouped_topk != 0 && p->use_grouped_topk != 1) return MOE_EINVAL;
  if (p->use_grouped_topk) {
    const int G = p->num_expert_group;
    if (G < 1 || E % G != 0 || p->topk_group < 1 || p->topk_group > G) return MOE_EINVAL;
    if (p->top_k > p->topk_group * (E / G)) return MOE_EINVAL;
    if (G > 64) return MOE_EUNSUPPORTED;
  }
  if (!isfinite(p->routed_scaling_factor)) return MOE_EINVAL;
  // a share may hold more slots than there are logical experts (replicas of a placement)
  if (p->num_local_experts < 1) return MOE_EINVAL;
  if (p->num_local_experts > 256) return MOE_EUNSUPPORTED;
  if (p->shared_intermediate_size < 0) return MOE_EINVAL;
  if (p->shared_intermediate_size > 0 && !mult64(p->shared_intermediate_size)) return MOE_EINVAL;
  if (E > 256 || p->top_k > 64) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_tokens(const moe_params& p, int64_t T) {
  if (T < 0) return MOE_EINVAL;
  // pair ids t*k+j and sorted rows are int32
  const int64_t rows = T * p.top_k + static_cast<int64_t>(p.num_local_experts) * 256;
  if (rows >= (int64_t{1} << 31)) return MOE_EUNSUPPORTED;
  // the GEMM kernels address each operand (activations, one expert's weights, the sorted
  // intermediate rows) with 32-bit byte offsets
  int64_t width = p.hidden_size;
  if (p.intermediate_size > width) width = p.intermediate_size;
  if (p.shared_intermediate_size > width) width = p.shared_intermediate_size;
  const int64_t eb = p.dtype == MOE_F32 ? 4 : 2;
  if (rows * width * eb >= (int64_t{1} << 32)) return MOE_EUNSUPPORTED;
  if (int64_t{2} * p.intermediate_size * p.hidden_size * eb >= (int64_t{1} << 32)) return MOE_EUNSUPPORTED;
  if (int64_t{2} * p.shared_intermediate_size * p.hidden_size * eb >= (int64_t{1} << 32))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Variable row blocks (block_m = 0) have a 320 x 256 bf16 tile: H and 2I multiples of 256.
bool var_blocks_ok(const moe_params& p) {
  return p.dtype == MOE_BF16 && p.hidden_size % 256 == 0 && p.intermediate_size % 128 == 0;
}

bool valid_block_m(const moe_params& p, int32_t bm) {
  return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256 || (bm == 0 && var_blocks_ok(p));
}

int pick_block_m(const moe_params& p, int64_t T) {
  // Expected rows per local expert under uniform routing: T*k/E.
  const double rows = static_cast<double>(T) * p.top_k / p.num_experts;
  if (p.dtype == MOE_F32) return 16;
  // measured on MI355X (granule sweep on every workload): past a handful of rows per expert
  // the 256-row LDS tile wins, because each expert's weights are streamed once per row block
  // (EP share 290 -> 276 us, DeepSeek-V2-shaped 747 -> 720 us, skewed T=256 329 -> 312 us
  // against granule 128); variable row blocks keep that tile height without the nearly empty
  // block of an expert whose rows run a little past a multiple of 256
  if (rows <= 12.0) return 16;
  return var_blocks_ok(p) && moe::prefer_var_blocks(p, T) ? 0 : 256;
}

// padding granule of the sorted rows
inline int granule(int bm) { return bm > 0 ? bm : 32; }

int64_t capacity(const moe_params& p, int64_t T, int bm) {
  return T * p.top_k + static_cast<int64_t>(p.num_local_experts) * (granule(bm) - 1);
}

// int32 entries of block_expert: one per block_m rows, or the variable block table (the
// count, (slot, first row) of at most capacity / 256 + 1 + E_l blocks, the end marker)
int64_t block_table_len(const moe_params& p, int64_t T, int bm) {
  const int64_t cap = capacity(p, T, bm);
  if (bm > 0) return cap / bm + 1;
  return 2 * (cap / 256 + 1 + p.num_local_experts) + 4;
}

// Workspace layout of moe_forward. Each split entry point uses only `scratch`-style
// regions it owns, placed from offset 0 of the caller's workspace.
struct Layout {
  size_t topk_ids, topk_w, topk_local, sorted_pairs, block_expert, pair_row, num_padded;
  size_t meta, chunk, y, shared_y, shared_act, scratch, total;
  // sizes of the split entry points' scratch needs
  size_t route_need, align_need, mlp_need, shared_need;
};

Layout layout(const moe_params& p, int64_t T, int bm) {
  Layout L{};
  const size_t tk = static_cast<size_t>(T) * p.top_k;
  const size_t cap = static_cast<size_t>(capacity(p, T, bm));
  const size_t eb = elt_bytes(p);
  const size_t E_l = p.num_local_experts;
  const size_t nch = static_cast<size_t>(align_chunks(T));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.topk_ids = take(tk * 4);
  L.topk_w = take(tk * 4);
  L.topk_local = take(tk * 4);
  L.sorted_pairs = take(cap * 4);
  L.block_expert = take(static_cast<size_t>(block_table_len(p, T, bm)) * 4);
  L.pair_row = take(tk * 4);
  L.num_padded = take(4);
  L.meta = take((2 * E_l + 2) * 4);
  L.chunk = take(nch * E_l * 4);
  L.y = take(cap * p.hidden_size * eb);
  L.shared_y = take(p.shared_intermediate_size ? static_cast<size_t>(T) * p.hidden_size * eb : 0);
  // the shared MLP's intermediate rows: its own region, since it runs beside the routed path
  L.shared_act = take(static_cast<size_t>(T) * p.shared_intermediate_size * eb);
  L.route_need = round_up(static_cast<size_t>(moe::router_splits(p, static_cast<int>(T))) * T *
                          p.num_experts * 4);
  L.align_need = round_up((2 * E_l + 2) * 4) + round_up(nch * E_l * 4);
  L.mlp_need = round_up(cap * p.intermediate_size * eb);
  L.shared_need = round_up(static_cast<size_t>(T) * p.shared_intermediate_size * eb);
  size_t need = L.route_need;
  if (L.mlp_need > need) need = L.mlp_need;
  L.scratch = take(need);
  L.total = o;
  // The split entry points place their own regions at offset 0; forward's total covers
  // each of them because it is at least the scratch region plus the align tables.
  if (L.align_need > L.total) L.total = L.align_need;
  return L;
}

template <typename T_>
T_* at(void* ws, size_t off) {
  return reinterpret_cast<T_*>(static_cast<char*>(ws) + off);
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Tensor pointers must be 16-byte aligned (the kernels move 16-byte vectors); NULL passes.
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return false;
  return true;
}

}  // namespace

extern "C" {

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported configuration";
    case MOE_ENOSPC: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown error";
  }
}

int moe_check_params(const moe_params* p) { return check_params(p); }

int moe_pack_weights(int64_t num_matrices, int64_t rows, int64_t cols, const void* src, void* dst,
                     void* stream) {
  if (num_matrices < 0 || rows < 16 || cols < 32 || rows % 16 != 0 || cols % 32 != 0) return MOE_EINVAL;
  if (num_matrices == 0) return MOE_OK;
  if (!src || !dst || !aligned16({src, dst})) return MOE_EINVAL;
  const int64_t chunks = num_matrices * rows * (cols / 8);
  if (chunks / num_matrices / rows != cols / 8 || chunks >= (int64_t{1} << 31)) return MOE_EINVAL;
  const int64_t bytes = chunks * 16;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_EINVAL;  // overlapping buffers
  return moe::launch_pack_weights(num_matrices, rows, cols, src, dst, as_stream(stream));
}

int moe_pick_block_m(const moe_params* p, int64_t num_tokens, int32_t* block_m) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!block_m || num_tokens < 0) return MOE_EINVAL;
  *block_m = pick_block_m(*p, num_tokens);
  return MOE_OK;
}

int64_t moe_sorted_capacity(const moe_params* p, int64_t num_tokens, int32_t block_m) {
  if (check_params(p) || num_tokens < 0 || !valid_block_m(*p, block_m)) return -1;
  return capacity(*p, num_tokens, block_m);
}

int moe_workspace_size(const moe_params* p, int64_t num_tokens, int32_t block_m, size_t* bytes) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (!valid_block_m(*p, block_m) && block_m != 0) return MOE_EINVAL;
  // 0: enough for moe_forward (its own granule) and for the split entry points with variable
  // row blocks where the shapes allow them
  size_t need = layout(*p, num_tokens, block_m == 0 ? pick_block_m(*p, num_tokens) : block_m).total;
  if (block_m == 0 && var_blocks_ok(*p)) {
    const size_t v = layout(*p, num_tokens, 0).total;
    if (v > need) need = v;
  }
  *bytes = need;
  return MOE_OK;
}

int moe_make_expert_map(int32_t num_experts, int32_t ep_size, int32_t ep_rank, int32_t* map_host) {
  if (!map_host || num_experts < 1 || ep_size < 1 || ep_size > num_experts) return MOE_EINVAL;
  if (num_experts % ep_size != 0 || ep_rank < 0 || ep_rank >= ep_size) return MOE_EINVAL;
  const int per = num_experts / ep_size;
  const int start = ep_rank * per;
  for (int e = 0; e < num_experts; ++e) map_host[e] = (e >= start && e < start + per) ? e - start : -1;
  return MOE_OK;
}

int64_t moe_weight_bytes(int64_t n_experts, int64_t hidden, int64_t inter, int32_t dtype_bytes,
                         int64_t layers) {
  if (n_experts < 0 || hidden < 0 || inter < 0 || dtype_bytes < 0 || layers < 0) return -1;
  return n_experts * (2 * inter * hidden + hidden * inter) * dtype_bytes * layers;
}

// moe_route with an optional replicated placement (eplb = NULL: the expert map is by expert id)
static int route_impl(const moe_params* p, const moe::EplbMap* eplb, int64_t num_tokens,
                      const void* x, const void* w_gate, const float* logit_bias,
                      const float* score_bias, const int32_t* expert_map, int32_t* topk_ids,
                      float* topk_w, int32_t* topk_local, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !w_gate || !expert_map || !topk_ids || !topk_w || !topk_local || !ws) return MOE_EINVAL;
  if (!aligned16({x, w_gate, ws})) return MOE_EINVAL;
  const Layout L = layout(*p, num_tokens, 16);
  if (ws_bytes < L.route_need) return MOE_ENOSPC;
  const int T = static_cast<int>(num_tokens);
  float* logits = static_cast<float*>(ws);
  return moe::launch_route(*p, T, x, w_gate, logits, logit_bias, score_bias, expert_map, topk_ids,
                           topk_w, topk_local, as_stream(stream), eplb);
}

int moe_route(const moe_params* p, int64_t num_tokens, const void* x, const void* w_gate,
              const float* logit_bias, const float* score_bias, const int32_t* expert_map,
              int32_t* topk_ids, float* topk_w, int32_t* topk_local, void* ws, size_t ws_bytes,
              void* stream) {
  return route_impl(p, nullptr, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                    topk_ids, topk_w, topk_local, ws, ws_bytes, stream);
}

int moe_align_permute(const moe_params* p, int64_t num_tokens, const int32_t* topk_local,
                      int32_t block_m, int32_t* sorted_pairs, int32_t* block_expert,
                      int32_t* pair_row, int32_t* num_padded, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (!valid_block_m(*p, block_m)) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!topk_local || !sorted_pairs || !block_expert || !pair_row || !num_padded || !ws)
    return MOE_EINVAL;
  if (!aligned16({ws})) return MOE_EINVAL;
  const Layout L = layout(*p, num_tokens, block_m);
  if (ws_bytes < L.align_need) return MOE_ENOSPC;
  int32_t* meta = static_cast<int32_t*>(ws);
  int32_t* chunk = at<int32_t>(ws, round_up((2 * static_cast<size_t>(p->num_local_experts) + 2) * 4));
  return moe::launch_align(*p, static_cast<int>(num_tokens), topk_local, block_m, sorted_pairs,
                           block_expert, pair_row, num_padded, meta, chunk, as_stream(stream));
}

int moe_grouped_mlp(const moe_params* p, int64_t num_tokens, const void* x, const void* w13,
                    const void* w2, const float* b13, const float* b2,
                    const int32_t* sorted_pairs, const int32_t* block_expert,
                    const int32_t* num_padded, int32_t block_m, void* y, void* ws,
                    size_t ws_bytes, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (!valid_block_m(*p, block_m)) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !w13 || !w2 || !sorted_pairs || !block_expert || !num_padded || !y || !ws)
    return MOE_EINVAL;
  if (!aligned16({x, w13, w2, b13, b2, y, ws})) return MOE_EINVAL;
  const Layout L = layout(*p, num_tokens, block_m);
  if (ws_bytes < L.mlp_need) return MOE_ENOSPC;
  const int rows = static_cast<int>(capacity(*p, num_tokens, block_m));
  return moe::launch_mlp(*p, static_cast<int>(num_tokens), x, w13, w2, p->intermediate_size,
                         sorted_pairs, num_padded, block_expert, block_m, rows, ws, y,
                         as_stream(stream), b13, b2);
}

int moe_expert_gate_up(const moe_params* p, int64_t num_tokens, const void* x, const void* w13,
                       const float* b13, const int32_t* sorted_pairs, const int32_t* block_expert,
                       const int32_t* num_padded, int32_t block_m, void* act, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (!valid_block_m(*p, block_m)) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !w13 || !sorted_pairs || !block_expert || !num_padded || !act) return MOE_EINVAL;
  if (!aligned16({x, w13, b13, act})) return MOE_EINVAL;
  const int rows = static_cast<int>(capacity(*p, num_tokens, block_m));
  return moe::launch_gate_up(*p, static_cast<int>(num_tokens), x, w13, p->intermediate_size,
                             sorted_pairs, num_padded, block_expert, block_m, rows, act,
                             as_stream(stream), b13);
}

int moe_expert_down(const moe_params* p, int64_t num_tokens, const void* act, const void* w2,
                    const float* b2, const int32_t* block_expert, const int32_t* num_padded,
                    int32_t block_m, void* y, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (!valid_block_m(*p, block_m)) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!act || !w2 || !block_expert || !num_padded || !y) return MOE_EINVAL;
  if (!aligned16({act, w2, b2, y})) return MOE_EINVAL;
  const int rows = static_cast<int>(capacity(*p, num_tokens, block_m));
  return moe::launch_down(*p, static_cast<int>(num_tokens), act, w2, p->intermediate_size,
                          num_padded, block_expert, block_m, rows, y, as_stream(stream), b2);
}

int moe_shared_mlp(const moe_params* p, int64_t num_tokens, const void* x,
                   const void* shared_w13, const void* shared_w2, void* shared_y, void* ws,
                   size_t ws_bytes, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (p->shared_intermediate_size == 0) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !shared_w13 || !shared_w2 || !shared_y || !ws) return MOE_EINVAL;
  if (!aligned16({x, shared_w13, shared_w2, shared_y, ws})) return MOE_EINVAL;
  const Layout L = layout(*p, num_tokens, 16);
  if (ws_bytes < L.shared_need) return MOE_ENOSPC;
  const int T = static_cast<int>(num_tokens);
  return moe::launch_mlp(*p, T, x, shared_w13, shared_w2, p->shared_intermediate_size, nullptr,
                         nullptr, nullptr, 0, T, ws, shared_y, as_stream(stream));
}

int moe_combine(const moe_params* p, int64_t num_tokens, const void* y, const int32_t* pair_row,
                const float* topk_w, const void* shared_y, void* out, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (num_tokens == 0) return MOE_OK;
  if (!y || !pair_row || !topk_w || !out) return MOE_EINVAL;
  if (!aligned16({y, shared_y, out})) return MOE_EINVAL;
  return moe::launch_combine(*p, static_cast<int>(num_tokens), y, pair_row, topk_w, shared_y, out,
                             as_stream(stream));
}

// moe_forward with an optional replicated placement (eplb = NULL: the expert map is by expert id)
// and an optional caller-owned side stream for the shared expert (side = NULL: one stream).
static int forward_impl(const moe_params* p, const moe::EplbMap* eplb, const moe_side_stream* side,
                        int64_t num_tokens, const void* x, const void* w_gate,
                        const float* logit_bias, const float* score_bias,
                        const int32_t* expert_map, const void* w13, const void* w2,
                        const float* b13, const float* b2, const void* shared_w13,
                        const void* shared_w2, void* out, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if ((shared_w13 == nullptr) != (shared_w2 == nullptr)) return MOE_EINVAL;
  const bool shared = shared_w13 != nullptr;
  if (shared && p->shared_intermediate_size == 0) return MOE_EINVAL;
  if (side && (!side->fork_event || !side->join_event || side->stream == stream)) return MOE_EINVAL;
  if (num_tokens == 0) return MOE_OK;
  if (!x || !w_gate || !expert_map || !w13 || !w2 || !out || !ws) return MOE_EINVAL;
  if (!aligned16({x, w_gate, w13, w2, b13, b2, shared_w13, shared_w2, out, ws})) return MOE_EINVAL;
  const int bm = pick_block_m(*p, num_tokens);
  const Layout L = layout(*p, num_tokens, bm);
  if (ws_bytes < L.total) return MOE_ENOSPC;
  const int T = static_cast<int>(num_tokens);
  const hipStream_t s = as_stream(stream);

  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.topk_ids);
  float* tw = topk_w_out ? topk_w_out : at<float>(ws, L.topk_w);
  int32_t* local = at<int32_t>(ws, L.topk_local);
  int32_t* sorted_pairs = at<int32_t>(ws, L.sorted_pairs);
  int32_t* block_expert = at<int32_t>(ws, L.block_expert);
  int32_t* pair_row = at<int32_t>(ws, L.pair_row);
  int32_t* num_padded = at<int32_t>(ws, L.num_padded);
  void* y = at<char>(ws, L.y);
  void* shared_y = shared ? at<char>(ws, L.shared_y) : nullptr;
  void* shared_act = at<char>(ws, L.shared_act);
  void* scratch = at<char>(ws, L.scratch);
  auto shared_mlp = [&](hipStream_t st) {
    return moe::launch_mlp(*p, T, x, shared_w13, shared_w2, p->shared_intermediate_size, nullptr,
                           nullptr, nullptr, 0, T, shared_act, shared_y, st);
  };

  // Shared expert beside the routed path, on the caller's side stream, when its gate/up
  // projection is at most four rounds of 256x256 tiles. Measured on MI355X: it then fills the
  // CUs that the routed path's launches leave idle (2-8% on the DeepSeek-V2-shaped layer at
  // T=4096 and the skewed layer at T=1 and T=256); two long GEMMs side by side (skewed T=16384,
  // six rounds) lose 1.6% to cache contention, so those run in order on `stream`.
  const int n_cu = moe::device_cu_count();
  const int64_t shared_tiles = (static_cast<int64_t>(T) + 255) / 256 *
                               ((2 * static_cast<int64_t>(p->shared_intermediate_size) + 255) / 256);
  const bool fork = side && shared && n_cu > 0 && shared_tiles <= 4 * static_cast<int64_t>(n_cu);
  hipStream_t ss = nullptr;
  hipEvent_t join = nullptr;
  if (fork) {
    ss = as_stream(side->stream);
    const hipEvent_t fork_ev = static_cast<hipEvent_t>(side->fork_event);
    join = static_cast<hipEvent_t>(side->join_event);
    if (hipEventRecord(fork_ev, s) != hipSuccess || hipStreamWaitEvent(ss, fork_ev, 0) != hipSuccess)
      return MOE_EHIP;
    rc = shared_mlp(ss);
    // the join is recorded whatever the launches returned, and `stream` always waits for it
    // below: no work on the side stream is left unjoined (a HIP graph capture needs every
    // forked stream joined back)
    if (hipEventRecord(join, ss) != hipSuccess) return rc ? rc : MOE_EHIP;
  }
  if (rc == MOE_OK)
    rc = moe::launch_route(*p, T, x, w_gate, static_cast<float*>(scratch), logit_bias, score_bias,
                           expert_map, ids, tw, local, s, eplb);
  if (rc == MOE_OK)
    rc = moe::launch_align(*p, T, local, bm, sorted_pairs, block_expert, pair_row, num_padded,
                           at<int32_t>(ws, L.meta), at<int32_t>(ws, L.chunk), s);
  if (rc == MOE_OK) {
    const int rows = static_cast<int>(capacity(*p, T, bm));
    rc = moe::launch_mlp(*p, T, x, w13, w2, p->intermediate_size, sorted_pairs, num_padded,
                         block_expert, bm, rows, scratch, y, s, b13, b2);
  }
  if (fork) {
    if (hipStreamWaitEvent(s, join, 0) != hipSuccess && rc == MOE_OK) rc = MOE_EHIP;
  } else if (rc == MOE_OK && shared) {
    rc = shared_mlp(s);
  }
  if (rc) return rc;
  return moe::launch_combine(*p, T, y, pair_row, tw, shared_y, out, s);
}

int moe_forward(const moe_params* p, int64_t num_tokens, const void* x, const void* w_gate,
                const float* logit_bias, const float* score_bias, const int32_t* expert_map,
                const void* w13, const void* w2, const float* b13, const float* b2,
                const void* shared_w13, const void* shared_w2, void* out, int32_t* topk_ids_out,
                float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(p, nullptr, nullptr, num_tokens, x, w_gate, logit_bias, score_bias,
                      expert_map, w13, w2, b13, b2, shared_w13, shared_w2, out, topk_ids_out,
                      topk_w_out, ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ replicated experts

namespace {

int check_eplb(const moe_params* p, const moe_eplb* e, moe::EplbMap* out) {
  if (!p || !e) return MOE_EINVAL;
  if (e->num_physical_experts < p->num_experts || e->num_physical_experts > kMaxPhysical)
    return MOE_EINVAL;
  if (e->max_replicas < 1 || e->max_replicas > e->num_physical_experts) return MOE_EINVAL;
  if (!e->logical_to_physical || !e->replica_count) return MOE_EINVAL;
  out->l2p = e->logical_to_physical;
  out->cnt = e->replica_count;
  out->max_rep = e->max_replicas;
  out->P = e->num_physical_experts;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_eplb_tables(int32_t num_logical, int32_t num_physical, const int32_t* physical_to_logical,
                    int32_t max_replicas, int32_t* logical_to_physical, int32_t* replica_count) {
  if (num_logical < 1 || num_physical < num_logical || num_physical > kMaxPhysical ||
      max_replicas < 1 || !physical_to_logical || !logical_to_physical || !replica_count)
    return MOE_EINVAL;
  for (int e = 0; e < num_logical; ++e) replica_count[e] = 0;
  for (int64_t i = 0; i < static_cast<int64_t>(num_logical) * max_replicas; ++i)
    logical_to_physical[i] = -1;
  for (int q = 0; q < num_physical; ++q) {
    const int e = physical_to_logical[q];
    if (e < 0 || e >= num_logical) return MOE_EINVAL;
    if (replica_count[e] == max_replicas) return MOE_EINVAL;
    logical_to_physical[static_cast<int64_t>(e) * max_replicas + replica_count[e]++] = q;
  }
  for (int e = 0; e < num_logical; ++e)
    if (replica_count[e] == 0) return MOE_EINVAL;
  return MOE_OK;
}

int moe_route_eplb(const moe_params* p, const moe_eplb* eplb, int64_t num_tokens, const void* x,
                   const void* w_gate, const float* logit_bias, const float* score_bias,
                   const int32_t* expert_map, int32_t* topk_ids, float* topk_w,
                   int32_t* topk_local, void* ws, size_t ws_bytes, void* stream) {
  moe::EplbMap m;
  int rc = check_eplb(p, eplb, &m);
  if (rc) return rc;
  return route_impl(p, &m, num_tokens, x, w_gate, logit_bias, score_bias, expert_map, topk_ids,
                    topk_w, topk_local, ws, ws_bytes, stream);
}

int moe_forward_eplb(const moe_params* p, const moe_eplb* eplb, int64_t num_tokens, const void* x,
                     const void* w_gate, const float* logit_bias, const float* score_bias,
                     const int32_t* expert_map, const void* w13, const void* w2,
                     const float* b13, const float* b2, const void* shared_w13,
                     const void* shared_w2, void* out, int32_t* topk_ids_out, float* topk_w_out,
                     void* ws, size_t ws_bytes, void* stream) {
  moe::EplbMap m;
  int rc = check_eplb(p, eplb, &m);
  if (rc) return rc;
  return forward_impl(p, &m, nullptr, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                      w13, w2, b13, b2, shared_w13, shared_w2, out, topk_ids_out, topk_w_out, ws,
                      ws_bytes, stream);
}

int moe_forward_overlap(const moe_params* p, const moe_eplb* eplb, const moe_side_stream* side,
                        int64_t num_tokens, const void* x, const void* w_gate,
                        const float* logit_bias, const float* score_bias,
                        const int32_t* expert_map, const void* w13, const void* w2,
                        const float* b13, const float* b2, const void* shared_w13,
                        const void* shared_w2, void* out, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  moe::EplbMap m;
  if (eplb) {
    int rc = check_eplb(p, eplb, &m);
    if (rc) return rc;
  }
  return forward_impl(p, eplb ? &m : nullptr, side, num_tokens, x, w_gate, logit_bias,
                      score_bias, expert_map, w13, w2, b13, b2, shared_w13, shared_w2, out,
                      topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ expert-parallel exchange

namespace {

int check_ep(const moe_params* p, int32_t ep_size) {
  int rc = check_params(p);
  if (rc) return rc;
  if (ep_size < 1 || ep_size > 256 || p->num_experts % ep_size != 0) return MOE_EINVAL;
  return MOE_OK;
}

int64_t ep_rows(const moe_params& p, int64_t T, int32_t ep_size) {
  return T * (p.top_k < ep_size ? p.top_k : ep_size);
}

struct EpLayout {
  size_t rank_of, sorted_pairs, chunk, total;
};

EpLayout ep_layout(const moe_params& p, int64_t T, int32_t ep_size) {
  EpLayout L{};
  const size_t pairs = static_cast<size_t>(T) * p.top_k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.rank_of = take(pairs * 4);
  L.sorted_pairs = take(pairs * 4);
  L.chunk = take(static_cast<size_t>(align_chunks(T)) * ep_size * 4);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

int64_t moe_ep_send_capacity(const moe_params* p, int64_t num_tokens, int32_t ep_size) {
  if (check_ep(p, ep_size) || num_tokens < 0) return -1;
  return ep_rows(*p, num_tokens, ep_size);
}

int moe_ep_workspace_size(const moe_params* p, int64_t num_tokens, int32_t ep_size, size_t* bytes) {
  int rc = check_ep(p, ep_size);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  *bytes = ep_layout(*p, num_tokens, ep_size).total;
  return MOE_OK;
}

int moe_ep_dispatch(const moe_params* p, int64_t num_tokens, int32_t ep_size,
                    const int32_t* topk_ids, const float* topk_w, const void* x, int32_t* send_pos,
                    int32_t* rank_meta, int32_t* send_token, void* send_x, int32_t* send_local,
                    float* send_w, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_ep(p, ep_size);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (num_tokens == 0) return MOE_OK;
  if (!topk_ids || !topk_w || !x || !send_pos || !rank_meta || !send_token || !send_x ||
      !send_local || !send_w || !ws)
    return MOE_EINVAL;
  if (!aligned16({x, send_x})) return MOE_EINVAL;
  const EpLayout L = ep_layout(*p, num_tokens, ep_size);
  if (ws_bytes < L.total) return MOE_ENOSPC;
  const moe::EpScratch sc{at<int32_t>(ws, L.rank_of), at<int32_t>(ws, L.sorted_pairs),
                          at<int32_t>(ws, L.chunk)};
  return moe::launch_ep_dispatch(*p, static_cast<int>(num_tokens), ep_size, topk_ids, topk_w, x,
                                 send_pos, rank_meta, send_token, send_x, send_local, send_w, sc,
                                 as_stream(stream));
}

int moe_ep_combine(const moe_params* p, int64_t num_tokens, const int32_t* send_pos,
                   const void* recv_y, void* out, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (num_tokens == 0) return MOE_OK;
  if (!send_pos || !recv_y || !out) return MOE_EINVAL;
  if (!aligned16({recv_y, out})) return MOE_EINVAL;
  return moe::launch_combine(*p, static_cast<int>(num_tokens), recv_y, send_pos, nullptr, nullptr,
                             out, as_stream(stream));
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation forward

namespace {

// moe_forward_noalloc's workspace: a file-scope device array, one copy per GPU, held until the
// process ends. Host code never passes its name (a host-side stand-in) to a kernel: it uses the
// device address that hipGetSymbolAddress returns, looked up once per device.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
};

// The device address of this device's copy of `scratch`, or NULL when the lookup failed.
void* scratch_address() {
  static ScratchAddr addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchAddr& a = addr[dev];
  std::call_once(a.once, [&a] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) a.ptr = p;
  });
  return a.ptr;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_params* p, int64_t num_tokens, const void* x,
                                   const void* w_gate, const float* logit_bias,
                                   const float* score_bias, const int32_t* expert_map,
                                   const void* w13, const void* w2, const float* b13,
                                   const float* b2, const void* shared_w13, const void* shared_w2,
                                   void* out, int32_t* topk_ids_out, float* topk_w_out,
                                   void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_tokens(*p, num_tokens))) return rc;
  if (num_tokens == 0) return MOE_OK;
  const size_t need = layout(*p, num_tokens, pick_block_m(*p, num_tokens)).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPC;
  void* ws = scratch_address();
  if (ws == nullptr) return MOE_EHIP;
  return forward_impl(p, nullptr, nullptr, num_tokens, x, w_gate, logit_bias, score_bias,
                      expert_map, w13, w2, b13, b2, shared_w13, shared_w2, out, topk_ids_out,
                      topk_w_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
