/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer forward,
 * computed on one expert-parallel rank's share of the experts.
 *
 * What is computed (per token t of x [T, H]):
 *   logits  = x[t] . Wg^T (+ logit_bias)        replicated router gate over ALL E experts
 *   p       = softmax(logits) in fp32 (or the logistic sigmoid of each logit)
 *   ids     = top-k of p (+ score_bias, when given: it steers the choice only), plain or
 *             group-limited, ties to the lower expert id
 *   w       = p[ids] (/ sum if renormalize) * routed_scaling_factor
 *   out[t]  = sum over slots j whose expert is local of w[j] * MLP_{ids[j]}(x[t])
 *             (+ the shared expert's MLP(x[t]), weight 1, when its weights are given)
 *   MLP(x)  = W2 (silu(W1 x) * (W3 x))  (+ expert biases; or the clamped SwiGLU, see activation)
 * Sources: "[Feature] Expert parallelism support" (sglang issue #1435), MixtralMoE.forward
 * (gate, fp32 softmax, top-k, renormalise, weighted per-expert sum, all-reduce of the
 * rank's partial sum); "ep_fused_moe_patch.py: EP-aware FusedMoE override for vllm
 * 0.6.3", _ep_init / _ep_forward (global routing on every rank, local experts at full
 * intermediate size, renormalize / grouped top-k switches, per-token sum of weighted
 * rows); "vllm.model_executor.models.transformers.moe", MoEMixin.recursive_replace
 * (routed_scaling_factor, n_group / topk_group, silu, gate_up_proj (E, 2I, H), shared
 * experts inside the fused layer); "Expert Parallel" (vllm-omni), Step 5 (shared expert
 * added on every rank).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, borrowed: the caller owns them, they must
 *    stay alive until the work queued on `stream` has finished. The library never
 *    allocates or frees device memory and keeps no state of its own besides its loaded code
 *    objects (and a per-device cache of the compute-unit count): no streams, no events, no
 *    locks. Calls from several host threads are independent.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work
 *    on it: no host<->device synchronisation, no host reads of device data, so a call
 *    can be captured in a HIP graph.
 *  - Row-major layouts. x [T, H]; Wg [E, H]; w13 [E_l, 2I, H] (rows 0..I-1 = W1 "gate",
 *    rows I..2I-1 = W3 "up"); w2 [E_l, H, I]; shared_w13 [2 I_s, H]; shared_w2 [H, I_s];
 *    out [T, H]. x, weights, y and out use `dtype` (fp32 or bf16 bit patterns);
 *    router logits, probabilities and routing weights are fp32; ids are int32.
 *  - x, weights, y, shared_y, act, out and the workspace must be 16-byte aligned (hipMalloc
 *    and torch allocations are; kernels move 16-byte vectors), else MOE_EINVAL.
 *  - Return value: MOE_OK (0) or a negative MOE_E* code; nothing is enqueued on error,
 *    except MOE_EHIP, which reports a failed launch.
 *  - expert_map [E] int32 holds, for every GLOBAL expert id, its local slot in
 *    [0, E_l) or -1 when the expert lives on another rank. Its device contents are not
 *    validated (that would need a sync); slots outside [0, E_l) are treated as -1.
 *  - T = 0 is a valid no-op.
 *  - Size limits (MOE_EUNSUPPORTED beyond them): the GEMM kernels address each operand with
 *    32-bit byte offsets, so (T*k + E_l*256) * max(H, I, I_s) * dtype_bytes must stay below
 *    4 GiB (for bf16 at H = 4096 and k = 2, below about 262 000 tokens; at I = 14336, about
 *    74 000), and so must 2*I*H*dtype_bytes and 2*I_s*H*dtype_bytes (one expert's w13);
 *    T*k + E_l*256 must stay below 2^31.
 */
#ifndef EXPERT_MOE_AMD_MOE_H
#define EXPERT_MOE_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* a parameter or a required pointer is invalid */
#define MOE_EUNSUPPORTED (-2) /* a valid request the library has no kernel for */
#define MOE_ENOSPC (-3)       /* the workspace is smaller than moe_workspace_size() */
#define MOE_EHIP (-4)         /* a HIP launch failed */

#define MOE_F32 0
#define MOE_BF16 1

#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1

#define MOE_ACT_SILU 0
#define MOE_ACT_SWIGLUOAI 1

#define MOE_WEIGHTS_ROW_MAJOR 0
#define MOE_WEIGHTS_PACKED 1

/*
 * Layer parameters, named after the EP-aware FusedMoE constructor (_ep_init on the
 * ep_fused_moe_patch.py page) and the config fields of MoEMixin.recursive_replace.
 *  num_experts               E, the GLOBAL expert count the router scores (1..256).
 *  top_k                     k, experts per token (1..E).
 *  hidden_size               H, multiple of 64.
 *  intermediate_size         I of one routed expert at full size (no TP split), multiple of 64.
 *  renormalize               1: divide the k routing weights by their sum (over all k
 *                            global picks, before the expert_map mask); 0: keep p.
 *  use_grouped_topk          1: group-limited routing; E % num_expert_group == 0,
 *                            1 <= topk_group <= num_expert_group, k <= topk_group*E/G.
 *                            A group's score is its largest probability.
 *  routed_scaling_factor     multiplies the routing weights after renormalisation
 *                            (1.0 = off); never applied to the shared expert.
 *  num_local_experts         E_l, number of local slots (1..256; more than E only for a
 *                            replicated placement, see moe_eplb; above 256: MOE_EUNSUPPORTED).
 *  shared_intermediate_size  I_s of the shared expert MLP (n_shared * I), 0 = none,
 *                            multiple of 64 otherwise.
 *  dtype                     MOE_F32 or MOE_BF16 (x, weights, y, out).
 *  scoring_func              MOE_SCORE_SOFTMAX (0, the default of a zeroed struct) or
 *                            MOE_SCORE_SIGMOID (1: p = 1 / (1 + exp(-logit)) per expert, as
 *                            DeepSeek-V3 scores; the pages name the switch, not its formula).
 *  activation                MOE_ACT_SILU (0, the default): act = silu(g) * u, or
 *                            MOE_ACT_SWIGLUOAI (1, gpt-oss): g' = min(g, 7), u' = clamp(u, -7, 7),
 *                            act = g' * sigmoid(1.702 g') * (u' + 1). recursive_replace names
 *                            "swigluoai" for gpt-oss; the formula is gpt-oss's. Applies to the
 *                            routed and the shared experts.
 *  weight_layout             MOE_WEIGHTS_ROW_MAJOR (0, the default): w13, w2, shared_w13 and
 *                            shared_w2 as listed under "Row-major layouts"; or
 *                            MOE_WEIGHTS_PACKED (1, bf16 only, else MOE_EUNSUPPORTED): the
 *                            same matrices rearranged by moe_pack_weights. The router gate
 *                            Wg is always row-major. The arithmetic (and so every result bit)
 *                            is the same for both layouts; packed weights stream from HBM in
 *                            whole 1 KiB blocks instead of row segments of 64 or 128 bytes.
 *
 * Expert biases (has_bias of recursive_replace): optional fp32 b13 [E_l, 2I] (per slot: the I
 * gate biases, then the I up biases, the order of w13's rows) added to the gate/up
 * pre-activations, and b2 [E_l, H] added to the expert output before the routing weight
 * multiplies it. NULL = none; 16-byte aligned. The shared expert has none.
 *
 * Selection bias (score_bias, "e_score_correction_bias" on the transformers MoE page, named
 * there without its use): an fp32 [E] device vector added to p for the choice only, as
 * DeepSeek-V3 does. Candidates rank by the fp32 sum p + b; with group-limited routing a
 * group's score becomes the sum of its two largest biased scores (one score for groups of
 * one); the weights still come from p. NULL = no bias (groups score by their largest p).
 */
typedef struct moe_params {
  int32_t num_experts;
  int32_t top_k;
  int32_t hidden_size;
  int32_t intermediate_size;
  int32_t renormalize;
  int32_t use_grouped_topk;
  int32_t num_expert_group;
  int32_t topk_group;
  float routed_scaling_factor;
  int32_t num_local_experts;
  int32_t shared_intermediate_size;
  int32_t dtype;
  int32_t scoring_func;
  int32_t activation;
  int32_t weight_layout;
} moe_params;

/* ------------------------------------------------------------------ host helpers */

/* Human-readable name of a return code. Never NULL. */
const char* moe_strerror(int code);

/*
 * Checks `p` (the rules listed with moe_params). MOE_OK, MOE_EINVAL or MOE_EUNSUPPORTED.
 */
int moe_check_params(const moe_params* p);

/*
 * Rearranges num_matrices row-major bf16 matrices [rows, cols], stored back to back (w13
 * [E_l, 2I, H] is E_l matrices [2I, H], w2 [E_l, H, I] is E_l matrices [H, I]; the shared
 * expert's are one matrix each), into the packed weight layout of MOE_WEIGHTS_PACKED: per
 * matrix, the 16-row panels one after the other; per panel, its cols / 32 blocks in column
 * order; per block, its 16 rows x 32 elements row-major (1 KiB). Element (m, r, c) goes to
 * element ((m * rows/16 + r/16) * cols/32 + c/32) * 512 + (r % 16) * 32 + c % 32 of dst.
 * A weight preparation step, run once per weight set: dst has the size of src and must not
 * overlap it; both 16-byte aligned device pointers. rows % 16 == 0 and cols % 32 == 0 (every
 * weight matrix of a layer with H, I, I_s multiples of 64), num_matrices >= 0, the total
 * below 2^31 16-byte chunks per call; else MOE_EINVAL. Enqueued on `stream`.
 */
int moe_pack_weights(int64_t num_matrices, int64_t rows, int64_t cols, const void* src, void* dst,
                     void* stream);

/*
 * The per-expert padding granule moe_forward uses for T tokens: the M-tile of the grouped
 * GEMM that fits the expected rows per local expert. Writes *block_m: 16, 32, 64, 128, 256, or
 * 0 for variable row blocks.
 *
 * Variable row blocks (block_m = 0; bf16 layers with H and 2I multiples of 256, else
 * MOE_EINVAL where a granule is passed): each local expert's segment of sorted rows is padded
 * to a multiple of 32 and cut into blocks of 256 rows, except that a last piece of at most 64
 * rows stays in the block before it, so a block has 32 to 320 rows (an expert with 1033 rows
 * takes four blocks, not four and a nearly empty fifth). block_expert then holds the block
 * table: [nb, slot_0, row_0, slot_1, row_1, ..., slot_{nb-1}, row_{nb-1}, -1, num_padded],
 * block b covering sorted rows [row_b, row_{b+1}) of slot slot_b; it needs
 * 2 * (moe_sorted_capacity / 256 + 1 + E_l) + 4 int32.
 */
int moe_pick_block_m(const moe_params* p, int64_t num_tokens, int32_t* block_m);

/*
 * Rows of the expert-sorted buffers (sorted_pairs, y) for T tokens and granule block_m:
 * T*k + E_l*(block_m-1) (T*k + E_l*31 for variable row blocks), the worst case over all
 * routings (every pair local). -1 on error.
 */
int64_t moe_sorted_capacity(const moe_params* p, int64_t num_tokens, int32_t block_m);

/*
 * Workspace bytes that moe_forward needs for T tokens (block_m = 0: the granule
 * moe_forward picks, and enough for the split entry points with variable row blocks), which is
 * also enough for any single split entry point called with the same T and block_m. Depends
 * only on host values, so no readback is ever needed.
 */
int moe_workspace_size(const moe_params* p, int64_t num_tokens, int32_t block_m, size_t* bytes);

/*
 * Contiguous expert share of rank `ep_rank` out of `ep_size`: global experts
 * [rank*E/ep, (rank+1)*E/ep) get slots 0..E/ep-1, all others -1 (per_rank = E/ep_size,
 * start = ep_rank*per_rank in _ep_init on the ep_fused_moe_patch.py page; "Expert
 * Parallel" Step 1). MOE_EINVAL if ep_size < 1, ep_size > E (the "more ranks than
 * experts" error of MixtralMoE), E % ep_size != 0 (the divisibility assert), ep_rank out
 * of range or map_host NULL. `map_host` is HOST memory of E int32.
 */
int moe_make_expert_map(int32_t num_experts, int32_t ep_size, int32_t ep_rank, int32_t* map_host);

/*
 * Expert-weight bytes per card: n_experts * (2*I*H + H*I) * dtype_bytes * layers, the
 * per-card memory arithmetic of the ep_fused_moe_patch.py docstring ("Memory layout
 * comparison"). -1 if any argument is negative.
 */
int64_t moe_weight_bytes(int64_t n_experts, int64_t hidden, int64_t inter, int32_t dtype_bytes,
                         int64_t layers);

/* ------------------------------------------------------------------ device entry points */

/*
 * Router: logits = x . Wg^T (+ logit_bias), fp32 softmax (or sigmoid), plain or grouped
 * top-k (steered by score_bias when given), renormalisation, routed scaling, expert_map
 * lookup (MixtralMoE.forward's gate / softmax / topk / renormalise; select_experts in
 * _ep_forward Step 1).
 *  x [T, H] dtype; w_gate [E, H] dtype; logit_bias [E] fp32 or NULL; score_bias [E] fp32 or
 *  NULL; expert_map [E].
 *  Outputs [T, k]: topk_ids (global ids, probability descending, ties to the lower id),
 *  topk_w (fp32), topk_local (expert_map[topk_ids], -1 = not local).
 *  ws: device scratch of at least moe_workspace_size(p, T, 0) bytes. On completion its
 *  first T*E*4 bytes hold the fp32 router logits x . Wg^T [T, E] (without logit_bias).
 */
int moe_route(const moe_params* p, int64_t num_tokens, const void* x, const void* w_gate,
              const float* logit_bias, const float* score_bias, const int32_t* expert_map,
              int32_t* topk_ids, float* topk_w, int32_t* topk_local, void* ws, size_t ws_bytes,
              void* stream);

/*
 * Groups the (token, slot) pairs by local expert, stable in pair id p = t*k + j, each
 * expert's segment padded to a multiple of block_m (the per-expert work list of the
 * expert loop in MixtralMoE.forward / the sort before fused_experts in _ep_forward).
 *  topk_local [T, k]: slot of each pair or -1 (may come from the caller's own routing;
 *    the slots of one token must be distinct, as top-k gives them).
 *  block_m: 16, 32, 64, 128, 256, or 0 for variable row blocks (see moe_pick_block_m).
 *  Outputs: sorted_pairs [moe_sorted_capacity] (pair ids; -1 in padding and in every
 *  entry past *num_padded), block_expert [capacity / block_m] (slot owning each
 *  block_m rows; the block table for block_m = 0), pair_row [T*k] (row of each pair in sorted
 *  order, -1 if not local), num_padded [1] (device int32: total padded rows).
 *  ws: device scratch, at least moe_workspace_size(p, T, block_m) bytes.
 */
int moe_align_permute(const moe_params* p, int64_t num_tokens, const int32_t* topk_local,
                      int32_t block_m, int32_t* sorted_pairs, int32_t* block_expert,
                      int32_t* pair_row, int32_t* num_padded, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Grouped expert MLP over the sorted pairs: for each row r < *num_padded with pair
 * p = sorted_pairs[r] >= 0 and slot e = block_expert[r / block_m] (block_m = 0: the slot of
 * r's block in the block table),
 *   y[r] = W2_e act(W1_e x[p / k] + b1_e, W3_e x[p / k] + b3_e) + b2_e
 * (MixtralMLP of MixtralMoE; fused_experts with w13 / w2 in _ep_forward Step 3); the biases
 * b13 / b2 are optional (NULL = none), act follows p->activation.
 * Padding rows of y hold unspecified values (they may be left unwritten). y
 * [moe_sorted_capacity, H] dtype.
 * The routing weight is NOT applied here (moe_combine applies it).
 *  ws: device scratch, at least moe_workspace_size(p, T, block_m) bytes.
 */
int moe_grouped_mlp(const moe_params* p, int64_t num_tokens, const void* x, const void* w13,
                    const void* w2, const float* b13, const float* b2,
                    const int32_t* sorted_pairs, const int32_t* block_expert,
                    const int32_t* num_padded, int32_t block_m, void* y, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * The two stages of moe_grouped_mlp, for callers that want them apart (e.g. to time or
 * overlap them). Same row rules as moe_grouped_mlp.
 *  moe_expert_gate_up: act[r] = act(W1_e x[p / k] + b1_e, W3_e x[p / k] + b3_e),
 *    act [capacity, I] dtype (the gate/up projection and activation of the expert MLP).
 *  moe_expert_down:    y[r] = W2_e act[r] + b2_e, y [capacity, H] dtype (the down projection).
 * Neither needs a workspace.
 */
int moe_expert_gate_up(const moe_params* p, int64_t num_tokens, const void* x, const void* w13,
                       const float* b13, const int32_t* sorted_pairs, const int32_t* block_expert,
                       const int32_t* num_padded, int32_t block_m, void* act, void* stream);

int moe_expert_down(const moe_params* p, int64_t num_tokens, const void* act, const void* w2,
                    const float* b2, const int32_t* block_expert, const int32_t* num_padded,
                    int32_t block_m, void* y, void* stream);

/*
 * Shared expert on every token: shared_y [T, H] = W2s (silu(W1s x) * (W3s x)) with
 * shared_w13 [2 I_s, H], shared_w2 [H, I_s] ("Expert Parallel" Step 5 shared_mlp;
 * shared experts of recursive_replace). MOE_EINVAL if p->shared_intermediate_size == 0.
 *  ws: device scratch, at least moe_workspace_size(p, T, 0) bytes.
 */
int moe_shared_mlp(const moe_params* p, int64_t num_tokens, const void* x,
                   const void* shared_w13, const void* shared_w2, void* shared_y, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Weighted combine back to token order, without atomics:
 *   out[t] = sum_{j < k, pair_row[t*k+j] >= 0} topk_w[t*k+j] * y[pair_row[t*k+j]]
 *            (+ shared_y[t] when shared_y != NULL)
 * accumulated in fp32 in slot order and rounded once to dtype (the per-token scatter-add
 * of _ep_forward Step 4; "+ shared_mlp" of "Expert Parallel" Step 5). Overwrites out.
 */
int moe_combine(const moe_params* p, int64_t num_tokens, const void* y, const int32_t* pair_row,
                const float* topk_w, const void* shared_y, void* out, void* stream);

/*
 * The whole layer on this share: moe_route -> moe_align_permute -> moe_grouped_mlp
 * (-> moe_shared_mlp) -> moe_combine, with the granule of moe_pick_block_m, all on `stream`,
 * in order: it starts after the work queued there before it, and the work queued after it
 * sees its outputs (moe_forward_overlap runs the shared expert beside the routed path on a
 * caller-owned stream). out [T, H] = this share's partial sum; summing the outputs of all
 * disjoint shares (the shared expert passed to exactly one of them) gives the full layer.
 * A share that receives no pairs writes zeros (plus the shared expert).
 *  logit_bias, score_bias: as moe_route. b13, b2: the expert biases (NULL = none).
 *  shared_w13 / shared_w2: both NULL (no shared expert on this share) or both given
 *    (then p->shared_intermediate_size > 0).
 *  topk_ids_out / topk_w_out: optional [T, k] copies of the routing (NULL = not wanted).
 *  ws: device scratch of at least moe_workspace_size(p, T, 0) bytes.
 */
int moe_forward(const moe_params* p, int64_t num_tokens, const void* x, const void* w_gate,
                const float* logit_bias, const float* score_bias, const int32_t* expert_map,
                const void* w13, const void* w2, const float* b13, const float* b2,
                const void* shared_w13, const void* shared_w2, void* out, int32_t* topk_ids_out,
                float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ replicated experts */
/*
 * Expert-parallel load balancing ("vllm.model_executor.models.transformers.moe",
 * update_physical_experts_metadata and the EPLB settings of recursive_replace): E logical
 * experts are served by P = E + num_redundant_experts physical experts, each rank holding
 * an equal contiguous share of the physical ids, and the expert map is rebuilt over physical
 * experts. The pages give no rule for splitting a logical expert's tokens among its
 * replicas; here token t's pair with logical expert e goes to replica (t mod
 * replica_count[e]) of e, so consecutive tokens spread evenly over the replicas.
 *  num_physical_experts  P, num_experts <= P <= 4096; expert_map then has P entries
 *                        (local slot of each physical expert on this share, -1 elsewhere);
 *                        p->num_local_experts counts the share's physical experts.
 *  max_replicas          row length of logical_to_physical, 1..P.
 *  logical_to_physical   device int32 [E, max_replicas]: physical ids of logical e's replicas
 *                        in entries 0 .. replica_count[e]-1.
 *  replica_count         device int32 [E], 1..max_replicas.
 * Table entries outside those ranges make the pair non-local (no out-of-range access).
 * The tables are only read; the caller owns them.
 */
typedef struct moe_eplb {
  int32_t num_physical_experts;
  int32_t max_replicas;
  const int32_t* logical_to_physical;
  const int32_t* replica_count;
} moe_eplb;

/*
 * Host helper: the replica tables of a placement. physical_to_logical (host [P]) names the
 * logical expert each physical expert holds; writes logical_to_physical (host
 * [E * max_replicas], replicas in increasing physical id, -1 after the last) and
 * replica_count (host [E]). MOE_EINVAL when an id is out of range, a logical expert has no
 * replica or more than max_replicas.
 */
int moe_eplb_tables(int32_t num_logical, int32_t num_physical, const int32_t* physical_to_logical,
                    int32_t max_replicas, int32_t* logical_to_physical, int32_t* replica_count);

/*
 * moe_route with a replicated placement: topk_ids are the logical experts the router picked
 * (as moe_route), topk_local the local slot of the replica each pair goes to. Arguments and
 * errors as moe_route; eplb as above (MOE_EINVAL when it breaks the rules above).
 */
int moe_route_eplb(const moe_params* p, const moe_eplb* eplb, int64_t num_tokens, const void* x,
                   const void* w_gate, const float* logit_bias, const float* score_bias,
                   const int32_t* expert_map, int32_t* topk_ids, float* topk_w,
                   int32_t* topk_local, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward with a replicated placement: w13 / w2 hold the share's physical experts (slot s
 * = local physical expert s, a copy of its logical expert's weights). Arguments, workspace
 * and errors as moe_forward.
 */
int moe_forward_eplb(const moe_params* p, const moe_eplb* eplb, int64_t num_tokens, const void* x,
                     const void* w_gate, const float* logit_bias, const float* score_bias,
                     const int32_t* expert_map, const void* w13, const void* w2,
                     const float* b13, const float* b2, const void* shared_w13,
                     const void* shared_w2, void* out, int32_t* topk_ids_out, float* topk_w_out,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ no-allocation forward */
/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward without a workspace argument. The
 * workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU the library runs on, held until the process ends; its device address is looked up
 * once per device, on the first call there. The call allocates nothing (no hipMalloc, no
 * allocating library routine).
 *  Arguments, results and errors as moe_forward, except: MOE_ENOSPC when
 *  moe_workspace_size(p, T, 0) exceeds MOE_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. every
 *  decode-sized call, T <= 32, of the Mixtral-, DeepSeek-V2-, DeepSeek-V3- and skewed-shaped
 *  layers, and T <= 256 on most of them); MOE_EHIP when the array's address cannot be found.
 *  Every call on one GPU shares that GPU's array and leaves its contents behind (nothing in it
 *  needs to start at zero): calls that overlap on one GPU (two streams, two threads, two
 *  graphs replayed at once) race and must be ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int moe_forward_noalloc(const moe_params* p, int64_t num_tokens, const void* x, const void* w_gate,
                        const float* logit_bias, const float* score_bias,
                        const int32_t* expert_map, const void* w13, const void* w2,
                        const float* b13, const float* b2, const void* shared_w13,
                        const void* shared_w2, void* out, int32_t* topk_ids_out, float* topk_w_out,
                        void* stream);

/* ------------------------------------------------------------------ overlapped shared expert */
/*
 * A caller-owned side stream and two caller-owned events (hipStream_t / hipEvent_t, passed as
 * void*) for moe_forward_overlap. The stream must differ from the call's `stream`; the events
 * need no timing. Calls that run at the same time need their own event pair each (a record /
 * wait pair must not interleave with another call's).
 */
typedef struct moe_side_stream {
  void* stream;
  void* fork_event;
  void* join_event;
} moe_side_stream;

/*
 * moe_forward (eplb = NULL) or moe_forward_eplb (eplb given), with the shared expert's MLP
 * beside the routed path: it reads only x and its own weights, so it can fill the compute units
 * that the router, the alignment and the last rounds of the routed GEMMs leave idle
 * ("Expert Parallel" Step 5: the shared MLP is computed on every rank beside the routed
 * experts). When a shared expert is given and its gate/up projection is at most four rounds of
 * 256x256 tiles, fork_event is recorded on `stream`, side->stream waits for it and runs the
 * shared MLP, join_event is recorded there, and `stream` waits for join_event before the
 * combine. The join is enqueued on every path that enqueued the fork, error returns included,
 * so the pattern can be captured into a HIP graph. Otherwise (no shared expert, or a long one
 * that fills the GPU by itself) the call is exactly moe_forward and side is not touched.
 * side = NULL is also moe_forward. MOE_EINVAL if side->fork_event or side->join_event is NULL
 * or side->stream equals `stream`. Arguments, workspace and errors otherwise as moe_forward.
 */
int moe_forward_overlap(const moe_params* p, const moe_eplb* eplb, const moe_side_stream* side,
                        int64_t num_tokens, const void* x, const void* w_gate,
                        const float* logit_bias, const float* score_bias,
                        const int32_t* expert_map, const void* w13, const void* w2,
                        const float* b13, const float* b2, const void* shared_w13,
                        const void* shared_w2, void* out, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ expert-parallel exchange */
/*
 * The steps on either side of the path when tokens travel to the ranks that own their experts
 * ("ep_fused_moe_patch.py", _ep_forward Step 2 dispatch and Step 4 combine). Ranks own
 * contiguous shares of E / ep_size experts (as moe_make_expert_map). A token travels to each
 * of its destination ranks once: its first slot j whose expert lives on rank r owns the row,
 * and the row carries all k slots, so the receiving rank applies every one of its experts
 * that the token picked. On one GPU these are layout transforms; between GPUs each rank's
 * part of the send buffers is the segment of an all-to-all.
 *  ep_size: 1..256, dividing p->num_experts; MOE_EINVAL otherwise.
 */

/* Send rows for T tokens: T * min(k, ep_size) (every token to min(k, ep_size) ranks); -1 on
 * invalid arguments. */
int64_t moe_ep_send_capacity(const moe_params* p, int64_t num_tokens, int32_t ep_size);

/* Workspace bytes that moe_ep_dispatch needs for T tokens. */
int moe_ep_workspace_size(const moe_params* p, int64_t num_tokens, int32_t ep_size,
                          size_t* bytes);

/*
 * Dispatch plan and send buffers (Step 2). Rows are grouped by destination rank, rank 0 first,
 * and follow increasing token index inside a rank; no sort, no host synchronisation. Inputs:
 * topk_ids / topk_w [T, k] (global expert ids in [0, E); ids outside are not sent) and
 * x [T, H] (p->dtype). Outputs, device memory, capacity R = moe_ep_send_capacity rows:
 *  send_pos   [T*k]  the row of pair (t, j) when it owns one, else -1;
 *  rank_meta  [2*ep_size + 2]  n_send, then the ranks' row offsets (ep_size + 1), then their
 *             row counts (ep_size): rank r's rows are [offsets[r], offsets[r+1]);
 *  send_token [R]    the token of each row;
 *  send_x     [R, H] the token's hidden row (16-byte aligned, as x);
 *  send_local [R, k] the token's k slots seen from the row's rank: local expert index there,
 *             or -1 for experts of other ranks (moe_align_permute's topk_local on that rank);
 *  send_w     [R, k] the token's k routing weights.
 * Rows past n_send are not written.
 *  ws: at least moe_ep_workspace_size bytes.
 */
int moe_ep_dispatch(const moe_params* p, int64_t num_tokens, int32_t ep_size,
                    const int32_t* topk_ids, const float* topk_w, const void* x,
                    int32_t* send_pos, int32_t* rank_meta, int32_t* send_token, void* send_x,
                    int32_t* send_local, float* send_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Combine side (Step 4): recv_y [n_send, H] holds, row by row in the order of the dispatch,
 * the result that row's rank computed for its token (that rank's share of the layer: the
 * weighted sum over its experts, as moe_combine writes it). Then
 *   out[t] = sum_{j < k, send_pos[t*k+j] >= 0} recv_y[send_pos[t*k+j]]
 * accumulated in fp32 in slot order and rounded once to dtype (the per-token scatter-add).
 * Overwrites out [T, H].
 */
int moe_ep_combine(const moe_params* p, int64_t num_tokens, const int32_t* send_pos,
                   const void* recv_y, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EXPERT_MOE_AMD_MOE_H */
