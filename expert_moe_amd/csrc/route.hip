// Router of the fused MoE forward on gfx950: logits GEMM launch and the per-token fp32
// scores / top-k epilogue, one wavefront per token.
//
// Steps ("[Feature] Expert parallelism support", MixtralMoE.forward; "ep_fused_moe_patch.py",
// _ep_forward Step 1 select_experts; "vllm.model_executor.models.transformers.moe",
// recursive_replace routed_scaling_factor / n_group / topk_group):
//   p = softmax(logits + bias) in fp32 over all E global experts, or with the sigmoid scoring
//       function 1 / (1 + exp(-(logits + bias))) per expert (scoring_func, named on the
//       transformers MoE page; the logistic form is DeepSeek-V3's)
//   s = p + score_bias (the selection-only e_score_correction_bias, DeepSeek-V3's use), or p
//   grouped: group score = largest s of each contiguous group of E/G experts, or with a
//            score bias the sum of its two largest s; keep the topk_group best groups;
//            experts of other groups are excluded
//   ids = k best candidates by s, descending, ties to the lower id
//   w = p[ids], / sum_j w (slot order) if renormalize, * routed_scaling_factor
//   local = expert_map[ids] (-1 if not on this share)
#include <math.h>

#include "gemm.h"
#include "launch.h"

namespace moe {

namespace {

struct TopkArgs {
  float* logits;  // [splits, T, E] partial sums; their total is written back to split 0
  int splits;
  const float* bias;   // added to the logits
  const float* sbias;  // added to the scores for the choice only, or NULL
  int sigmoid;         // 1: logistic scores, 0: softmax
  const int32_t* emap;
  const int32_t* l2p;  // replicated experts: [E, max_rep] physical ids, or NULL
  const int32_t* cnt;  // [E] replica counts
  int max_rep, P;
  int32_t* ids;
  float* w;
  int32_t* local;
  int T, E, k, renorm, grouped, G, keep, E_l;
  float rsf;
};

// Wave-wide reductions as a butterfly of in-register lane exchanges (no LDS crossbar):
// DPP quad_perm for lane distances 1 and 2, row_half_mirror and row_mirror to join groups of
// 4 and 8 lanes inside a 16-lane row, then gfx950 v_permlane16_swap / v_permlane32_swap to join
// rows (each lane ends with the result). The lane layouts of all six were checked with an
// in-bounds probe on the box.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int kXor1 = 0xB1;        // quad_perm(1, 0, 3, 2)
constexpr int kXor2 = 0x4E;        // quad_perm(2, 3, 0, 1)
constexpr int kHalfMirror = 0x141; // row_half_mirror
constexpr int kMirror = 0x140;     // row_mirror

// (a, b) = both values of a pair of lanes 16 (S = 16) or 32 (S = 32) apart.
template <int S>
__device__ __forceinline__ void swap_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  }
}

// Op is a commutative, associative combine on the raw 32-bit lanes.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, dpp_partner<kXor1>(v));
  v = op(v, dpp_partner<kXor2>(v));
  v = op(v, dpp_partner<kHalfMirror>(v));
  v = op(v, dpp_partner<kMirror>(v));
  uint32_t x, y;
  swap_pair<16>(v, x, y);
  v = op(x, y);
  swap_pair<32>(v, x, y);
  return op(x, y);
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
}

__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  }));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

// Selection key of a score of either sign: the bit pattern with the sign bit set for
// non-negative values and all bits flipped for negative ones is ordered like the value, and
// no finite score maps to 0, which marks an expert that may not be chosen (excluded group, or
// past E).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scores, selection and outputs of token t, whose logits plus logit bias lane l holds in
// pv[q] (expert l + 64 q; -inf past E or for an invalid token) and its selection biases in
// sb[q]; sp: this wave's LDS row of 64 NQ floats (grouped routing only). Every lane of the
// wave calls it; lanes < k write the token's outputs.
template <int NQ>
__device__ __forceinline__ void select_token(const TopkArgs& a, int t, bool valid, float (&pv)[NQ],
                                             const float (&sb)[NQ], float* sp, int lane) {
  const int E = a.E;
  if (a.sigmoid) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) pv[q] = (lane + 64 * q < E) ? 1.f / (1.f + expf(-pv[q])) : 0.f;
  } else {
    float lmax = pv[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) lmax = fmaxf(lmax, pv[q]);
    const float m = wave_max(lmax);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      pv[q] = (lane + 64 * q < E) ? expf(pv[q] - m) : 0.f;
      part += pv[q];
    }
    const float ssum = wave_sum(part);
#pragma unroll
    for (int q = 0; q < NQ; ++q) pv[q] = pv[q] / ssum;
  }

  // selection scores: p, plus the selection bias when there is one
  float sv[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) sv[q] = pv[q] + sb[q];
  uint32_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) key[q] = (lane + 64 * q < E) ? order_key(sv[q]) : 0u;

  if (a.grouped) {
    // group score over the group's E/G contiguous experts: the largest score, or with a
    // selection bias the sum of the two largest biased scores (the larger first); the
    // topk_group best groups (ties to the lower group) stay candidates
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (lane + 64 * q < E) sp[lane + 64 * q] = sv[q];
    // the wave reads back only its own row: its LDS accesses are processed in order
    __builtin_amdgcn_wave_barrier();
    const int gsz = E / a.G;
    float gs = -INFINITY;
    if (lane < a.G) {
      if (a.sbias == nullptr) {
        for (int i = 0; i < gsz; ++i) gs = fmaxf(gs, sp[lane * gsz + i]);
      } else {
        float t1 = -INFINITY, t2 = -INFINITY;
        for (int i = 0; i < gsz; ++i) {
          const float v = sp[lane * gsz + i];
          if (v > t1) {
            t2 = t1;
            t1 = v;
          } else if (v > t2) {
            t2 = v;
          }
        }
        gs = gsz > 1 ? t1 + t2 : t1;
      }
    }
    uint32_t gk = lane < a.G ? order_key(gs) : 0u;
    uint64_t kept = 0;
    for (int r = 0; r < a.keep; ++r) {
      const uint32_t best = wave_max_u32(gk);
      const int g = __builtin_ctzll(__ballot(gk == best));
      kept |= 1ull << g;
      if (lane == g) gk = 0u;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((kept >> (e / gsz)) & 1ull)) key[q] = 0u;
    }
  }
  if (!valid) return;

  // k rounds: the largest key left, at its lowest expert id (lowest q, then lowest lane)
  int my_id = 0;
  float my_w = 0.f;
  float wsum = 0.f;
  for (int j = 0; j < a.k; ++j) {
    uint32_t lk = key[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) lk = key[q] > lk ? key[q] : lk;
    const uint32_t best = wave_max_u32(lk);
    int id = 0;
#pragma unroll
    for (int q = NQ - 1; q >= 0; --q) {
      const uint64_t hit = __ballot(key[q] == best);
      if (hit) id = 64 * q + __builtin_ctzll(hit);
    }
    if ((id & 63) == lane) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if ((id >> 6) == q) key[q] = 0u;
    }
    // the chosen expert's own score p (the weight never includes the selection bias)
    float pc = pv[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q)
      if ((id >> 6) == q) pc = pv[q];
    const float bv = __shfl(pc, id & 63);
    if (lane == j) { my_id = id; my_w = bv; }
    wsum = j == 0 ? bv : wsum + bv;
  }
  if (lane < a.k) {
    float w = my_w;
    if (a.renorm) w = w / wsum;
    w = w * a.rsf;
    const int64_t o = static_cast<int64_t>(t) * a.k + lane;
    a.ids[o] = my_id;
    a.w[o] = w;
    int s = -1;
    if (a.l2p == nullptr) {
      s = a.emap[my_id];
    } else {
      // replica t mod cnt of the logical expert (entries outside the tables' ranges: not local)
      const int c = a.cnt[my_id];
      if (c >= 1 && c <= a.max_rep) {
        const int q = a.l2p[static_cast<int64_t>(my_id) * a.max_rep + t % c];
        if (q >= 0 && q < a.P) s = a.emap[q];
      }
    }
    a.local[o] = (s >= 0 && s < a.E_l) ? s : -1;
  }
}

// 4 tokens per workgroup (one per wave); lane l holds experts l + 64 q for q < NQ, E <= 64 NQ.
template <int NQ>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  __shared__ float sp[4][64 * NQ];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < a.T;
  const int E = a.E;

  // Every load of the token goes out before the first use (addresses clamped into the
  // arrays, values masked afterwards): the logits, the K-split partial sums four splits at a
  // time, and the biases. Loads behind per-value guards each waited for the one before.
  const int tc = valid ? t : a.T - 1;
  float* row = a.logits + static_cast<int64_t>(tc) * E;
  const int64_t stride = static_cast<int64_t>(a.T) * E;
  int ec[NQ];
  float pv[NQ], lb[NQ], sb[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    ec[q] = min(lane + 64 * q, E - 1);
    pv[q] = row[ec[q]];
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    lb[q] = a.bias ? a.bias[ec[q]] : 0.f;
    sb[q] = a.sbias ? a.sbias[ec[q]] : 0.f;
  }
  for (int s0 = 1; s0 < a.splits; s0 += 4) {
    float v[4][NQ];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t off = static_cast<int64_t>(min(s0 + j, a.splits - 1)) * stride;
#pragma unroll
      for (int q = 0; q < NQ; ++q) v[j][q] = row[off + ec[q]];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < a.splits) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) pv[q] += v[j][q];
      }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const bool ok = valid && lane + 64 * q < E;
    if (ok && a.splits > 1) row[ec[q]] = pv[q];
    pv[q] = ok ? pv[q] + lb[q] : -INFINITY;
  }
  select_token<NQ>(a, t, valid, pv, sb, sp[wave], lane);
}

}  // namespace

int router_splits(const moe_params& p, int T) {
  if (p.dtype == MOE_F32) return 1;
  const int rows = T <= 64 ? 16 : 64;
  const int bnr = 64;
  const int blocks = ((T + rows - 1) / rows) * ((p.num_experts + bnr - 1) / bnr);
  int sp = 1;
  while (sp < 16 && blocks * sp < 256 && p.hidden_size % (256 * 2 * sp) == 0) sp *= 2;
  if (sp == 1 && blocks < 256) {
    // hidden sizes with no power-of-two split (e.g. 2880 = 45 x 64): the largest split of at
    // most 16 that divides H into whole K steps of the logits kernel, at least four each, and
    // stays under about two workgroups per CU
    const int units = p.hidden_size / (T <= 64 ? 32 : 64);
    for (int d = 16; d > 1; --d)
      if (units % d == 0 && units / d >= 4 && blocks * d < 512) {
        sp = d;
        break;
      }
  }
  return sp;
}

int launch_router_logits(const moe_params& p, int T, const void* x, const void* w_gate,
                         float* logits, hipStream_t s) {
  GemmArgs a{};
  a.A = x;
  a.row_map = nullptr;
  a.row_div = 1;
  a.M_pairs = 0;
  a.M_rows = T;
  a.num_padded = nullptr;
  a.block_expert = nullptr;
  a.block_m = 1;
  a.B = w_gate;
  a.b_stride = 0;
  a.K = p.hidden_size;
  a.N = p.num_experts;
  a.N_valid = p.num_experts;
  a.C = logits;
  a.ldc = p.num_experts;
  const int bnr = 64;
  const int n_tiles = ceil_div(p.num_experts, bnr);
  a.k_splits = router_splits(p, T);
  a.c_split_stride = static_cast<int64_t>(T) * p.num_experts;
  if (p.dtype == MOE_F32) {
    a.m_blocks = ceil_div(T, 16);
    return launch(gemm_f32_tile<kStoreF32>, a.m_blocks * n_tiles, 256, 0, s, a);
  } else if (T <= 64) {
    a.m_blocks = ceil_div(T, 16);
    a.n_tiles = n_tiles;
    return launch(gemm_bf16_stream<4, kStoreF32>, dim3(tile_grid(a.m_blocks, n_tiles), a.k_splits),
                  256, 0, s, a);
  } else {
    a.m_blocks = ceil_div(T, 64);
    a.n_tiles = n_tiles;
    const dim3 grid(tile_grid(a.m_blocks, n_tiles), a.k_splits);
    // 64x64 tiles, three LDS stages: the loads run two K steps ahead, which this short-K,
    // latency-bound launch needs (measured: EP share 42 -> 35 us, with splits for about one
    // workgroup per CU); 64-row tiles give twice the workgroups of 128-row ones for the same
    // LDS per CU (route stage: DeepSeek-V2-shaped 39.2 -> 36.9 us, skewed T=16384 58 -> 54.5 us)
    return launch(gemm_bf16_dma<64, 64, 2, 2, kStoreF32, 3>, grid, 256, 0, s, a);
  }
}

namespace {

TopkArgs topk_args(const moe_params& p, int T, float* logits, int splits, const float* bias,
                   const float* score_bias, const int32_t* expert_map, int32_t* ids, float* w,
                   int32_t* local, const EplbMap* eplb) {
  TopkArgs a;
  a.logits = logits;
  a.splits = splits;
  a.bias = bias;
  a.sbias = score_bias;
  a.sigmoid = p.scoring_func == MOE_SCORE_SIGMOID;
  a.emap = expert_map;
  a.l2p = eplb ? eplb->l2p : nullptr;
  a.cnt = eplb ? eplb->cnt : nullptr;
  a.max_rep = eplb ? eplb->max_rep : 0;
  a.P = eplb ? eplb->P : 0;
  a.ids = ids;
  a.w = w;
  a.local = local;
  a.T = T;
  a.E = p.num_experts;
  a.k = p.top_k;
  a.renorm = p.renormalize;
  a.grouped = p.use_grouped_topk;
  a.G = p.use_grouped_topk ? p.num_expert_group : 1;
  a.keep = p.use_grouped_topk ? p.topk_group : 1;
  a.E_l = p.num_local_experts;
  a.rsf = p.routed_scaling_factor;
  return a;
}

}  // namespace

int launch_topk(const moe_params& p, int T, float* logits, const float* bias,
                const float* score_bias, const int32_t* expert_map, int32_t* ids, float* w,
                int32_t* local, hipStream_t s, const EplbMap* eplb) {
  const TopkArgs a = topk_args(p, T, logits, router_splits(p, T), bias, score_bias, expert_map, ids,
                               w, local, eplb);
  const int blocks = ceil_div(T, 4);
  if (a.E <= 64) return launch(topk_kernel<1>, blocks, 256, 0, s, a);
  if (a.E <= 128) return launch(topk_kernel<2>, blocks, 256, 0, s, a);
  return launch(topk_kernel<4>, blocks, 256, 0, s, a);
}

int launch_route(const moe_params& p, int T, const void* x, const void* w_gate, float* logits,
                 const float* bias, const float* score_bias, const int32_t* expert_map,
                 int32_t* ids, float* w, int32_t* local, hipStream_t s, const EplbMap* eplb) {
  if (int rc = launch_router_logits(p, T, x, w_gate, logits, s)) return rc;
  return launch_topk(p, T, logits, bias, score_bias, expert_map, ids, w, local, s, eplb);
}

}  // namespace moe
