// Router of the fused MoE forward on gfx950: logits GEMM launch and the per-token fp32
// softmax / top-k epilogue, one wavefront per token.
//
// Steps ("[Feature] Expert parallelism support", MixtralMoE.forward; "ep_fused_moe_patch.py",
// _ep_forward Step 1 select_experts; "vllm.model_executor.models.transformers.moe",
// recursive_replace routed_scaling_factor / n_group / topk_group):
//   p = softmax(logits + bias) in fp32 over all E global experts
//   grouped: group score = largest p of each contiguous group of E/G experts; keep the
//            topk_group best groups; experts of other groups are excluded
//   ids = k best candidates, probability descending, ties to the lower id
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
  const float* bias;
  const int32_t* emap;
  int32_t* ids;
  float* w;
  int32_t* local;
  int T, E, k, renorm, grouped, G, keep, E_l;
  float rsf;
};

// (v1, i1) ranks before (v2, i2): larger value, then lower index.
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m, 64);
    const int oi = __shfl_xor(i, m, 64);
    if (ranks_before(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// 4 tokens per workgroup (one per wave); E <= 256 so a lane holds experts lane + 64 q.
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  __shared__ float sp[4][256];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < a.T;
  const int E = a.E;

  float pv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    float l = -INFINITY;
    if (valid && e < E) {
      float* lp = a.logits + static_cast<int64_t>(t) * E + e;
      l = lp[0];
      const int64_t stride = static_cast<int64_t>(a.T) * E;
      for (int sp = 1; sp < a.splits; ++sp) l += lp[sp * stride];
      if (a.splits > 1) lp[0] = l;
      if (a.bias) l += a.bias[e];
    }
    pv[q] = l;
  }
  const float m = wave_max(fmaxf(fmaxf(pv[0], pv[1]), fmaxf(pv[2], pv[3])));
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pv[q] = (lane + 64 * q < E) ? expf(pv[q] - m) : 0.f;
    part += pv[q];
  }
  const float ssum = wave_sum(part);
#pragma unroll
  for (int q = 0; q < 4; ++q) pv[q] = pv[q] / ssum;

  // Candidate scores: p for candidates, -inf for excluded / absent experts.
  float cv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cv[q] = (lane + 64 * q < E) ? pv[q] : -INFINITY;

  if (a.grouped) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q < E) sp[wave][lane + 64 * q] = pv[q];
    __syncthreads();
    const int gsz = E / a.G;
    float gs = -INFINITY;
    if (lane < a.G)
      for (int i = 0; i < gsz; ++i) gs = fmaxf(gs, sp[wave][lane * gsz + i]);
    uint64_t kept = 0;
    for (int r = 0; r < a.keep; ++r) {
      float bv = gs;
      int bi = lane;
      wave_argmax(bv, bi);
      kept |= 1ull << bi;
      if (lane == bi) gs = -INFINITY;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((kept >> (e / gsz)) & 1ull)) cv[q] = -INFINITY;
    }
  }
  if (!valid) return;

  int my_id = 0;
  float my_w = 0.f;
  float wsum = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bv = cv[0];
    int bi = lane;
#pragma unroll
    for (int q = 1; q < 4; ++q)
      if (ranks_before(cv[q], lane + 64 * q, bv, bi)) { bv = cv[q]; bi = lane + 64 * q; }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) cv[bi >> 6] = -INFINITY;
    if (lane == j) { my_id = bi; my_w = bv; }
    wsum = j == 0 ? bv : wsum + bv;
  }
  if (lane < a.k) {
    float w = my_w;
    if (a.renorm) w = w / wsum;
    w = w * a.rsf;
    const int64_t o = static_cast<int64_t>(t) * a.k + lane;
    a.ids[o] = my_id;
    a.w[o] = w;
    int s = a.emap[my_id];
    a.local[o] = (s >= 0 && s < a.E_l) ? s : -1;
  }
}

}  // namespace

int router_splits(const moe_params& p, int T) {
  if (p.dtype == MOE_F32) return 1;
  const int rows = T <= 64 ? 16 : 128;
  const int bnr = 64;
  const int blocks = ((T + rows - 1) / rows) * ((p.num_experts + bnr - 1) / bnr);
  int sp = 1;
  while (sp < 16 && blocks * sp < 512 && p.hidden_size % (256 * 2 * sp) == 0) sp *= 2;
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
    gemm_f32_tile<kStoreF32><<<a.m_blocks * n_tiles, 256, 0, s>>>(a);
  } else if (T <= 64) {
    a.m_blocks = ceil_div(T, 16);
    a.n_tiles = n_tiles;
    gemm_bf16_stream<4, kStoreF32><<<dim3(tile_grid(a.m_blocks, n_tiles), a.k_splits), 256, 0, s>>>(a);
  } else {
    a.m_blocks = ceil_div(T, 128);
    a.n_tiles = n_tiles;
    const dim3 grid(tile_grid(a.m_blocks, n_tiles), a.k_splits);
    if (bnr == 256)
      gemm_bf16_dma<128, 256, 2, 2, kStoreF32><<<grid, 256, 0, s>>>(a);
    else if (bnr == 128)
      gemm_bf16_dma<128, 128, 2, 2, kStoreF32><<<grid, 256, 0, s>>>(a);
    else
      gemm_bf16_dma<128, 64, 4, 1, kStoreF32><<<grid, 256, 0, s>>>(a);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_topk(const moe_params& p, int T, float* logits, const float* bias,
                const int32_t* expert_map, int32_t* ids, float* w, int32_t* local, hipStream_t s) {
  TopkArgs a;
  a.logits = logits;
  a.splits = router_splits(p, T);
  a.bias = bias;
  a.emap = expert_map;
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
  topk_kernel<<<ceil_div(T, 4), 256, 0, s>>>(a);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
