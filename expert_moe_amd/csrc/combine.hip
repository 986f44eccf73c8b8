// Routing-weighted combine back to token order (gfx950), without atomics.
//
// out[t] = sum_{j < k, pair_row[t*k+j] >= 0} w[t*k+j] * y[pair_row[t*k+j]] (+ shared_y[t])
//
// The per-token sum of the weighted expert rows ("ep_fused_moe_patch.py", _ep_forward
// Step 4, scatter-add by token; the weighted accumulation of MixtralMoE.forward) plus the
// shared expert ("Expert Parallel", Step 5). Each token is gathered by one workgroup, so no
// two workgroups write the same output and no atomics are needed; the sum is fp32 in slot
// order, rounded once to the output type.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

__global__ void __launch_bounds__(256) combine_bf16(const uint16_t* __restrict__ y,
                                                    const int32_t* __restrict__ pair_row,
                                                    const float* __restrict__ w,
                                                    const uint16_t* __restrict__ shared_y,
                                                    uint16_t* __restrict__ out, int k, int H) {
  const int t = blockIdx.x;
  const int64_t pbase = static_cast<int64_t>(t) * k;
  for (int v = threadIdx.x; v < H / 8; v += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = pair_row[pbase + j];
      if (r < 0) continue;
      const float wt = w[pbase + j];
      const uint4 q = load16(y + static_cast<int64_t>(r) * H + v * 8);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wt * bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
        acc[2 * i + 1] += wt * bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
      }
    }
    if (shared_y) {
      const uint4 q = load16(shared_y + static_cast<int64_t>(t) * H + v * 8);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
        acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * H + v * 8) = o;
  }
}

__global__ void __launch_bounds__(256) combine_f32(const float* __restrict__ y,
                                                   const int32_t* __restrict__ pair_row,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ shared_y,
                                                   float* __restrict__ out, int k, int H) {
  const int t = blockIdx.x;
  const int64_t pbase = static_cast<int64_t>(t) * k;
  for (int v = threadIdx.x; v < H / 4; v += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = pair_row[pbase + j];
      if (r < 0) continue;
      const float wt = w[pbase + j];
      const float4 q = *reinterpret_cast<const float4*>(y + static_cast<int64_t>(r) * H + v * 4);
      acc.x += wt * q.x;
      acc.y += wt * q.y;
      acc.z += wt * q.z;
      acc.w += wt * q.w;
    }
    if (shared_y) {
      const float4 q = *reinterpret_cast<const float4*>(shared_y + static_cast<int64_t>(t) * H + v * 4);
      acc.x += q.x;
      acc.y += q.y;
      acc.z += q.z;
      acc.w += q.w;
    }
    *reinterpret_cast<float4*>(out + static_cast<int64_t>(t) * H + v * 4) = acc;
  }
}

}  // namespace

int launch_combine(const moe_params& p, int T, const void* y, const int32_t* pair_row,
                   const float* topk_w, const void* shared_y, void* out, hipStream_t s) {
  if (p.dtype == MOE_F32)
    combine_f32<<<T, 256, 0, s>>>(static_cast<const float*>(y), pair_row, topk_w,
                                  static_cast<const float*>(shared_y), static_cast<float*>(out),
                                  p.top_k, p.hidden_size);
  else
    combine_bf16<<<T, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_row, topk_w,
                                   static_cast<const uint16_t*>(shared_y),
                                   static_cast<uint16_t*>(out), p.top_k, p.hidden_size);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
