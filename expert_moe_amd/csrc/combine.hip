// Routing-weighted combine back to token order (gfx950), without atomics.
//
// out[t] = sum_{j < k, pair_row[t*k+j] >= 0} w[t*k+j] * y[pair_row[t*k+j]] (+ shared_y[t])
// (w = NULL: weight 1, the unpack of the expert-parallel exchange)
//
// The per-token sum of the weighted expert rows ("ep_fused_moe_patch.py", _ep_forward
// Step 4, scatter-add by token; the weighted accumulation of MixtralMoE.forward) plus the
// shared expert ("Expert Parallel", Step 5). Each token is gathered by one workgroup, so no
// two workgroups write the same output and no atomics are needed; the sum is fp32 in slot
// order, rounded once to the output type. The token's local slots are compacted first, so
// the loads of up to 8 rows are in flight together.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// The token's local slots, compacted in slot order into LDS (k <= 64: one wave's ballot), so
// that the row loads of several slots can be in flight together. Returns their number.
__device__ __forceinline__ int local_slots(const int32_t* __restrict__ pair_row,
                                           const float* __restrict__ w, int64_t pbase, int k,
                                           int* s_r, float* s_w, int* s_n) {
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const int r = j < k ? pair_row[pbase + j] : -1;
    const float wt = j < k ? (w ? w[pbase + j] : 1.f) : 0.f;  // no weights: each row counts once
    const unsigned long long m = __ballot(r >= 0);
    if (r >= 0) {
      const int pos = __popcll(m & ((1ull << j) - 1ull));
      s_r[pos] = r;
      s_w[pos] = wt;
    }
    if (j == 0) *s_n = __popcll(m);
  }
  __syncthreads();
  return *s_n;
}

__global__ void __launch_bounds__(256) combine_bf16(const uint16_t* __restrict__ y,
                                                    const int32_t* __restrict__ pair_row,
                                                    const float* __restrict__ w,
                                                    const uint16_t* __restrict__ shared_y,
                                                    uint16_t* __restrict__ out, int k, int H) {
  __shared__ int s_r[64];
  __shared__ float s_w[64];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int n = local_slots(pair_row, w, static_cast<int64_t>(t) * k, k, s_r, s_w, &s_n);
  for (int v = threadIdx.x; v < H / 8; v += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += 8) {
      uint4 q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < n) q[j] = load16(y + static_cast<int64_t>(s_r[j0 + j]) * H + v * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= n) break;
        const float wt = s_w[j0 + j];
        const uint32_t u[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wt * bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
          acc[2 * i + 1] += wt * bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
        }
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
  __shared__ int s_r[64];
  __shared__ float s_w[64];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int n = local_slots(pair_row, w, static_cast<int64_t>(t) * k, k, s_r, s_w, &s_n);
  for (int v = threadIdx.x; v < H / 4; v += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n; ++j) {
      const float wt = s_w[j];
      const float4 q = *reinterpret_cast<const float4*>(y + static_cast<int64_t>(s_r[j]) * H + v * 4);
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
    return launch(combine_f32, T, 256, 0, s, static_cast<const float*>(y), pair_row, topk_w,
                  static_cast<const float*>(shared_y), static_cast<float*>(out), p.top_k,
                  p.hidden_size);
  return launch(combine_bf16, T, 256, 0, s, static_cast<const uint16_t*>(y), pair_row, topk_w,
                static_cast<const uint16_t*>(shared_y), static_cast<uint16_t*>(out), p.top_k,
                p.hidden_size);
}

}  // namespace moe
