// Grouped "NT" GEMM kernels of the expert MLP (gfx950).
//
//   C[r, n] = sum_k A[src(r), k] * B_slot(r)[n, k]
//
// A rows are token activations, gathered through the expert-sorted pair list
// (src(r) = sorted_pairs[r] / top_k, padding rows read token 0) or taken in order
// (identity, for the shared expert and the router). B is a weight matrix stored with the
// reduction dimension contiguous ([rows, K]), selected per block of rows by block_expert.
// Epilogues: fused silu(gate) * up for the w13 projection (gate rows [0, N), up rows
// [N, 2N) of B), plain bf16 store for the w2 projection, bounded fp32 store for router
// logits.
#pragma once

#include "common.h"

namespace moe {

enum GemmMode { kSiluMul = 0, kStore = 1, kStoreF32 = 2 };

struct GemmArgs {
  const void* A;               // activations, [*, K] row-major
  const int32_t* row_map;      // sorted pair ids (-1 = padding) or NULL for identity rows
  int32_t row_div;             // pair id -> token row (top_k)
  int32_t M_pairs;             // row_map entries outside [0, M_pairs) read token 0
  int32_t M_rows;              // rows of the output buffer (stores past it are dropped);
                               // identity rows past it read the last row
  const int32_t* num_padded;   // device count of rows in use, or NULL (= M_rows)
  const int32_t* block_expert; // sorted rows: slot of each block of block_m rows (NULL = slot 0)
  int32_t block_m;             // padding granule of the sorted rows (a multiple of the tile rows)
  const void* B;               // weights of slot s at B + s * b_stride elements, [rows, K]
  int64_t b_stride;
  int32_t K;
  int32_t N;                   // kSiluMul: output columns (I); else output columns
  int32_t N_valid;             // kStoreF32: valid output columns (B rows past it are clamped)
  void* C;                     // output, row stride ldc elements
  int64_t ldc;
  int32_t m_blocks;            // grid extent along rows
};

__device__ __forceinline__ int gemm_src_row(const GemmArgs& a, int r) {
  if (a.row_map) {
    const int p = a.row_map[r];
    return (p < 0 || p >= a.M_pairs) ? 0 : p / a.row_div;
  }
  return r < a.M_rows ? r : a.M_rows - 1;
}

__device__ __forceinline__ int gemm_rows_active(const GemmArgs& a) {
  return a.num_padded ? *a.num_padded : a.M_rows;
}

// ----------------------------------------------------------------------------------------
// Large-M tile: BM x BNR (B rows) per workgroup of 4 waves (WM x WN), K step 64, two LDS
// stages, v_mfma_f32_32x32x16_bf16. In kSiluMul the BNR rows are BNR/2 gate rows followed
// by the BNR/2 matching up rows, so each lane holds gate and up of the same output.
// ----------------------------------------------------------------------------------------
template <int BM, int BNR, int WM, int WN, int MODE>
__global__ void __launch_bounds__(256) gemm_bf16_tile(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;  // +16 bytes per LDS row: conflict-free 16-byte fragment reads
  constexpr int TM = BM / WM;
  constexpr int TMB = TM / 32;
  constexpr int TNR = BNR / WN;
  constexpr int TNB = TNR / 32;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TMB >= 1 && TNB >= 1, "wave tile at least 32x32");
  static_assert(MODE != kSiluMul || (TNB % 2 == 0), "gate/up pairs");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BNR][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mb = blockIdx.x % a.m_blocks;
  const int nt = blockIdx.x / a.m_blocks;
  const int m0 = mb * BM;
  if (m0 >= gemm_rows_active(a)) return;
  const int slot = a.block_expert ? a.block_expert[m0 / a.block_m] : 0;
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(a.B) + slot * a.b_stride;
  const int K = a.K;

  // Global -> register assignment: 8 threads per 64-element row slice, 32 rows per pass.
  const int lc = tid & 7;
  const int lr = tid >> 3;
  const uint16_t* pa[BM / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
    pa[i] = A + static_cast<int64_t>(gemm_src_row(a, m0 + lr + 32 * i)) * K + lc * 8;
  const uint16_t* pb[BNR / 32];
#pragma unroll
  for (int i = 0; i < BNR / 32; ++i) {
    const int r = lr + 32 * i;
    int brow;
    if (MODE == kSiluMul)
      brow = r < BNR / 2 ? nt * (BNR / 2) + r : a.N + nt * (BNR / 2) + (r - BNR / 2);
    else {
      brow = nt * BNR + r;
      if (MODE == kStoreF32 && brow >= a.N_valid) brow = a.N_valid - 1;
    }
    pb[i] = B + static_cast<int64_t>(brow) * K + lc * 8;
  }

  uint4 ra[BM / 32], rb[BNR / 32];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) ra[i] = load16(pa[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < BNR / 32; ++i) rb[i] = load16(pb[i] + kt * BK);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) *reinterpret_cast<uint4*>(&sA[buf][lr + 32 * i][lc * 8]) = ra[i];
#pragma unroll
    for (int i = 0; i < BNR / 32; ++i) *reinterpret_cast<uint4*>(&sB[buf][lr + 32 * i][lc * 8]) = rb[i];
  };

  const int wm = wave % WM;
  const int wn = wave / WM;
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  int brow0[TNB];
#pragma unroll
  for (int j = 0; j < TNB; ++j) {
    if (MODE == kSiluMul)
      brow0[j] = j < TNB / 2 ? wn * (TNR / 2) + j * 32 : BNR / 2 + wn * (TNR / 2) + (j - TNB / 2) * 32;
    else
      brow0[j] = wn * TNR + j * 32;
  }

  f32x16 acc[TMB][TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fa[TMB], fb[TNB];
#pragma unroll
      for (int i = 0; i < TMB; ++i)
        fa[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&sA[cur][wm * TM + i * 32 + fr][kk + fk]));
#pragma unroll
      for (int j = 0; j < TNB; ++j)
        fb[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&sB[cur][brow0[j] + fr][kk + fk]));
#pragma unroll
      for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int j = 0; j < TNB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue. acc[i][j][r] sits at tile row wm*TM + i*32 + 8*(r/4) + 4*(lane/32) + r%4 and
  // tile B row brow0[j] + lane%32.
#pragma unroll
  for (int i = 0; i < TMB; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= a.M_rows) continue;
      if (MODE == kSiluMul) {
        uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
#pragma unroll
        for (int j = 0; j < TNB / 2; ++j) {
          const int col = nt * (BNR / 2) + wn * (TNR / 2) + j * 32 + fr;
          C[col] = f32_to_bf16(silu_mul(acc[i][j][r], acc[i][j + TNB / 2][r]));
        }
      } else if (MODE == kStore) {
        uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
#pragma unroll
        for (int j = 0; j < TNB; ++j) C[nt * BNR + brow0[j] + fr] = f32_to_bf16(acc[i][j][r]);
      } else {
        float* C = static_cast<float*>(a.C) + static_cast<int64_t>(row) * a.ldc;
#pragma unroll
        for (int j = 0; j < TNB; ++j) {
          const int col = nt * BNR + brow0[j] + fr;
          if (col < a.N_valid) C[col] = acc[i][j][r];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Small-M tile for weight streaming: 16 rows x 16*NB B rows per workgroup; the 4 waves
// split K, each streams its K range of every B row straight from global memory into
// v_mfma_f32_16x16x32_bf16 operands; partial sums meet in LDS.
// ----------------------------------------------------------------------------------------
template <int NB, int MODE>
__global__ void __launch_bounds__(256) gemm_bf16_stream(GemmArgs a) {
  constexpr int BNR = 16 * NB;
  constexpr int U = 4;  // K steps in flight per wave
  static_assert(MODE != kSiluMul || NB % 2 == 0, "gate/up pairs");
  __shared__ float red[4][NB][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mb = blockIdx.x % a.m_blocks;
  const int nt = blockIdx.x / a.m_blocks;
  const int m0 = mb * 16;
  if (m0 >= gemm_rows_active(a)) return;
  const int slot = a.block_expert ? a.block_expert[m0 / a.block_m] : 0;
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(a.B) + slot * a.b_stride;
  const int K = a.K;
  const int q = lane & 15;
  const int kq = (lane >> 4) * 8;

  const uint16_t* pa = A + static_cast<int64_t>(gemm_src_row(a, m0 + q)) * K + kq;
  const uint16_t* pb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int brow;
    if (MODE == kSiluMul)
      brow = nb < NB / 2 ? nt * (BNR / 2) + nb * 16 + q : a.N + nt * (BNR / 2) + (nb - NB / 2) * 16 + q;
    else {
      brow = nt * BNR + nb * 16 + q;
      if (MODE == kStoreF32 && brow >= a.N_valid) brow = a.N_valid - 1;
    }
    pb[nb] = B + static_cast<int64_t>(brow) * K + kq;
  }

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = K / 32;
  const int s0 = steps * wave / 4;
  const int s1 = steps * (wave + 1) / 4;
  int s = s0;
  for (; s + U <= s1; s += U) {
    uint4 va[U], vb[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      va[u] = load16(pa + (s + u) * 32);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vb[u][nb] = load16(pb[nb] + (s + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[u]), as_bf16x8(vb[u][nb]),
                                                          acc[nb], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const bf16x8 fa = as_bf16x8(load16(pa + s * 32));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, as_bf16x8(load16(pb[nb] + s * 32)),
                                                        acc[nb], 0, 0, 0);
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][nb][r][lane] = acc[nb][r];
  __syncthreads();

  // acc[nb][r] of lane l sits at row 4*(l/16) + r, B row nb*16 + l%16.
  constexpr int NOUT = (MODE == kSiluMul ? NB / 2 : NB) * 4 * 64;
  for (int idx = tid; idx < NOUT; idx += 256) {
    const int l = idx & 63;
    const int r = (idx >> 6) & 3;
    const int nb = idx >> 8;
    const int row = m0 + 4 * (l >> 4) + r;
    if (row >= a.M_rows) continue;
    const float v = red[0][nb][r][l] + red[1][nb][r][l] + red[2][nb][r][l] + red[3][nb][r][l];
    if (MODE == kSiluMul) {
      const int nu = nb + NB / 2;
      const float u = red[0][nu][r][l] + red[1][nu][r][l] + red[2][nu][r][l] + red[3][nu][r][l];
      uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
      C[nt * (BNR / 2) + nb * 16 + (l & 15)] = f32_to_bf16(silu_mul(v, u));
    } else if (MODE == kStore) {
      uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
      C[nt * BNR + nb * 16 + (l & 15)] = f32_to_bf16(v);
    } else {
      const int col = nt * BNR + nb * 16 + (l & 15);
      if (col < a.N_valid) static_cast<float*>(a.C)[static_cast<int64_t>(row) * a.ldc + col] = v;
    }
  }
}

// ----------------------------------------------------------------------------------------
// fp32 tile (FMA): 16 rows x 64 B rows per workgroup, K step 16. Thread (ty, tx) owns row ty
// and 4 B rows; in kSiluMul the 64 B rows are 32 gate rows then the 32 matching up rows and
// a thread owns gate and up of 2 output columns.
// ----------------------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(256) gemm_f32_tile(GemmArgs a) {
  constexpr int BM = 16, BNR = 64, BK = 16;
  __shared__ float sA[BK][BM + 1];
  __shared__ float sB[BK][BNR + 1];
  const int tid = threadIdx.x;
  const int mb = blockIdx.x % a.m_blocks;
  const int nt = blockIdx.x / a.m_blocks;
  const int m0 = mb * BM;
  if (m0 >= gemm_rows_active(a)) return;
  const int slot = a.block_expert ? a.block_expert[m0 / a.block_m] : 0;
  const float* __restrict__ A = static_cast<const float*>(a.A);
  const float* __restrict__ B = static_cast<const float*>(a.B) + slot * a.b_stride;
  const int K = a.K;

  // loads: A 16x16 (1 per thread), B 64x16 (4 per thread); k fastest across threads
  const int lk = tid & 15;
  const int lr = tid >> 4;  // 0..15
  const float* pa = A + static_cast<int64_t>(gemm_src_row(a, m0 + lr)) * K + lk;
  const float* pb[4];
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 16 * i;
    int brow;
    if (MODE == kSiluMul)
      brow = r < BNR / 2 ? nt * (BNR / 2) + r : a.N + nt * (BNR / 2) + (r - BNR / 2);
    else {
      brow = nt * BNR + r;
      if (MODE == kStoreF32 && brow >= a.N_valid) brow = a.N_valid - 1;
    }
    pb[i] = B + static_cast<int64_t>(brow) * K + lk;
  }
  const int ty = tid >> 4;
  const int tx = tid & 15;
  int bcol[4];
  if (MODE == kSiluMul) {
    bcol[0] = 2 * tx; bcol[1] = 2 * tx + 1; bcol[2] = 32 + 2 * tx; bcol[3] = 33 + 2 * tx;
  } else {
    for (int c = 0; c < 4; ++c) bcol[c] = 4 * tx + c;
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += BK) {
    sA[lk][lr] = pa[k0];
    for (int i = 0; i < 4; ++i) sB[lk][lr + 16 * i] = pb[i][k0];
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float xv = sA[kk][ty];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(xv, sB[kk][bcol[c]], acc[c]);
    }
    __syncthreads();
  }
  const int row = m0 + ty;
  if (row >= a.M_rows) return;
  float* C = static_cast<float*>(a.C) + static_cast<int64_t>(row) * a.ldc;
  if (MODE == kSiluMul) {
    C[nt * (BNR / 2) + 2 * tx] = silu_mul(acc[0], acc[2]);
    C[nt * (BNR / 2) + 2 * tx + 1] = silu_mul(acc[1], acc[3]);
  } else {
    for (int c = 0; c < 4; ++c) {
      const int col = nt * BNR + bcol[c];
      if (MODE == kStore || col < a.N_valid) C[col] = acc[c];
    }
  }
}

}  // namespace moe
