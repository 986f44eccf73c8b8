// Grouped "NT" GEMM kernels of the expert MLP (gfx950).
//
//   C[r, n] = sum_k A[src(r), k] * B_slot(r)[n, k]
//
// A rows are token activations, gathered through the expert-sorted pair list
// (src(r) = sorted_pairs[r] / top_k, padding rows read token 0) or taken in order
// (identity, for the shared expert and the router). B is a weight matrix stored with the
// reduction dimension contiguous ([rows, K]), selected per block of rows by block_expert.
// Epilogues: fused act(gate + b_gate, up + b_up) for the w13 projection (gate rows [0, N), up
// rows [N, 2N) of B; act = silu(g) * u or gpt-oss's clamped SwiGLU; the per-slot biases
// optional), bf16 store (+ optional per-slot bias) for the w2 projection, bounded fp32 store
// for router logits.
#pragma once

#include <type_traits>

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
  const int32_t* block_expert; // sorted rows: slot of each block of block_m rows (NULL = slot 0);
                               // variable row blocks: the block table (count, then slot and
                               // first row of each block, then -1 and the padded total)
  const int32_t* valid_map;    // LDS tile with SKIP: the sorted pair list, whose -1 entries mark
                               // padding rows (padding ends each expert's segment)
  const int32_t* store_map;    // LDS tile, bf16 out: rows whose entry is < 0 (padding of the
                               // sorted pair list) are not stored; NULL = every row
  int32_t block_m;             // padding granule of the sorted rows (a multiple of the tile rows)
  const void* B;               // weights of slot s at B + s * b_stride elements, [rows, K]
  int64_t b_stride;
  int32_t K;
  int32_t N;                   // kSiluMul: output columns (I); else output columns
  int32_t N_valid;             // kStoreF32: valid output columns (B rows past it are clamped)
  void* C;                     // output, row stride ldc elements
  int64_t ldc;
  int32_t m_blocks;            // grid extent along rows (the largest possible row-block count)
  int32_t n_tiles;             // output tiles along the B rows
  int32_t k_splits;            // kStoreF32 only: blockIdx.y takes K range y*K/k_splits.. and
                               // writes its partial sums to C + y * c_split_stride (0 or 1 = no split)
  int64_t c_split_stride;
  int32_t tail_mode;           // LDS tile only. 0: every active tile; 1: every active tile but the
                               // tail (tail_tiles); 2: the quarter tiles (half BM, half BNR) of the
                               // tail of the tiling with twice this kernel's BM and BNR
  int32_t n_cu;                // tiles per round (one workgroup per CU) for the tail rule
  const float* bias;           // kSiluMul: [slots, 2N] gate then up biases; kStore: [slots, N];
                               // slot s at bias + s * bias_stride; NULL = none
  int64_t bias_stride;
  int32_t act;                 // kSiluMul: 0 = silu, 1 = swigluoai
  int32_t b_packed;            // 1: B in the packed weight layout (b_offset), bf16 kernels only
  int32_t b_nt;                // LDS tile kernels: 1 = weight loads with the non-temporal hint
                               // (the launch picks the kernel instantiation that has it)
};

// Packed weight layout: each [rows, K] bf16 matrix is stored as 1 KiB blocks of 16 rows x 32
// K elements (row-major inside the block); the K blocks of one 16-row panel follow each other,
// then the next panel. A load instruction that fetches 16 rows x 64 bytes, or 8 rows x 128
// bytes, then reads one or two contiguous pieces of 1 KiB or 512 bytes instead of 16 or 8
// separate row segments. Byte offset of element (row, k), k a multiple of 8:
__device__ __forceinline__ uint32_t b_offset(const GemmArgs& a, int row, int k) {
  if (!a.b_packed) return static_cast<uint32_t>(row) * static_cast<uint32_t>(a.K * 2) + k * 2;
  return (static_cast<uint32_t>(row >> 4) * static_cast<uint32_t>(a.K >> 5) + (k >> 5)) * 1024u +
         (row & 15) * 64 + (k & 31) * 2;
}

// Bytes between the B data of consecutive K steps of bk elements (bk a multiple of 32).
__device__ __forceinline__ uint32_t b_step(const GemmArgs& a, int bk) {
  return a.b_packed ? bk * 32 : bk * 2;
}

// K range [k0, k0 + klen) of this workgroup (blockIdx.y selects the split).
__device__ __forceinline__ void k_range(const GemmArgs& a, int& k0, int& klen) {
  const int s = a.k_splits > 1 ? a.k_splits : 1;
  klen = a.K / s;
  k0 = static_cast<int>(blockIdx.y) * klen;
}

// MI355X dispatches workgroup i to XCD i % 8; each XCD has its own L2.
constexpr int kXcds = 8;
// N tiles that run side by side on one XCD and share their A row-block through its L2.
constexpr int kGroupN = 4;

// XCD-aware tile order. The active tiles (row blocks below the device row count) are cut
// into kXcds contiguous runs, one per XCD, so that workgroups on one XCD share operands in
// its L2. Inside a run, tiles go row-block-major within groups of kGroupN N tiles: the row
// blocks of one expert that read the same weight tile are consecutive and run together.
//
// N tiles per group in the variable-block kernels' tile order: eight 256-wide weight tiles
// times an expert's row blocks stay on one XCD, so its L2 serves the weight tile to every row
// block of the expert (measured 0.5% faster than four on the Mixtral-shaped layer, 16 is 8% slower).
constexpr int kVarGroupN = 8;

// Linear tile L -> (row block, N tile), in groups of gn N tiles.
__device__ __forceinline__ void tile_coords(int L, int active_m, int n_tiles, int& mb, int& nt,
                                            int gn = kGroupN) {
  const int ng = L / (active_m * gn);
  const int rem = L - ng * active_m * gn;
  const int width = min(gn, n_tiles - ng * gn);
  mb = rem / width;
  nt = ng * gn + rem % width;
}

// Workgroup bid -> linear tile of the first `count`, striped over the XCDs; false for
// workgroups that have no tile (the grid is sized for the worst case).
__device__ __forceinline__ bool xcd_tile(int bid, int count, int& L) {
  const int per_xcd = (count + kXcds - 1) / kXcds;
  const int slot = bid / kXcds;
  if (slot >= per_xcd) return false;
  L = (bid % kXcds) * per_xcd + slot;
  return L < count;
}

__device__ __forceinline__ bool tile_of_block(int bid, int active_m, int n_tiles, int& mb, int& nt) {
  int L;
  if (!xcd_tile(bid, active_m * n_tiles, L)) return false;
  tile_coords(L, active_m, n_tiles, mb, nt);
  return true;
}

// Tail balancing. With one workgroup per CU, `total` tiles run in rounds of n_cu; a last
// partial round of rem tiles takes as long as a full one. When four quarter tiles (half the
// rows, half the weight rows) per tail tile still fit one round, a second launch of the
// quarter-tile kernel takes the last rem tiles of the order: no reduction is involved, each
// output element still has one writer and one K loop.
__device__ __forceinline__ int tail_tiles(int total, int n_cu) {
  const int rem = n_cu > 0 ? total % n_cu : 0;
  return 4 * rem <= n_cu ? rem : 0;
}

// Grid size for the tile order above.
inline int tile_grid(int m_blocks, int n_tiles) {
  return (m_blocks * n_tiles + kXcds - 1) / kXcds * kXcds;
}

__device__ __forceinline__ int gemm_src_row(const GemmArgs& a, int r) {
  if (a.row_map) {
    const int p = a.row_map[r];
    return (p < 0 || p >= a.M_pairs) ? 0 : p / a.row_div;
  }
  return r < a.M_rows ? r : a.M_rows - 1;
}

// Source rows of N tile rows (each below the device row count) at once: the N pair-list
// loads are all issued before any is used, one memory round trip instead of N, and the
// padding / range rule is applied without branches.
template <int N>
__device__ __forceinline__ void gemm_src_rows(const GemmArgs& a, const int (&r)[N], int (&src)[N]) {
  if (a.row_map) {
    int p[N];
#pragma unroll
    for (int j = 0; j < N; ++j) p[j] = a.row_map[r[j]];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int q = p[j] < 0 || p[j] >= a.M_pairs ? 0 : p[j];
      src[j] = static_cast<int>(static_cast<uint32_t>(q) / static_cast<uint32_t>(a.row_div));
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) src[j] = min(r[j], a.M_rows - 1);
  }
}

__device__ __forceinline__ int gemm_rows_active(const GemmArgs& a) {
  return a.num_padded ? *a.num_padded : a.M_rows;
}

// Tile of this workgroup for a BM-row LDS tile kernel under a.tail_mode.
template <int BM>
__device__ __forceinline__ bool gemm_tile(const GemmArgs& a, int& mb, int& nt) {
  const int rows = gemm_rows_active(a);
  if (a.tail_mode == 2) {
    const int am = (rows + 2 * BM - 1) / (2 * BM);
    const int nb = a.n_tiles / 2;
    const int total = am * nb;
    const int rem = tail_tiles(total, a.n_cu);
    const int u = static_cast<int>(blockIdx.x);
    if (u >= 4 * rem) return false;
    int MB, NT;
    tile_coords(total - rem + u / 4, am, nb, MB, NT);
    mb = 2 * MB + ((u >> 1) & 1);
    nt = 2 * NT + (u & 1);
    return true;
  }
  const int am = (rows + BM - 1) / BM;
  const int total = am * a.n_tiles;
  const int count = a.tail_mode == 1 ? total - tail_tiles(total, a.n_cu) : total;
  int L;
  if (!xcd_tile(static_cast<int>(blockIdx.x), count, L)) return false;
  tile_coords(L, am, a.n_tiles, mb, nt);
  return true;
}

// ----------------------------------------------------------------------------------------
// Large-M tile fed by global->LDS loads (gfx950 global_load_lds_dwordx4): each lane's 16 bytes
// go straight from memory into LDS without passing through registers, so the waves issue
// only the loads, the LDS fragment reads and the MFMAs. 4 or 8 waves (with 8, two per SIMD:
// one wave's waits are covered by the other's MFMAs), K step BK = 64, two LDS stages
// (separate arrays, addressed statically).
//
// Schedule of K step t (stage S = t % 2, the other stage S' holds step t + 1, in flight):
//   slice 0..2 : read the fragments of slice s+1 from S, then the MFMAs of slice s
//   sync point : wait for this wave's loads of step t+1 and its slice-3 reads, barrier
//                (now every load of step t+1 has landed and no wave reads S any more)
//   slice 3    : read slice 0 of step t+1 from S', then the MFMAs of slice 3 with the loads
//                of step t+2 into S spread between them
// so the MFMA pipe keeps working across the step boundary and the loads have a whole step
// to land.
// LDS rows are the 64 bf16 (128 bytes) of one tile row; the eight 16-byte chunks of row r are
// stored at chunk ^ sw(r), sw(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads of
// 16 consecutive rows hit distinct banks. One load instruction fills 8 rows (1 KiB, lane l at
// byte 16 l): lane l loads row 8 j + l / 8, logical chunk (l % 8) ^ sw(row). NT: the weight
// loads carry the non-temporal hint (a compile-time choice, as in gemm_bf16_var4: measured,
// skewed T=16384 layer 6.50 -> 6.40 ms and DeepSeek-V2-shaped 0.616 -> 0.607 ms against a
// branch on GemmArgs::b_nt per weight load).
// ----------------------------------------------------------------------------------------
template <int BM, int BNR, int WM, int WN, int MODE, int NS = 2, bool SKIP = false, bool NT = false>
__global__ void __launch_bounds__(64 * WM * WN) gemm_bf16_dma(GemmArgs a) {
  constexpr int NW = WM * WN;              // waves (4, or 8 = two per SIMD)
  constexpr int BK = 64;
  constexpr int ROWB = 128;                // bytes of one LDS row
  constexpr int TM = BM / WM;
  constexpr int TMB = TM / 32;
  constexpr int TNR = BNR / WN;
  constexpr int TNB = TNR / 32;
  constexpr int NA = BM / (8 * NW);        // A load instructions per wave per K step
  constexpr int NB = BNR / (8 * NW);       // B load instructions per wave per K step
  constexpr int ND = NA + NB;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(TMB >= 1 && TNB >= 1 && NA >= 1 && NB >= 1, "tile too small");
  static_assert(MODE != kSiluMul || (TNB % 2 == 0), "gate/up pairs");
  static_assert(NS == 2 || NS == 3, "two or three LDS stages");

  __shared__ __attribute__((aligned(1024))) uint8_t sA[NS][BM * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[NS][BNR * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int mb, nt;
  if (!gemm_tile<BM>(a, mb, nt)) return;
  const int m0 = mb * BM;
  const int slot = a.block_expert ? a.block_expert[m0 / a.block_m] : 0;
  const char* const Abase = static_cast<const char*>(a.A);
  const char* const Bbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.B) + slot * a.b_stride);
  const int K = a.K;
  int k0, klen;
  k_range(a, k0, klen);

  // Load sources: instruction d < NA of this wave fills A rows 8 (wave + NW d) .. +7, the
  // others B rows likewise. Kept as 32-bit byte offsets from the (wave-uniform) operand
  // bases: an expert's weights and the activations are each far below 4 GiB.
  const int lrow = lane >> 3;
  uint32_t goff[ND];
  {
    int rows[NA], src[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) rows[j] = m0 + 8 * (wave + NW * j) + lrow;
    gemm_src_rows(a, rows, src);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int blk = wave + NW * j;
      const int c = (lane & 7) ^ lrow ^ (blk & 1);
      goff[j] = static_cast<uint32_t>(src[j]) * static_cast<uint32_t>(K * 2) + c * 16 + k0 * 2;
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int blk = wave + NW * j;
    const int r = 8 * blk + lrow;
    const int c = (lane & 7) ^ lrow ^ (blk & 1);
    int brow;
    if (MODE == kSiluMul)
      brow = r < BNR / 2 ? nt * (BNR / 2) + r : a.N + nt * (BNR / 2) + (r - BNR / 2);
    else {
      brow = nt * BNR + r;
      if (MODE == kStoreF32 && brow >= a.N_valid) brow = a.N_valid - 1;
    }
    goff[NA + j] = b_offset(a, brow, k0 + c * 8);
  }
  const uint32_t bstep = b_step(a, BK);
  // SKIP: real rows of the tile (a prefix, since padding ends each expert's segment). Every
  // tile row is one of this lane group's DMA rows; lanes with (lane & 7) == 0 count each once.
  __shared__ int real_rows[SKIP ? NW : 1];
  if constexpr (SKIP) {
    int rows[NA], pv[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) rows[j] = m0 + 8 * (wave + NW * j) + lrow;
#pragma unroll
    for (int j = 0; j < NA; ++j) pv[j] = a.valid_map[rows[j]];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NA; ++j) cnt += __popcll(__ballot((lane & 7) == 0 && pv[j] >= 0));
    if (lane == 0) real_rows[wave] = cnt;
  }
  uint32_t lA[NS], lB[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    lA[st] = lds_addr(sA[st]);
    lB[st] = lds_addr(sB[st]);
  }
  // load instruction d of K step kt into stage st
  auto dma = [&](int d, int kt, int st) {
    const uint32_t voff = goff[d] + static_cast<uint32_t>(kt) * (d < NA ? BK * 2 : bstep);
    if (d < NA) {
      dma16(Abase, voff, __builtin_amdgcn_readfirstlane(lA[st] + (wave + NW * d) * 1024));
    } else {
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lB[st] + (wave + NW * (d - NA)) * 1024);
      if constexpr (NT)
        dma16_nt(Bbase, voff, lds);
      else
        dma16(Bbase, voff, lds);
    }
  };

  // wave -> (row group, weight-row group)
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int fr = lane & 31;
  // swizzle of the fragment rows (their tile row is a multiple of 32 plus fr)
  const int sw = (fr & 7) ^ ((fr >> 3) & 1);
  int coff[BK / 16];  // byte offset of this lane's 16-byte chunk in K slice ks
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) coff[ks] = ((2 * ks + (lane >> 5)) ^ sw) * 16;
  int arow[TMB], brow0[TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i) arow[i] = (wm * TM + i * 32 + fr) * ROWB;
#pragma unroll
  for (int j = 0; j < TNB; ++j) {
    const int r0 = MODE == kSiluMul
                       ? (j < TNB / 2 ? wn * (TNR / 2) + j * 32 : BNR / 2 + wn * (TNR / 2) + (j - TNB / 2) * 32)
                       : wn * TNR + j * 32;
    brow0[j] = (r0 + fr) * ROWB;
  }

  f32x16 acc[TMB][TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[2][TMB], fb[2][TNB];  // fragments of two K slices
  int nact = TMB;                  // SKIP: MFMA row blocks of this wave with real rows
  auto frags = [&](const uint8_t* pA, const uint8_t* pB, int ks, int set) {
#pragma unroll
    for (int i = 0; i < TMB; ++i) fa[set][i] = as_bf16x8(*reinterpret_cast<const uint4*>(pA + arow[i] + coff[ks]));
#pragma unroll
    for (int j = 0; j < TNB; ++j) fb[set][j] = as_bf16x8(*reinterpret_cast<const uint4*>(pB + brow0[j] + coff[ks]));
  };
  // MFMAs of one K slice. DM = 0: nothing else; DM = 1 + st: loads D0 .. D1-1 of K step
  // kt_dma into stage st go between them.
  auto mfmas = [&](int set, auto dm_c, int kt_dma, auto d0_c, auto d1_c) {
    constexpr int DM = decltype(dm_c)::value;
    constexpr int D0 = decltype(d0_c)::value;
    constexpr int D1 = decltype(d1_c)::value;
    constexpr int NM = TMB * TNB;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      // weight fragment first: acc holds the transposed block (see the epilogue). With SKIP,
      // row blocks of padding only are skipped (their accumulators stay 0): about 3% of the
      // sorted prefill GEMM; a dense launch keeps the branch-free loop.
      if (!SKIP || m / TNB < nact)
        acc[m / TNB][m % TNB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][m % TNB], fa[set][m / TNB],
                                                                        acc[m / TNB][m % TNB], 0, 0, 0);
      if constexpr (DM != 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = D0 + m * (D1 - D0) / NM; d < D0 + (m + 1) * (D1 - D0) / NM; ++d) dma(d, kt_dma, DM - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using CND = std::integral_constant<int, ND>;
  // Loads of K step kt+2 and where they go. Two stages: into this step's stage, after the
  // sync point, all during slice 3. Three stages: into the stage of step kt-1 (free since the
  // sync point of step kt-1), spread over slices 0..2 of this step, so they have two steps to
  // land; the sync point then waits for step kt+1 only (vmcnt(ND)).
  // K step kt on stage ST. KIND 0: step kt+2 gets loaded; 1: step kt+1 is the last;
  // 2: kt is the last step.
  auto step = [&](auto st_c, auto kind_c, int kt) {
    constexpr int ST = decltype(st_c)::value;
    constexpr int KIND = decltype(kind_c)::value;
    constexpr int NX = (ST + 1) % NS;                    // stage of step kt+1
    constexpr int NL = NS == 3 ? (ST + 2) % NS : ST;     // stage that receives step kt+2
    using L3 = std::integral_constant<int, (NS == 3 && KIND == 0) ? 1 + NL : 0>;
    using T1 = std::integral_constant<int, ND / 3>;
    using T2 = std::integral_constant<int, 2 * ND / 3>;
    __builtin_amdgcn_sched_barrier(0);
    frags(sA[ST], sB[ST], 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0, L3{}, kt + 2, C0{}, T1{});
    __builtin_amdgcn_sched_barrier(0);
    frags(sA[ST], sB[ST], 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1, L3{}, kt + 2, T1{}, T2{});
    __builtin_amdgcn_sched_barrier(0);
    frags(sA[ST], sB[ST], 3, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0, L3{}, kt + 2, T2{}, CND{});
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KIND < 2) {
      if constexpr (NS == 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
        __syncthreads();
      } else {
        __builtin_amdgcn_s_waitcnt(KIND == 0 ? wait_vm_lgkm0(ND) : kWaitVmLgkm0);
        wg_barrier();
      }
      frags(sA[NX], sB[NX], 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NS == 2 && KIND == 0)
        mfmas(1, std::integral_constant<int, 1 + NL>{}, kt + 2, C0{}, CND{});
      else
        mfmas(1, C0{}, 0, C0{}, C0{});
    } else {
      mfmas(1, C0{}, 0, C0{}, C0{});
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: steps 0 and 1 in flight into stages 0 and 1, wait for step 0, slice 0 read.
  const int nk = klen / BK;
#pragma unroll
  for (int d = 0; d < ND; ++d) dma(d, 0, 0);
  if (nk > 1) {
#pragma unroll
    for (int d = 0; d < ND; ++d) dma(d, 1, 1);
    __builtin_amdgcn_s_waitcnt(wait_vm(ND));
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
  __syncthreads();
  if constexpr (SKIP) {
    int nreal = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) nreal += real_rows[w];
    nact = __builtin_amdgcn_readfirstlane(min(TMB, max(0, (nreal - wm * TM + 31) / 32)));
  }
  frags(sA[0], sB[0], 0, 0);
  if constexpr (NS == 2) {
    if (nk == 1) {
      step(C0{}, C2{}, 0);
    } else if ((nk & 1) == 0) {
      for (int kt = 0; kt < nk - 2; kt += 2) {
        step(C0{}, C0{}, kt);
        step(C1{}, C0{}, kt + 1);
      }
      step(C0{}, C1{}, nk - 2);
      step(C1{}, C2{}, nk - 1);
    } else {
      for (int kt = 0; kt < nk - 3; kt += 2) {
        step(C0{}, C0{}, kt);
        step(C1{}, C0{}, kt + 1);
      }
      step(C0{}, C0{}, nk - 3);
      step(C1{}, C1{}, nk - 2);
      step(C0{}, C2{}, nk - 1);
    }
  } else {
    // groups of three loading steps, then a static tail of 2..4 steps (stage of kt: kt % 3)
    int kt = 0;
    if (nk >= 2) {
      for (; kt + 5 <= nk; kt += 3) {
        step(C0{}, C0{}, kt);
        step(C1{}, C0{}, kt + 1);
        step(C2{}, C0{}, kt + 2);
      }
    }
    const int r = nk - kt;
    if (nk == 1) {
      step(C0{}, C2{}, 0);
    } else if (r == 2) {
      step(C0{}, C1{}, kt);
      step(C1{}, C2{}, kt + 1);
    } else if (r == 3) {
      step(C0{}, C0{}, kt);
      step(C1{}, C1{}, kt + 1);
      step(C2{}, C2{}, kt + 2);
    } else {
      step(C0{}, C0{}, kt);
      step(C1{}, C0{}, kt + 1);
      step(C2{}, C1{}, kt + 2);
      step(C0{}, C2{}, kt + 3);
    }
  }

  // Epilogue. The MFMAs take the weight fragment as first operand, so acc[i][j] is the
  // transposed 32x32 block: register r of lane l belongs to output row wm*TM + i*32 + l%32 and
  // to column 8*(r/4) + 4*(l/32) + r%4 of the block's 32 output columns, i.e. each lane holds
  // four consecutive columns in each group q = r/4.
  const int orow = m0 + wm * TM + fr;
  if constexpr (MODE == kStoreF32) {
#pragma unroll
    for (int i = 0; i < TMB; ++i) {
      const int row = orow + i * 32;
      if (row >= a.M_rows) continue;
      float* C = static_cast<float*>(a.C) + blockIdx.y * a.c_split_stride + static_cast<int64_t>(row) * a.ldc;
#pragma unroll
      for (int j = 0; j < TNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = nt * BNR + wn * TNR + j * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (col < a.N_valid) C[col] = acc[i][j][r];
        }
    }
  } else {
    // bf16 out: pack each group's four columns into two dwords, then swap groups between
    // lanes l and l + 32 (v_permlane32_swap) so that lane l < 32 holds columns 0..7 and
    // 16..23 of the block and lane l + 32 columns 8..15 and 24..31: two 16-byte stores.
    constexpr int OUTB = MODE == kSiluMul ? TNB / 2 : TNB;  // 32-column output blocks per wave
    const int col0 = (MODE == kSiluMul ? nt * (BNR / 2) + wn * (TNR / 2) : nt * BNR + wn * TNR) + 8 * (lane >> 5);
    // column of register 4 q + 2 h (and + 1) of block j before the lane swap:
    // colb + 32 j + 8 q + 2 h
    const int colb = col0 - 8 * (lane >> 5) + 4 * (lane >> 5);
    const float* const bias = a.bias ? a.bias + slot * a.bias_stride : nullptr;
    const int act = a.act;
#pragma unroll
    for (int i = 0; i < TMB; ++i) {
      const int row = orow + i * 32;
      const bool keep = row < a.M_rows && (!a.store_map || a.store_map[row] >= 0);
      uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc + col0;
#pragma unroll
      for (int j = 0; j < OUTB; ++j) {
        uint32_t p[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float v0, v1;
            if constexpr (MODE == kSiluMul) {
              float g0 = acc[i][j][4 * q + 2 * h], g1 = acc[i][j][4 * q + 2 * h + 1];
              float u0 = acc[i][j + TNB / 2][4 * q + 2 * h], u1 = acc[i][j + TNB / 2][4 * q + 2 * h + 1];
              if (bias) {
                const int c = colb + 32 * j + 8 * q + 2 * h;
                const float2 bg = *reinterpret_cast<const float2*>(bias + c);
                const float2 bu = *reinterpret_cast<const float2*>(bias + a.N + c);
                g0 += bg.x;
                g1 += bg.y;
                u0 += bu.x;
                u1 += bu.y;
              }
              if (act == 0) {
                v0 = silu_mul(g0, u0);
                v1 = silu_mul(g1, u1);
              } else {
                v0 = swigluoai_mul(g0, u0);
                v1 = swigluoai_mul(g1, u1);
              }
            } else {
              v0 = acc[i][j][4 * q + 2 * h];
              v1 = acc[i][j][4 * q + 2 * h + 1];
              if (bias) {
                const float2 b = *reinterpret_cast<const float2*>(bias + colb + 32 * j + 8 * q + 2 * h);
                v0 += b.x;
                v1 += b.y;
              }
            }
            p[q][h] = pack_bf16x2(v0, v1);
          }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto s01 = __builtin_amdgcn_permlane32_swap(p[0][h], p[1][h], false, false);
          const auto s23 = __builtin_amdgcn_permlane32_swap(p[2][h], p[3][h], false, false);
          p[0][h] = s01[0];
          p[1][h] = s01[1];
          p[2][h] = s23[0];
          p[3][h] = s23[1];
        }
        if (keep) {
          *reinterpret_cast<uint4*>(C + j * 32) = uint4{p[0][0], p[0][1], p[1][0], p[1][1]};
          *reinterpret_cast<uint4*>(C + j * 32 + 16) = uint4{p[2][0], p[2][1], p[3][0], p[3][1]};
        }
      }
    }
  }
}

// Epilogue of the variable-block kernels: the wave's TMB x TNB accumulator blocks (transposed
// MFMA blocks, as gemm_bf16_dma) to bf16 rows of C, with the activation (gate/up) or the bias;
// rows past the block (m0 + vrows) or the output are not stored.
template <int MODE, int TMB, int TNB, int TM, int TNR, int BNR>
__device__ __forceinline__ void var_epilogue(const GemmArgs& a, f32x16 (&acc)[TMB][TNB], int m0, int vrows,
                                             int slot, int nt, int wm, int wn, int lane) {
  const int fr = lane & 31;
  const int orow = m0 + wm * TM + fr;
  constexpr int OUTB = MODE == kSiluMul ? TNB / 2 : TNB;
  const int col0 = (MODE == kSiluMul ? nt * (BNR / 2) + wn * (TNR / 2) : nt * BNR + wn * TNR) + 8 * (lane >> 5);
  const int colb = col0 - 8 * (lane >> 5) + 4 * (lane >> 5);
  const float* const bias = a.bias ? a.bias + slot * a.bias_stride : nullptr;
  const int act = a.act;
  const int rend = min(m0 + vrows, a.M_rows);
#pragma unroll
  for (int i = 0; i < TMB; ++i) {
    const int row = orow + i * 32;
    const bool keep = row < rend && (!a.store_map || a.store_map[row] >= 0);
    uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc + col0;
#pragma unroll
    for (int j = 0; j < OUTB; ++j) {
      uint32_t p[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v0, v1;
          if constexpr (MODE == kSiluMul) {
            float g0 = acc[i][j][4 * q + 2 * h], g1 = acc[i][j][4 * q + 2 * h + 1];
            float u0 = acc[i][j + TNB / 2][4 * q + 2 * h], u1 = acc[i][j + TNB / 2][4 * q + 2 * h + 1];
            if (bias) {
              const int c = colb + 32 * j + 8 * q + 2 * h;
              const float2 bg = *reinterpret_cast<const float2*>(bias + c);
              const float2 bu = *reinterpret_cast<const float2*>(bias + a.N + c);
              g0 += bg.x;
              g1 += bg.y;
              u0 += bu.x;
              u1 += bu.y;
            }
            v0 = act_mul(g0, u0, act);
            v1 = act_mul(g1, u1, act);
          } else {
            v0 = acc[i][j][4 * q + 2 * h];
            v1 = acc[i][j][4 * q + 2 * h + 1];
            if (bias) {
              const float2 b = *reinterpret_cast<const float2*>(bias + colb + 32 * j + 8 * q + 2 * h);
              v0 += b.x;
              v1 += b.y;
            }
          }
          p[q][h] = pack_bf16x2(v0, v1);
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto s01 = __builtin_amdgcn_permlane32_swap(p[0][h], p[1][h], false, false);
        const auto s23 = __builtin_amdgcn_permlane32_swap(p[2][h], p[3][h], false, false);
        p[0][h] = s01[0];
        p[1][h] = s01[1];
        p[2][h] = s23[0];
        p[3][h] = s23[1];
      }
      if (keep) {
        *reinterpret_cast<uint4*>(C + j * 32) = uint4{p[0][0], p[0][1], p[1][0], p[1][1]};
        *reinterpret_cast<uint4*>(C + j * 32 + 16) = uint4{p[2][0], p[2][1], p[3][0], p[3][1]};
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Variable row blocks: one block of the block table per tile row range (32 .. 320 rows, a
// multiple of 32, inside one expert's segment: 256-row blocks, where an expert's last piece of
// at most 64 rows joins the block before it instead of taking a nearly empty tile of its own).
// 320 x 256 tile, 8 waves (2 x 4, 160 x 64 each, two per SIMD), v_mfma_f32_32x32x16_bf16. Each
// wave runs the K loop compiled for the number of its five 32-row MFMA blocks that hold rows of
// the block (no MFMA or fragment read for the others). Register budget (two waves per SIMD):
// the A fragments are single-buffered, each read for the next K slice right after its row
// block's last MFMA of this slice; the B fragments alternate between two sets.
// K step 32 and four LDS stages in a ring (144 KiB), so the loads run three and a half K steps
// ahead of the MFMAs: about 108 KiB in flight per CU. Measured against a two-stage version
// with K step 64 (loads one and a half steps ahead): EP share T=8192 gate/up 87 -> 80 us, down
// 57 -> 52 us, Mixtral-shaped T=4096 layer 2.48 -> 2.44 ms (same box, two rounds). Weight
// loads carry the non-temporal hint where the weights stream (NT, taken from GemmArgs::b_nt
// at launch). The hint is a compile-time choice: one branch per weight load on the flag cost
// 1-1.7% on the Mixtral-shaped layer (two branches per K step in the loop).
// LDS rows are the 32 bf16 (64 bytes) of one tile row; the four 16-byte chunks of row r sit at
// chunk ^ ((r >> 2) & 3), so the fragment reads of 16 consecutive rows cover all banks. One
// load instruction fills 16 rows (lane l: row 16 j + l / 4, position l % 4). Per wave and K
// step: A instructions j = 0..2 for 16-row groups wave + 8 j < 20 that start inside the block,
// B instructions j = 0, 1. A wave waits at each step boundary for its loads of the next step
// only (vmcnt = its loads issued since), then the workgroup meets at a barrier without the
// fence of __syncthreads (which would wait for every load in flight).
// ----------------------------------------------------------------------------------------
template <int MODE, bool NT>
__global__ void __launch_bounds__(512) gemm_bf16_var4(GemmArgs a) {
  constexpr int BM = 320, BNR = 256, WM = 2, WN = 4, NW = 8;
  constexpr int BK = 32, ROWB = 64, NS = 4;
  constexpr int TM = BM / WM, TMB = TM / 32;        // 160 rows, 5 MFMA row blocks per wave
  constexpr int TNR = BNR / WN, TNB = TNR / 32;     // 64 weight rows, 2 MFMA column blocks
  constexpr int AG = BM / 16, BG = BNR / 16;        // 16-row load groups: 20 and 16
  constexpr int NA = (AG + NW - 1) / NW, NB = BG / NW, ND = NA + NB;
  constexpr int SA = BM * ROWB, SB = BNR * ROWB;    // stage bytes
  static_assert(MODE != kStoreF32, "bf16 outputs");
  static_assert(BG % NW == 0, "whole B load groups per wave");

  __shared__ __attribute__((aligned(1024))) uint8_t sA[NS * SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[NS * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* bt = a.block_expert;
  const int nblk = bt[0];
  int L, mb, nt;
  if (!xcd_tile(static_cast<int>(blockIdx.x), nblk * a.n_tiles, L)) return;
  tile_coords(L, nblk, a.n_tiles, mb, nt, kVarGroupN);
  const int slot = bt[1 + 2 * mb];
  const int m0 = bt[2 + 2 * mb];
  const int vrows = min(BM, bt[4 + 2 * mb] - m0);
  const char* const Abase = static_cast<const char*>(a.A);
  const char* const Bbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.B) + slot * a.b_stride);
  const int K = a.K;

  // load sources (rows past the block read its last row)
  const int lrow = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t goff[ND];
  {
    int rows[NA], src[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) rows[j] = m0 + min(16 * (wave + NW * j) + lrow, vrows - 1);
    gemm_src_rows(a, rows, src);
#pragma unroll
    for (int j = 0; j < NA; ++j) goff[j] = static_cast<uint32_t>(src[j]) * static_cast<uint32_t>(K * 2) + lchunk * 16;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = 16 * (wave + NW * j) + lrow;
    const int brow = MODE == kSiluMul ? (r < BNR / 2 ? nt * (BNR / 2) + r : a.N + nt * (BNR / 2) + (r - BNR / 2))
                                      : nt * BNR + r;
    goff[NA + j] = b_offset(a, brow, lchunk * 8);
  }
  const uint32_t bstep = b_step(a, BK);
  const uint32_t lA0 = lds_addr(sA), lB0 = lds_addr(sB);
  // A load instructions of this wave (bit j): the 16-row groups wave + 8 j of the 20; the last
  // one only where its group starts inside the block (rows 256 .. 319 of a block of at most 256
  // rows would move copies of its last row into LDS). Every wave keeps at least AG / NW A loads
  // per K step, the count the waits assume.
  static_assert(NA == 3 && AG / NW == NA - 1, "the last A load is the only one skipped");
  const int glast = wave + NW * (NA - 1);
  const uint32_t amask = glast < AG && 16 * glast < vrows ? (1u << NA) - 1 : (1u << (NA - 1)) - 1;
  constexpr int kMinLoads = AG / NW + NB;  // load instructions per K step of every wave, at least
  // load instruction d of K step kt into stage st
  auto dma = [&](int d, int kt, int st) {
    const uint32_t voff = goff[d] + static_cast<uint32_t>(kt) * (d < NA ? BK * 2 : bstep);
    if (d < NA) {
      if (amask & (1u << d))
        dma16(Abase, voff, __builtin_amdgcn_readfirstlane(lA0 + st * SA + (wave + NW * d) * 1024));
    } else {
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lB0 + st * SB + (wave + NW * (d - NA)) * 1024);
      if constexpr (NT)
        dma16_nt(Bbase, voff, lds);
      else
        dma16(Bbase, voff, lds);
    }
  };

  const int wm = wave / WN;
  const int wn = wave % WN;
  const int fr = lane & 31;
  const int sw = (fr >> 2) & 3;
  int coff[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) coff[ks] = ((2 * ks + (lane >> 5)) ^ sw) * 16;
  const int arow = (wm * TM + fr) * ROWB;  // + i * 32 * ROWB for row block i
  int brow0[TNB];
#pragma unroll
  for (int j = 0; j < TNB; ++j) {
    const int r0 = MODE == kSiluMul
                       ? (j < TNB / 2 ? wn * (TNR / 2) + j * 32 : BNR / 2 + wn * (TNR / 2) + (j - TNB / 2) * 32)
                       : wn * TNR + j * 32;
    brow0[j] = (r0 + fr) * ROWB;
  }

  f32x16 acc[TMB][TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;  // at least NS: K is a multiple of 128

  auto kloop = [&](auto nact_c) {
    constexpr int NACT = decltype(nact_c)::value;
    constexpr int NM = NACT * TNB;
    bf16x8 fa[TMB], fb[2][TNB];
    auto readA = [&](const uint8_t* pA, int ks, int i) {
      fa[i] = as_bf16x8(*reinterpret_cast<const uint4*>(pA + arow + i * 32 * ROWB + coff[ks]));
    };
    auto readB = [&](const uint8_t* pB, int ks, int set) {
#pragma unroll
      for (int j = 0; j < TNB; ++j)
        fb[set][j] = as_bf16x8(*reinterpret_cast<const uint4*>(pB + brow0[j] + coff[ks]));
    };
    // MFMAs of one K slice on B set `set`; NEXT: after row block i's MFMAs, A fragment i of
    // slice ks of pA is read; DMA: the loads of K step kt_dma into stage dst go between them
    auto slice = [&](int set, auto next_c, const uint8_t* pA, int ks, auto dma_c, int kt_dma, int dst) {
      constexpr bool NEXT = decltype(next_c)::value != 0;
      constexpr bool DMA = decltype(dma_c)::value != 0;
      if constexpr (DMA && NM == 0) {
#pragma unroll
        for (int d = 0; d < ND; ++d) dma(d, kt_dma, dst);
      }
#pragma unroll
      for (int i = 0; i < NACT; ++i) {
#pragma unroll
        for (int j = 0; j < TNB; ++j) {
          const int m = i * TNB + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[i], acc[i][j], 0, 0, 0);
          if constexpr (DMA) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = m * ND / (NM > 0 ? NM : 1); d < (m + 1) * ND / (NM > 0 ? NM : 1); ++d) dma(d, kt_dma, dst);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (NEXT) readA(pA, ks, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using On = std::integral_constant<int, 1>;
    using Off = std::integral_constant<int, 0>;

    // K step kt on stage kt % NS. KIND 0: the loads of step kt+NS go out during slice 1;
    // 1, 2, 3: no more loads, the boundary waits for all but 2, 1, 0 steps' loads; 4: the last
    // step (no boundary). Waits count kMinLoads loads per step: a wave with one A instruction
    // more waits for one or two loads of a later step as well.
    auto step = [&](auto kind_c, int kt) {
      constexpr int KIND = decltype(kind_c)::value;
      const int st = kt & (NS - 1);
      const uint8_t* pA = sA + st * SA;
      const uint8_t* pB = sB + st * SB;
      if (NACT > 0) readB(pB, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      slice(0, On{}, pA, 1, Off{}, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (KIND < 4) {
        // the loads of step kt+1 landed and every wave's reads of stage st are done
        constexpr int kAhead = KIND <= 1 ? 2 : 3 - KIND;
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kAhead * kMinLoads));
        wg_barrier();
        const int nx = (kt + 1) & (NS - 1);
        if (NACT > 0) readB(sB + nx * SB, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KIND == 0)
          slice(1, On{}, sA + nx * SA, 0, On{}, kt + NS, st);
        else
          slice(1, On{}, sA + nx * SA, 0, Off{}, 0, 0);
      } else {
        slice(1, Off{}, pA, 0, Off{}, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: steps 0 .. NS-1 in flight (nk >= NS), wait for step 0, slice 0 read
#pragma unroll
    for (int kt = 0; kt < NS; ++kt) {
#pragma unroll
      for (int d = 0; d < ND; ++d) dma(d, kt, kt);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 1) * kMinLoads));
    wg_barrier();
    if (NACT > 0) readB(sB, 0, 0);
#pragma unroll
    for (int i = 0; i < NACT; ++i) readA(sA, 0, i);
    int kt = 0;
    for (; kt + NS < nk; ++kt) step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt);
    step(std::integral_constant<int, 2>{}, kt + 1);
    step(std::integral_constant<int, 3>{}, kt + 2);
    step(std::integral_constant<int, 4>{}, kt + 3);
  };
  // this wave's MFMA row blocks that hold rows of the block
  const int na = __builtin_amdgcn_readfirstlane(min(TMB, max(0, (vrows - wm * TM + 31) / 32)));
  switch (na) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    default: kloop(std::integral_constant<int, 5>{}); break;
  }

  var_epilogue<MODE, TMB, TNB, TM, TNR, BNR>(a, acc, m0, vrows, slot, nt, wm, wn, lane);
}

// ----------------------------------------------------------------------------------------
// Weight-streaming tile for small row counts: 16*MB rows x 16*NB B rows per workgroup; the 4
// waves split K, each streams its K range of every B row and A row straight from global
// memory into v_mfma_f32_16x16x32_bf16 operands (U K steps in flight); partial sums meet in
// LDS. Tiles follow the XCD-aware order of the LDS-fed kernel. A weight tile is read by the
// one or few row blocks of its expert: the weight loads carry the non-temporal hint (measured: skewed share T=1 layer
// 0.182 -> 0.125 ms, Mixtral-shaped T=32 0.544 -> 0.460 ms).
// ----------------------------------------------------------------------------------------
template <int NB, int MODE, int MB = 1>
__global__ void __launch_bounds__(256) gemm_bf16_stream(GemmArgs a) {
  constexpr int BNR = 16 * NB;
  constexpr int U = MB >= 4 ? 2 : 4;  // K steps in flight per wave
  static_assert(MODE != kSiluMul || NB % 2 == 0, "gate/up pairs");
  __shared__ float red[4][MB][NB][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int mb, nt;
  if (!tile_of_block(blockIdx.x, (gemm_rows_active(a) + 16 * MB - 1) / (16 * MB), a.n_tiles, mb, nt))
    return;
  const int m0 = mb * 16 * MB;
  const int slot = a.block_expert ? a.block_expert[m0 / a.block_m] : 0;
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(a.A);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(a.B) + slot * a.b_stride;
  const int K = a.K;
  const int q = lane & 15;
  const int kq = (lane >> 4) * 8;
  int k0, klen;
  k_range(a, k0, klen);

  const uint16_t* pa[MB];
  {
    int rows[MB], src[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) rows[i] = m0 + 16 * i + q;
    gemm_src_rows(a, rows, src);
#pragma unroll
    for (int i = 0; i < MB; ++i) pa[i] = A + static_cast<int64_t>(src[i]) * K + k0 + kq;
  }
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
    pb[nb] = B + b_offset(a, brow, k0 + kq) / 2;
  }
  const int bstep = static_cast<int>(b_step(a, 32) / 2);  // elements per K step of 32

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[i][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = klen / 32;
  const int s0 = steps * wave / 4;
  const int s1 = steps * (wave + 1) / 4;
  // batches of U K steps, double-buffered: the loads of batch b+1 go out before the MFMAs of
  // batch b wait for theirs, so a wave always has a batch in flight
  auto load_batch = [&](uint4 (&va)[U][MB], uint4 (&vb)[U][NB], int sb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vb[u][nb] = load16_nt(pb[nb] + (sb + u) * bstep);
#pragma unroll
      for (int i = 0; i < MB; ++i) va[u][i] = load16(pa[i] + (sb + u) * 32);
    }
  };
  auto mfma_batch = [&](const uint4 (&va)[U][MB], const uint4 (&vb)[U][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[u][i]), as_bf16x8(vb[u][nb]),
                                                               acc[i][nb], 0, 0, 0);
  };
  int s = s0;
  if (s + U <= s1) {
    uint4 va0[U][MB], vb0[U][NB], va1[U][MB], vb1[U][NB];
    load_batch(va0, vb0, s);
    // each path has its own MFMA copy: where a path without the next batch's loads joins one
    // with them, the compiler's wait counts take the smaller and drain the next batch too
    while (true) {
      if (s + 2 * U <= s1) {
        load_batch(va1, vb1, s + U);
        mfma_batch(va0, vb0);
        s += U;
      } else {
        mfma_batch(va0, vb0);
        s += U;
        break;
      }
      if (s + 2 * U <= s1) {
        load_batch(va0, vb0, s + U);
        mfma_batch(va1, vb1);
        s += U;
      } else {
        mfma_batch(va1, vb1);
        s += U;
        break;
      }
    }
  }
  for (; s < s1; ++s) {
    bf16x8 fa[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[i] = as_bf16x8(load16(pa[i] + s * 32));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 fb = as_bf16x8(load16_nt(pb[nb] + s * bstep));
#pragma unroll
      for (int i = 0; i < MB; ++i)
        acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb, acc[i][nb], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][i][nb][r][lane] = acc[i][nb][r];
  __syncthreads();

  // acc[i][nb][r] of lane l sits at row 16 i + 4*(l/16) + r, B row nb*16 + l%16.
  constexpr int NOUT = MB * (MODE == kSiluMul ? NB / 2 : NB) * 4 * 64;
  for (int idx = tid; idx < NOUT; idx += 256) {
    const int l = idx & 63;
    const int r = (idx >> 6) & 3;
    const int nb = (idx >> 8) % (MODE == kSiluMul ? NB / 2 : NB);
    const int i = (idx >> 8) / (MODE == kSiluMul ? NB / 2 : NB);
    const int row = m0 + 16 * i + 4 * (l >> 4) + r;
    if (row >= a.M_rows) continue;
    const float v = red[0][i][nb][r][l] + red[1][i][nb][r][l] + red[2][i][nb][r][l] + red[3][i][nb][r][l];
    if (MODE == kSiluMul) {
      const int nu = nb + NB / 2;
      float u = red[0][i][nu][r][l] + red[1][i][nu][r][l] + red[2][i][nu][r][l] + red[3][i][nu][r][l];
      float g = v;
      const int col = nt * (BNR / 2) + nb * 16 + (l & 15);
      if (a.bias) {
        g += a.bias[slot * a.bias_stride + col];
        u += a.bias[slot * a.bias_stride + a.N + col];
      }
      uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
      C[col] = f32_to_bf16(act_mul(g, u, a.act));
    } else if (MODE == kStore) {
      const int col = nt * BNR + nb * 16 + (l & 15);
      const float b = a.bias ? a.bias[slot * a.bias_stride + col] : 0.f;
      uint16_t* C = static_cast<uint16_t*>(a.C) + static_cast<int64_t>(row) * a.ldc;
      C[col] = f32_to_bf16(a.bias ? v + b : v);
    } else {
      const int col = nt * BNR + nb * 16 + (l & 15);
      if (col < a.N_valid)
        static_cast<float*>(a.C)[blockIdx.y * a.c_split_stride + static_cast<int64_t>(row) * a.ldc + col] = v;
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
  const float* const bias = a.bias ? a.bias + slot * a.bias_stride : nullptr;
  if (MODE == kSiluMul) {
    for (int c = 0; c < 2; ++c) {
      const int col = nt * (BNR / 2) + 2 * tx + c;
      const float g = acc[c] + (bias ? bias[col] : 0.f);
      const float u = acc[2 + c] + (bias ? bias[a.N + col] : 0.f);
      C[col] = act_mul(g, u, a.act);
    }
  } else {
    for (int c = 0; c < 4; ++c) {
      const int col = nt * BNR + bcol[c];
      if (MODE == kStore) C[col] = bias ? acc[c] + bias[col] : acc[c];
      else if (col < a.N_valid) C[col] = acc[c];
    }
  }
}

}  // namespace moe
