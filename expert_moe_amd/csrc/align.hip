// Alignment of the (token, slot) pairs by local expert (gfx950).
//
// The expert loop of "[Feature] Expert parallelism support" (MixtralMoE.forward) works
// expert by expert; "ep_fused_moe_patch.py" (_ep_forward Steps 2-3) sorts the work items
// before handing them to the fused expert kernel. Here the pairs p = t*k + j whose slot is
// local are grouped by slot, kept in increasing p inside a slot, and each slot's segment is
// padded to a multiple of block_m rows so that a GEMM tile never straddles two experts.
//
// Three passes, no host synchronisation (one single-workgroup kernel when T fits one chunk;
// up to 64 chunks the scan runs inside every scatter workgroup, two kernels):
//   count   : one workgroup per chunk of 256 tokens, LDS histogram of its pairs per slot; the
//             workgroups also fill the whole sorted list with -1 (padding)
//   scan    : one workgroup; per-slot exclusive scan over chunks (chunk bases, read in
//             batches of 16), padded segment sizes, exclusive scan over slots (offsets),
//             block -> slot table
//   scatter : one workgroup per chunk; each wave marks its 64 tokens per slot in an LDS
//             64-bit mask; a pair's rank inside its slot is the chunk base plus the number of
//             marked tokens before it (earlier waves, then earlier lanes), which keeps the
//             order stable without sorting
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// Slots of a token's pairs in batches of kSlotBatch (pairs i0 .. i0 + n - 1, n >= 1): the
// batch's loads are all issued before the first is used (addresses clamped to the last pair,
// values past n masked), one memory round trip per batch; -1 for a slot that is not local.
constexpr int kSlotBatch = 8;
__device__ __forceinline__ void load_slots(const int32_t* tl, int64_t i0, int n, int E_l,
                                           int (&s)[kSlotBatch]) {
#pragma unroll
  for (int u = 0; u < kSlotBatch; ++u) s[u] = tl[i0 + min(u, n - 1)];
#pragma unroll
  for (int u = 0; u < kSlotBatch; ++u) s[u] = (u < n && s[u] >= 0 && s[u] < E_l) ? s[u] : -1;
}

// Exclusive prefix sum of v over the 256 threads of the workgroup (thread order), and the
// total: a lane-shift scan inside each wave, then the earlier waves' totals. Every thread
// must call it (it holds a barrier); wsum is 4 ints of LDS.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return before + x - v;
}

// Padded rows and row blocks of one slot's segment of `count` pairs. bm > 0: padded to a
// multiple of bm, one block per bm rows. bm == 0 (variable blocks): padded to a multiple of 32
// and cut into blocks of 256 rows, where a last piece of at most 64 rows joins the block before
// it (blocks of 32 .. 320 rows, every one a multiple of 32).
__device__ __forceinline__ void segment(int count, int bm, int& padded, int& nblocks) {
  if (bm > 0) {
    padded = (count + bm - 1) / bm * bm;
    nblocks = padded / bm;
    return;
  }
  padded = (count + 31) / 32 * 32;
  const int q = padded / 256;
  const int r = padded - 256 * q;
  nblocks = (q >= 1 && r <= 64) ? q : q + (r > 0 ? 1 : 0);
}

// The row-block table of the segments. bm > 0: block_expert[b] = slot of rows [b bm, (b+1) bm).
// bm == 0: bt[0] = number of blocks nb; block b is rows [bt[2 + 2b], bt[2 + 2(b+1)]) of slot
// bt[1 + 2b], with bt[1 + 2 nb] = -1 and bt[2 + 2 nb] = the padded total. Thread e (< E_l) holds
// slot e's segment (offset off, padded rows, row blocks); every thread of the workgroup must
// call it (the variable form holds a scan with barriers; wsum is 4 ints of LDS).
__device__ void write_blocks(int32_t* __restrict__ bt, int e, int E_l, int bm, int off,
                             int padded, int nblocks, int total, int* wsum) {
  if (bm > 0) {
    if (e < E_l)
      for (int b = off / bm; b < (off + padded) / bm; ++b) bt[b] = e;
    return;
  }
  __syncthreads();  // wsum may still be read by the offsets scan
  int nb;
  const int first = wg_exclusive_scan(e < E_l ? nblocks : 0, wsum, nb);
  if (e < E_l)
    for (int j = 0; j < nblocks; ++j) {
      bt[1 + 2 * (first + j)] = e;
      bt[2 + 2 * (first + j)] = off + 256 * j;
    }
  if (e == 0) {
    bt[0] = nb;
    bt[1 + 2 * nb] = -1;
    bt[2 + 2 * nb] = total;
  }
}

// Scatter of one chunk's pairs (chunk blockIdx.x): each wave marks its 64 tokens per slot in
// an LDS mask, and a pair's position is base[slot] plus the marked tokens before it (earlier
// waves, then earlier lanes). base holds this chunk's start per slot and mask is zeroed, both
// visible to the workgroup; every thread must call it (it holds a barrier).
__device__ __forceinline__ void chunk_scatter(const int32_t* __restrict__ tl, int T, int k,
                                              int E_l, const int* base,
                                              unsigned long long (*mask)[256],
                                              int32_t* __restrict__ sorted_pairs,
                                              int32_t* __restrict__ pair_row) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int t = blockIdx.x * kAlignChunk + tid;
  const bool valid = t < T;
  if (valid)
    for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
      int sl[kSlotBatch];
      load_slots(tl, static_cast<int64_t>(t) * k + j0, min(kSlotBatch, k - j0), E_l, sl);
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)
        if (sl[u] >= 0) atomicOr(&mask[wave][sl[u]], 1ull << lane);
    }
  __syncthreads();
  if (!valid) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
    int sl[kSlotBatch];
    const int n = min(kSlotBatch, k - j0);
    load_slots(tl, static_cast<int64_t>(t) * k + j0, n, E_l, sl);
#pragma unroll
    for (int u = 0; u < kSlotBatch; ++u) {
      if (u >= n) break;
      const int64_t pid = static_cast<int64_t>(t) * k + j0 + u;
      const int s = sl[u];
      if (s < 0) {
        pair_row[pid] = -1;
        continue;
      }
      int before = __popcll(mask[wave][s] & below);
      for (int w = 0; w < wave; ++w) before += __popcll(mask[w][s]);
      const int pos = base[s] + before;
      sorted_pairs[pos] = static_cast<int32_t>(pid);
      pair_row[pid] = pos;
    }
  }
}

__global__ void __launch_bounds__(256) align_count(const int32_t* __restrict__ tl, int T, int k,
                                                   int E_l, int32_t* __restrict__ chunk,
                                                   int32_t* __restrict__ sorted_pairs, int cap) {
  __shared__ int hist[256];
  // every sorted slot starts as padding (-1); the scatter pass overwrites the real ones
  for (int i = blockIdx.x * 256 + threadIdx.x; i < cap; i += gridDim.x * 256) sorted_pairs[i] = -1;
  for (int e = threadIdx.x; e < E_l; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kAlignChunk + threadIdx.x;
  if (t < T)
    for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
      int sl[kSlotBatch];
      load_slots(tl, static_cast<int64_t>(t) * k + j0, min(kSlotBatch, k - j0), E_l, sl);
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)
        if (sl[u] >= 0) atomicAdd(&hist[sl[u]], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E_l; e += 256) chunk[static_cast<int64_t>(blockIdx.x) * E_l + e] = hist[e];
}

__global__ void __launch_bounds__(256) align_scan(int32_t* __restrict__ chunk, int nchunks, int E_l,
                                                  int bm, int32_t* __restrict__ meta,
                                                  int32_t* __restrict__ num_padded,
                                                  int32_t* __restrict__ block_expert) {
  __shared__ int wsum[4];
  int32_t* offsets = meta + 1;
  int32_t* counts = meta + 1 + (E_l + 1);
  const int e = threadIdx.x;
  int run = 0;
  int padded = 0;
  if (e < E_l) {
    // chunk counts in batches: the batch's loads are all issued before its stores, one
    // memory round trip per batch instead of one per chunk
    constexpr int kBatch = 16;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < nchunks ? chunk[static_cast<int64_t>(c0 + j) * E_l + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < nchunks) chunk[static_cast<int64_t>(c0 + j) * E_l + e] = run;
        run += v[j];
      }
    }
    counts[e] = run;
  }
  int nblocks = 0;
  segment(run, bm, padded, nblocks);
  if (e >= E_l) padded = nblocks = 0;
  int acc;
  const int off = wg_exclusive_scan(padded, wsum, acc);
  if (e == 0) {
    offsets[E_l] = acc;
    meta[0] = acc;
    *num_padded = acc;
  }
  if (e < E_l) offsets[e] = off;
  // NULL: no row-block table wanted (the exchange's rank grouping)
  if (block_expert) write_blocks(block_expert, e, E_l, bm, off, padded, nblocks, acc, wsum);
}

__global__ void __launch_bounds__(256) align_scatter(const int32_t* __restrict__ tl, int T, int k,
                                                     int E_l, const int32_t* __restrict__ chunk,
                                                     const int32_t* __restrict__ meta,
                                                     int32_t* __restrict__ sorted_pairs,
                                                     int32_t* __restrict__ pair_row) {
  __shared__ unsigned long long mask[4][256];
  __shared__ int base[256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int32_t* offsets = meta + 1;
  for (int e = tid; e < E_l; e += 256) {
    base[e] = offsets[e] + chunk[static_cast<int64_t>(blockIdx.x) * E_l + e];
    mask[0][e] = mask[1][e] = mask[2][e] = mask[3][e] = 0ull;
  }
  __syncthreads();
  chunk_scatter(tl, T, k, E_l, base, mask, sorted_pairs, pair_row);
}

// Scan and scatter in one pass, for a few chunks (the launch then has two kernels instead of
// three): every workgroup reads all chunks' counts per slot (nchunks x E_l values), takes its
// own chunk base and the padded segment offsets from them, and workgroup 0 writes the
// metadata and the block -> slot table that align_scan writes in the three-pass form.
__global__ void __launch_bounds__(256) align_scan_scatter(const int32_t* __restrict__ tl, int T,
                                                          int k, int E_l, int bm,
                                                          const int32_t* __restrict__ chunk,
                                                          int nchunks, int32_t* __restrict__ meta,
                                                          int32_t* __restrict__ num_padded,
                                                          int32_t* __restrict__ block_expert,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_row) {
  __shared__ unsigned long long mask[4][256];
  __shared__ int base[256];
  __shared__ int wsum[4];
  const int e = threadIdx.x;  // slot of this thread (E_l <= 256)
  const int c = blockIdx.x;
  int pre = 0, tot = 0;
  if (e < E_l) {
    constexpr int kBatch = 16;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < nchunks ? chunk[static_cast<int64_t>(c0 + j) * E_l + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < c) pre += v[j];
        tot += v[j];
      }
    }
    mask[0][e] = mask[1][e] = mask[2][e] = mask[3][e] = 0ull;
  }
  int padded = 0, nblocks = 0;
  segment(tot, bm, padded, nblocks);
  if (e >= E_l) padded = nblocks = 0;
  int acc;
  const int off = wg_exclusive_scan(padded, wsum, acc);
  if (e < E_l) base[e] = off + pre;
  if (c == 0) {
    int32_t* offsets = meta + 1;
    int32_t* counts = meta + 1 + (E_l + 1);
    if (e < E_l) {
      counts[e] = tot;
      offsets[e] = off;
    }
    if (e == 0) {
      offsets[E_l] = acc;
      meta[0] = acc;
      *num_padded = acc;
    }
    if (block_expert) write_blocks(block_expert, e, E_l, bm, off, padded, nblocks, acc, wsum);
  }
  __syncthreads();
  chunk_scatter(tl, T, k, E_l, base, mask, sorted_pairs, pair_row);
}

// All three passes in one workgroup, for T <= kAlignChunk (one chunk): LDS histogram and
// per-wave masks, scan, then the scatter. The -1 fill of the sorted list is ordered before the
// scatter's stores by the barrier (its fence waits for this thread's stores).
__global__ void __launch_bounds__(256) align_single(const int32_t* __restrict__ tl, int T, int k,
                                                    int E_l, int bm, int cap,
                                                    int32_t* __restrict__ meta,
                                                    int32_t* __restrict__ num_padded,
                                                    int32_t* __restrict__ block_expert,
                                                    int32_t* __restrict__ sorted_pairs,
                                                    int32_t* __restrict__ pair_row) {
  __shared__ int hist[256];
  __shared__ int seg[256];
  __shared__ int wsum[4];
  __shared__ unsigned long long mask[4][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  for (int i = tid; i < cap; i += 256) sorted_pairs[i] = -1;
  for (int e = tid; e < E_l; e += 256) {
    hist[e] = 0;
    mask[0][e] = mask[1][e] = mask[2][e] = mask[3][e] = 0ull;
  }
  __syncthreads();
  const bool valid = tid < T;
  if (valid)
    for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
      int sl[kSlotBatch];
      load_slots(tl, static_cast<int64_t>(tid) * k + j0, min(kSlotBatch, k - j0), E_l, sl);
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)
        if (sl[u] >= 0) {
          atomicAdd(&hist[sl[u]], 1);
          atomicOr(&mask[wave][sl[u]], 1ull << lane);
        }
    }
  __syncthreads();
  int32_t* offsets = meta + 1;
  int32_t* counts = meta + 1 + (E_l + 1);
  // E_l <= 256: thread e owns slot e
  int padded = 0, nblocks = 0;
  if (tid < E_l) {
    segment(hist[tid], bm, padded, nblocks);
    counts[tid] = hist[tid];
  }
  int acc;
  const int off = wg_exclusive_scan(padded, wsum, acc);
  if (tid < E_l) {
    seg[tid] = off;
    offsets[tid] = off;
  }
  if (tid == 0) {
    offsets[E_l] = acc;
    meta[0] = acc;
    *num_padded = acc;
  }
  if (block_expert) write_blocks(block_expert, tid, E_l, bm, off, padded, nblocks, acc, wsum);
  __syncthreads();
  if (!valid) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
    int sl[kSlotBatch];
    const int n = min(kSlotBatch, k - j0);
    load_slots(tl, static_cast<int64_t>(tid) * k + j0, n, E_l, sl);
#pragma unroll
    for (int u = 0; u < kSlotBatch; ++u) {
      if (u >= n) break;
      const int64_t pid = static_cast<int64_t>(tid) * k + j0 + u;
      const int s = sl[u];
      if (s < 0) {
        pair_row[pid] = -1;
        continue;
      }
      int before = __popcll(mask[wave][s] & below);
      for (int w = 0; w < wave; ++w) before += __popcll(mask[w][s]);
      const int pos = seg[s] + before;
      sorted_pairs[pos] = static_cast<int32_t>(pid);
      pair_row[pid] = pos;
    }
  }
}

}  // namespace

// Up to this many chunks (T <= 16384) each scatter workgroup scans the counts itself.
constexpr int kFusedScanChunks = 64;

int launch_align(const moe_params& p, int T, const int32_t* topk_local, int block_m,
                 int32_t* sorted_pairs, int32_t* block_expert, int32_t* pair_row,
                 int32_t* num_padded, int32_t* meta, int32_t* chunk, hipStream_t s) {
  const int E_l = p.num_local_experts;
  const int k = p.top_k;
  const int nchunks = align_chunks(T);
  const int cap = T * k + E_l * ((block_m > 0 ? block_m : 32) - 1);
  if (nchunks == 1) {
    return launch(align_single, 1, 256, 0, s, topk_local, T, k, E_l, block_m, cap, meta,
                  num_padded, block_expert, sorted_pairs, pair_row);
  }
  if (int rc = launch(align_count, nchunks, 256, 0, s, topk_local, T, k, E_l, chunk, sorted_pairs,
                      cap))
    return rc;
  if (nchunks <= kFusedScanChunks)
    return launch(align_scan_scatter, nchunks, 256, 0, s, topk_local, T, k, E_l, block_m, chunk,
                  nchunks, meta, num_padded, block_expert, sorted_pairs, pair_row);
  if (int rc = launch(align_scan, 1, 256, 0, s, chunk, nchunks, E_l, block_m, meta, num_padded,
                      block_expert))
    return rc;
  return launch(align_scatter, nchunks, 256, 0, s, topk_local, T, k, E_l, chunk, meta,
                sorted_pairs, pair_row);
}

}  // namespace moe
