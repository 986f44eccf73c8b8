// Expert-parallel exchange around the share's MoE path (gfx950): the dispatch plan and send
// buffers before it, the unpack of the returned rows after it.
//
// "ep_fused_moe_patch.py", _ep_forward Step 2: the destination rank of pair (t, j) is
// topk_ids[t, j] / (E / ep_size) (contiguous expert shares); work items are grouped by
// destination rank so that each rank's part of the all-to-all is contiguous. Step 4: the
// rows come back in the same order and are summed per token. Here a token travels to each
// of its destination ranks once: its first slot that goes to rank r owns the row, the others
// ride along (the receiving rank applies every one of its experts the token picked, through
// the k local slots that the send row carries). Ordering and counts come from the alignment
// passes (keyed by rank instead of local expert, granule 1), so the rows of a rank follow
// increasing token index without a sort; the pack then reads each token's hidden row once.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// Rank of the row that pair (t, j) owns, or -1 when an earlier slot of t goes to the same
// rank (or the id is out of range). One thread per pair; k <= 64.
__global__ void __launch_bounds__(256) ep_owner_rank(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                     int k, int E, int per,
                                                     int32_t* __restrict__ rank_of) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_pairs) return;
  const int64_t base = i - i % k;
  const int j = static_cast<int>(i - base);
  const int id = ids[i];
  int r = (id >= 0 && id < E) ? id / per : -1;
  for (int jj = 0; jj < j && r >= 0; ++jj) {
    const int o = ids[base + jj];
    if (o >= 0 && o < E && o / per == r) r = -1;
  }
  rank_of[i] = r;
}

// The send rows of token t (one workgroup per token): its owned slots are compacted in slot
// order into LDS (k <= 64: one wave's ballot), the hidden row is read once and written to each
// of them, then each row gets the token's k routing weights and its k slots seen from the
// row's rank (the local expert index there, else -1).
__global__ void __launch_bounds__(256) ep_pack(const int32_t* __restrict__ send_pos, int k, int E,
                                               int per, const uint4* __restrict__ x, int row_vec,
                                               const int32_t* __restrict__ ids,
                                               const float* __restrict__ w,
                                               int32_t* __restrict__ send_token,
                                               uint4* __restrict__ send_x,
                                               int32_t* __restrict__ send_local,
                                               float* __restrict__ send_w) {
  __shared__ int s_row[64];
  __shared__ int s_base[64];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int64_t pbase = static_cast<int64_t>(t) * k;
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const int row = j < k ? send_pos[pbase + j] : -1;
    const unsigned long long m = __ballot(row >= 0);
    if (row >= 0) {
      const int at = __popcll(m & ((1ull << j) - 1ull));
      s_row[at] = row;
      s_base[at] = (ids[pbase + j] / per) * per;  // first global expert of the row's rank
    }
    if (j == 0) s_n = __popcll(m);
  }
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const uint4* src = x + static_cast<int64_t>(t) * row_vec;
  for (int v = threadIdx.x; v < row_vec; v += 256) {
    const uint4 q = src[v];
    for (int i = 0; i < n; ++i) send_x[static_cast<int64_t>(s_row[i]) * row_vec + v] = q;
  }
  for (int e = threadIdx.x; e < n * k; e += 256) {
    const int i = e / k;
    const int j = e - i * k;
    const int64_t o = static_cast<int64_t>(s_row[i]) * k + j;
    const int id = ids[pbase + j];
    const int l = id - s_base[i];
    send_local[o] = (id >= 0 && id < E && l >= 0 && l < per) ? l : -1;
    send_w[o] = w[pbase + j];
  }
  if (threadIdx.x < n) send_token[s_row[threadIdx.x]] = t;
}

}  // namespace

int launch_ep_dispatch(const moe_params& p, int T, int ep_size, const int32_t* ids, const float* w,
                       const void* x, int32_t* send_pos, int32_t* rank_meta, int32_t* send_token,
                       void* send_x, int32_t* send_local, float* send_w, const EpScratch& ws,
                       hipStream_t s) {
  const int k = p.top_k;
  const int E = p.num_experts;
  const int per = E / ep_size;
  const int64_t n_pairs = static_cast<int64_t>(T) * k;
  if (int rc = launch(ep_owner_rank, static_cast<int>((n_pairs + 255) / 256), 256, 0, s, ids,
                      n_pairs, k, E, per, ws.rank_of))
    return rc;
  // rows grouped by rank, increasing pair (= token) index inside a rank, no padding
  moe_params pr = p;
  pr.num_local_experts = ep_size;
  int rc = launch_align(pr, T, ws.rank_of, 1, ws.sorted_pairs, nullptr, send_pos, rank_meta,
                        rank_meta, ws.chunk, s);
  if (rc) return rc;
  const int elt = p.dtype == MOE_F32 ? 4 : 2;
  return launch(ep_pack, T, 256, 0, s, send_pos, k, E, per, static_cast<const uint4*>(x),
                p.hidden_size * elt / 16, ids, w, send_token, static_cast<uint4*>(send_x),
                send_local, send_w);
}

}  // namespace moe
