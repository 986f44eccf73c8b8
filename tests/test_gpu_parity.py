"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small layers span several tiles with ragged tails and run the oracle on every token; the
five full-size layers compare routing on every token and outputs on >= 512 seeded tokens
that cover every local expert (all tokens where the layer is small). The comparison rules
are those of ``moe_case``.
"""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import oracle
import workloads as wl
from moe_case import (OUT_TOL, Layer, check_routing, dev_tensor, params, reference_routing,
                      rel_err, sample_rows, slot_of_row)

pytestmark = pytest.mark.gpu

W = wl.Workload
SMALL = {
    # fp32, every expert local, rows per expert ~16 (granule 16)
    "tiny_ragged": (W("tiny_ragged", 1, "tiny fp32, ragged T", "f32", (37,), 128, 8, 256, 2, True), 37),
    "tiny": (wl.WORKLOADS["tiny"], 64),
    # bf16 granule 64: 25 rows per expert
    "mix_s": (W("mix_s", 11, "small Mixtral-like", "bf16", (100,), 512, 8, 384, 2, True), 100),
    # EP share of 64 experts, granule 64
    "ep_s": (W("ep_s", 12, "small EP share", "bf16", (300,), 256, 64, 128, 8, True,
               ep_size=4, ep_rank=1), 300),
    # grouped routing, no renormalise, rsf 16, shared expert, H % 128 == 64 (64-row B tiles)
    "ds_s": (W("ds_s", 13, "small grouped", "bf16", (200,), 320, 32, 192, 6, False,
               use_grouped_topk=True, num_expert_group=8, topk_group=3,
               routed_scaling_factor=16.0, ep_size=8, ep_rank=0,
               shared_intermediate_size=384), 200),
    # skewed routing with a shared expert: decode-sized and prefill-sized token counts
    "skew_s1": (W("skew_s", 14, "small skewed", "bf16", (1, 7, 600), 256, 64, 256, 8, True,
                  ep_size=8, ep_rank=0, shared_intermediate_size=256, zipf_bias=1.2), 1),
    "skew_s7": (W("skew_s", 14, "small skewed", "bf16", (1, 7, 600), 256, 64, 256, 8, True,
                  ep_size=8, ep_rank=0, shared_intermediate_size=256, zipf_bias=1.2), 7),
    "skew_s600": (W("skew_s", 14, "small skewed", "bf16", (1, 7, 600), 256, 64, 256, 8, True,
                    ep_size=8, ep_rank=0, shared_intermediate_size=256, zipf_bias=1.2), 600),
    # granule 128: 250 rows per expert, ragged
    "mix_m": (W("mix_m", 15, "medium Mixtral-like", "bf16", (1000,), 256, 8, 256, 2, True), 1000),
    # a single 64-wide K step in the router, gate/up and down GEMMs
    "k64": (W("k64", 16, "one K step", "bf16", (300,), 64, 8, 64, 2, True), 300),
    # odd numbers of K steps (3 and 5) in 256-row tiles with 128- and 64-row weight tiles
    "odd_l": (W("odd_l", 17, "odd K steps, large tiles", "bf16", (2400,), 192, 4, 320, 2, True), 2400),
}


def _full_check(layer: Layer, rows=None, with_shared=True):
    w = layer.w
    out, ids, tw = layer.forward(with_shared=with_shared)
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    if rows is None:
        rows = np.arange(layer.T)
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows], with_shared)
    err = rel_err(out[rows], want)
    print(f"[{w.key} T={layer.T}] rel_err={err:.3e} near_ties={near} exempt_mismatch={mism.size} "
          f"checked_rows={len(rows)}", flush=True)
    assert err <= OUT_TOL[w.dtype], err
    return out, ids, tw


@pytest.mark.parametrize("case", sorted(SMALL))
def test_forward_small(case):
    w, T = SMALL[case]
    _full_check(Layer(w, T))


# moe_forward on variable row blocks (experts of ~300 rows: one block of 288 or 320 rows each
# where the 256 granule needs two) with a shared expert beside them, serial and overlapped
VAR_SHARED = W("var_sh", 18, "variable row blocks with a shared expert", "bf16", (1200, 3000), 256,
               8, 4096, 2, True, shared_intermediate_size=512)


# 1200 tokens: 300 rows per expert, weights streamed (non-temporal hint); 3000: 750, weight tiles
# shared by three row blocks (plain loads)
@pytest.mark.parametrize("T", VAR_SHARED.tokens)
@pytest.mark.parametrize("overlap", [False, True], ids=["serial", "overlap"])
def test_forward_variable_blocks_with_shared(overlap, T):
    w = VAR_SHARED
    p = params(w)
    assert moe.moe_pick_block_m(p, T) == 0, "this layer should take variable row blocks"
    layer = Layer(w, T)
    out, ids, tw = layer.forward()
    if overlap:
        d, dev = layer.d, layer.d["x"].device
        st = torch.cuda.Stream(device=dev)
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(st)
        join.record(st)
        side = moe.make_side_stream(st, fork, join)
        o2 = torch.empty(T, w.hidden_size, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
        moe.moe_forward_overlap(p, side, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"],
                                d["w2"], d["sw13"], d["sw2"], o2, None, None, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o2.float().cpu().numpy(), out)
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = sample_rows(ids, layer.emap, T)
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    err = rel_err(out[rows], layer.oracle_out(rows, ids_ref[rows], w_ref[rows]))
    print(f"[var_sh T={T}] rel_err={err:.3e} rows={len(rows)}", flush=True)
    assert err <= OUT_TOL[w.dtype], err


@pytest.mark.parametrize("case", ["ds_s", "ep_s", "skew_s1"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9, 16])
def test_forward_decode_sizes(case, T):
    """Decode-sized calls (1 to 16 tokens, granule 16, weight-streaming kernels; at 16 tokens on
    the skewed share one expert takes most of them): routing and output vs the oracle on every
    token."""
    w, _ = SMALL[case]
    _full_check(Layer(w, T))

FULL = [(k, T) for k in ("tiny", "mixtral", "ep_share", "dsv2", "skewed")
        for T in wl.WORKLOADS[k].tokens]


@pytest.mark.parametrize("key,T", FULL, ids=[f"{k}-T{T}" for k, T in FULL])
def test_forward_full_size(key, T):
    w = wl.WORKLOADS[key]
    layer = Layer(w, T)
    out, ids, tw = layer.forward()
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = np.arange(T) if T <= 256 else sample_rows(ids, layer.emap, T)
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows])
    err = rel_err(out[rows], want)
    print(f"[{key} T={T}] rel_err={err:.3e} near_ties={near} exempt_mismatch={mism.size} "
          f"rows={len(rows)}", flush=True)
    assert err <= OUT_TOL[w.dtype], err


def test_repeated_calls_bit_identical():
    w, T = SMALL["ep_s"]
    layer = Layer(w, T)
    a = layer.forward()
    b = layer.forward()
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _side(dev):
    """A side stream and a fork / join event pair, the events created (recorded once)."""
    st = torch.cuda.Stream(device=dev)
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    fork.record(st)
    join.record(st)
    return st, fork, join


@pytest.mark.parametrize("overlap", [False, True], ids=["serial", "overlap"])
@pytest.mark.parametrize("case", ["ds_s", "skew_s600"])
def test_concurrent_callers_match_single_thread(case, overlap):
    """Two host threads calling the layer at once, each on its own stream with its own buffers
    (and, with moe_forward_overlap, its own side stream and event pair; the library keeps no
    state that they could share): every call reproduces the single-thread output and routing
    bit for bit."""
    import threading
    w, T = SMALL[case]
    layer = Layer(w, T)
    ref = layer.forward()
    p = params(w)
    d = layer.d
    dev = d["x"].device
    n_threads, n_calls = 2, 6
    bufs = []
    for _ in range(n_threads):
        bufs.append(dict(
            st=torch.cuda.Stream(device=dev),
            out=torch.empty(T, w.hidden_size, dtype=d["x"].dtype, device=dev),
            ids=torch.empty(T, w.top_k, dtype=torch.int32, device=dev),
            tw=torch.empty(T, w.top_k, dtype=torch.float32, device=dev),
            ws=torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev),
            side=moe.make_side_stream(*_side(dev)) if overlap else None))
    torch.cuda.synchronize()
    results = [[] for _ in range(n_threads)]
    errors = []

    def worker(i):
        b = bufs[i]
        try:
            for _ in range(n_calls):
                if overlap:
                    moe.moe_forward_overlap(p, b["side"], T, d["x"], d["gate"], d["bias"],
                                            d["emap"], d["w13"], d["w2"], d["sw13"], d["sw2"],
                                            b["out"], b["ids"], b["tw"], b["ws"], stream=b["st"],
                                            score_bias=d["sbias"])
                else:
                    moe.moe_forward(p, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"],
                                    d["w2"], d["sw13"], d["sw2"], b["out"], b["ids"], b["tw"],
                                    b["ws"], stream=b["st"], score_bias=d["sbias"])
                b["st"].synchronize()
                results[i].append((b["out"].float().cpu().numpy(), b["ids"].cpu().numpy(),
                                   b["tw"].cpu().numpy()))
        except Exception as e:  # re-raised below in the test's thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(n_threads):
        assert len(results[i]) == n_calls
        for got in results[i]:
            for u, v in zip(got, ref):
                assert np.array_equal(u, v)


@pytest.mark.parametrize("case,ep", [("ep_s", 4), ("ds_s", 8), ("skew_s600", 8), ("tiny", 4)])
def test_share_sum_equals_all_local(case, ep):
    """Sum of every disjoint share's output (shared expert on rank 0) = the all-local layer."""
    w0, T = SMALL[case]
    total = None
    for r in range(ep):
        layer = Layer(w0.with_share(ep, r), T)
        out, _, _ = layer.forward()
        total = out.astype(np.float64) if total is None else total + out
    full_w = w0.with_share(1, 0)
    full = Layer(full_w, T)
    ref = full.oracle_route()
    out_full, ids, tw = full.forward()
    mism, _ = full.check_routing(ids, tw, ref)
    ids_ref, w_ref = reference_routing(full_w, ids, ref, mism)
    want = full.oracle_out(np.arange(T), ids_ref, w_ref)
    assert rel_err(total, want) <= OUT_TOL[w0.dtype]
    assert rel_err(total, out_full) <= OUT_TOL[w0.dtype]


def test_share_without_local_pairs():
    """A share that receives no pairs writes zeros, plus the shared expert when it carries it."""
    w0, T = SMALL["skew_s1"]
    layer = Layer(w0, T)
    _, ids, _ = layer.forward()
    used = set(ids.reshape(-1).tolist())
    n = w0.num_experts // 8
    empty = [r for r in range(8) if not used & set(range(r * n, (r + 1) * n))]
    assert empty, "the skewed single token should leave some share without pairs"
    r = empty[-1]
    lone = Layer(w0.with_share(8, r, shared=False), T)
    out, _, _ = lone.forward()
    assert np.all(out == 0.0)
    with_sh = Layer(w0.with_share(8, r, shared=True), T)
    out2, _, _ = with_sh.forward()
    want = oracle.gated_mlp(wl.to_f32(with_sh.x), wl.to_f32(with_sh.sw13), wl.to_f32(with_sh.sw2))
    assert rel_err(out2, want) <= OUT_TOL["bf16"]


@pytest.mark.parametrize("block_m", [0, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("case", ["ds_s", "tiny_ragged", "skew_s600"])
def test_split_entry_points(case, block_m):
    """route -> align_permute -> grouped_mlp (-> shared_mlp) -> combine, any granule (0: the
    variable row blocks, where the shapes allow them)."""
    w, T = SMALL[case]
    if block_m == 0 and not (w.dtype == "bf16" and w.hidden_size % 256 == 0
                             and w.intermediate_size % 128 == 0):
        pytest.skip("variable row blocks need bf16, H % 256 == 0 and 2I % 256 == 0")
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    k, H = w.top_k, w.hidden_size
    ws = torch.empty(moe.moe_workspace_size(p, T, block_m), dtype=torch.uint8, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    local = torch.empty(T, k, dtype=torch.int32, device=dev)
    moe.moe_route(p, T, d["x"], d["gate"], d["bias"], d["emap"], ids, tw, local, ws,
                  score_bias=d["sbias"])
    # the logits sit at the start of the workspace until the next call reuses it
    logits = ws[: T * w.num_experts * 4].view(torch.float32).view(T, w.num_experts).clone()
    cap = moe.moe_sorted_capacity(p, T, block_m)
    sp = torch.full((cap,), 7, dtype=torch.int32, device=dev)
    be = torch.full((moe.block_expert_len(p, T, block_m),), -5, dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, block_m, sp, be, pr, npad, ws)
    torch.cuda.synchronize()
    # alignment is integer work: bit-exact against the oracle on the same topk_local
    a = oracle.align_permute(local.cpu().numpy(), w.num_local_experts, block_m)
    n = int(npad.item())
    assert n == a["num_padded"]
    assert np.array_equal(sp.cpu().numpy()[:n], a["sorted_pairs"])
    nbe = len(a["block_expert"])
    assert np.array_equal(be.cpu().numpy()[:nbe], a["block_expert"])
    assert np.array_equal(pr.cpu().numpy(), a["pair_row"])
    y = torch.empty(cap, H, dtype=d["x"].dtype, device=dev)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, block_m, y, ws)
    sy = None
    if d["sw13"] is not None:
        sy = torch.empty(T, H, dtype=d["x"].dtype, device=dev)
        moe.moe_shared_mlp(p, T, d["x"], d["sw13"], d["sw2"], sy, ws)
    out = torch.empty(T, H, dtype=d["x"].dtype, device=dev)
    moe.moe_combine(p, T, y, pr, tw, sy, out)
    torch.cuda.synchronize()
    ids_h, tw_h = ids.cpu().numpy(), tw.cpu().numpy()
    ref = layer.oracle_route()
    mism, _ = check_routing(w, ids_h, tw_h, ref, logits.cpu().numpy(), layer.x, layer.gate,
                            layer.bias, label=f"split {case} block_m={block_m}")
    ids_ref, w_ref = reference_routing(w, ids_h, ref, mism)
    want = layer.oracle_out(np.arange(T), ids_ref, w_ref)
    assert rel_err(out.float().cpu().numpy(), want) <= OUT_TOL[w.dtype]
    # y rows of a few pairs against the oracle's expert MLP
    y_h = y.float().cpu().numpy()
    rows = [r for r in range(n) if a["sorted_pairs"][r] >= 0][:: max(1, n // 16)]
    for r in rows:
        pid = a["sorted_pairs"][r]
        s = slot_of_row(a["block_expert"], r, block_m)
        want_y = oracle.gated_mlp(wl.to_f32(layer.x[pid // k])[None], wl.to_f32(layer.w13[s]),
                                  wl.to_f32(layer.w2[s]))[0]
        assert rel_err(y_h[r], want_y) <= OUT_TOL[w.dtype] * 2


def test_external_routing_through_align():
    """Caller-provided slots (external routing) go through align + MLP + combine."""
    w, T = SMALL["mix_s"]
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    k = w.top_k
    r = layer.oracle_route()
    local = dev_tensor(layer.emap[r["ids"]].astype(np.int32))
    tw = dev_tensor(r["weights"])
    bm = 64
    ws = torch.empty(moe.moe_workspace_size(p, T, bm), dtype=torch.uint8, device=dev)
    cap = moe.moe_sorted_capacity(p, T, bm)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p, T, bm), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, bm, sp, be, pr, npad, ws)
    y = torch.empty(cap, w.hidden_size, dtype=d["x"].dtype, device=dev)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, bm, y, ws)
    out = torch.empty(T, w.hidden_size, dtype=d["x"].dtype, device=dev)
    moe.moe_combine(p, T, y, pr, tw, None, out)
    torch.cuda.synchronize()
    want = layer.oracle_out(np.arange(T), r["ids"], r["weights"])
    assert rel_err(out.float().cpu().numpy(), want) <= OUT_TOL["bf16"]


# Routings whose tile counts leave a short last round (at most a quarter of the CUs' worth of
# tiles), so the expert GEMMs hand the tail to the quarter-tile launch. (H, I, top_k, rows per
# local expert, block_m) and the tiles expected on a 256-CU MI355X:
TAIL = {
    # gate/up 256x256 tiles: 9 row blocks x 64 -> 576 tiles, 64 in the tail
    "gu_256x256": (256, 8192, 2, (513, 512, 512, 257), 256),
    # gate/up 128x256 tiles: 17 row blocks x 64 -> 1088 tiles, 64 in the tail
    "gu_128x256": (256, 8192, 2, (513, 513, 512, 258), 128),
    # gate/up 256x128 tiles: 17 row blocks x 32 -> 544 tiles, 32 in the tail
    "gu_256x128": (256, 2048, 1, (1025, 1024, 1024, 1024), 256),
    # down 256x256 tiles: 17 x 32 -> 544, 32 in the tail
    "dn_256x256": (8192, 256, 1, (1025, 1024, 1024, 1024), 256),
    # down 128x256 tiles: 33 x 32 -> 1056, 32 in the tail
    "dn_128x256": (8192, 256, 1, (1025, 1024, 1024, 1024), 128),
    # down 256x128 tiles (H = 33 x 128): 17 x 33 -> 561, 49 in the tail
    "dn_256x128": (4224, 256, 1, (1025, 1024, 1024, 1024), 256),
    # down 128x128 tiles: 32 x 33 -> 1056, 32 in the tail
    "dn_128x128": (4224, 256, 1, (1025, 1024, 1024, 896), 128),
}


@pytest.mark.parametrize("case", sorted(TAIL))
def test_tail_tiles(case):
    """Expert GEMMs whose last round is split into quarter tiles: every output row vs the oracle."""
    H, I, k, counts, bm = TAIL[case]
    E = len(counts)
    T = sum(counts) // k
    w = W(f"tail_{case}", 30 + sorted(TAIL).index(case), "tail tiles", "bf16", (T,), H, E, I, k,
          True)
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    # external routing with exactly `counts` pairs per expert, distinct experts per token
    flat = np.repeat(np.arange(E, dtype=np.int32), counts)
    ids = np.stack([flat[j * T:(j + 1) * T] for j in range(k)], axis=1)
    assert all(len(set(r)) == k for r in ids.tolist())
    rng = np.random.default_rng(7)
    tw_h = rng.uniform(0.25, 1.0, size=(T, k)).astype(np.float32)
    local = dev_tensor(ids)
    tw = dev_tensor(tw_h)
    ws = torch.empty(moe.moe_workspace_size(p, T, bm), dtype=torch.uint8, device=dev)
    cap = moe.moe_sorted_capacity(p, T, bm)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p, T, bm), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, bm, sp, be, pr, npad, ws)
    y = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, bm, y, ws)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    moe.moe_combine(p, T, y, pr, tw, None, out)
    torch.cuda.synchronize()
    blocks = sum((c + bm - 1) // bm for c in counts)
    assert int(npad.item()) == blocks * bm
    want = layer.oracle_out(np.arange(T), ids, tw_h)
    err = rel_err(out.float().cpu().numpy(), want)
    print(f"[{case}] T={T} row_blocks={blocks} rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL["bf16"], err


@pytest.mark.parametrize("T,E_l,block_m", [(257, 64, 256), (16384, 64, 256), (16385, 64, 128),
                                           (16385, 8, 16), (4000, 256, 16), (200, 64, 0),
                                           (16384, 64, 0), (16385, 256, 0)])
def test_align_chunk_counts(T, E_l, block_m):
    """moe_align_permute bit for bit against the oracle on both sides of the chunk count (64
    chunks of 256 tokens) up to which each scatter workgroup scans the counts itself; seeded
    slot lists with non-local (-1) entries."""
    k = 8
    rng = np.random.default_rng(T + E_l)
    local = np.stack([rng.permutation(E_l + 16)[:k] for _ in range(T)]).astype(np.int32)
    local[local >= E_l] = -1
    w = W("align_chunks", 70, "align sizes", "bf16", (T,), 256, E_l, 128, k, True)
    p = params(w)
    dev = torch.device("cuda:0")
    ws = torch.empty(moe.moe_workspace_size(p, T, block_m), dtype=torch.uint8, device=dev)
    cap = moe.moe_sorted_capacity(p, T, block_m)
    sp = torch.full((cap,), 7, dtype=torch.int32, device=dev)
    be = torch.full((moe.block_expert_len(p, T, block_m),), -5, dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, dev_tensor(local), block_m, sp, be, pr, npad, ws)
    torch.cuda.synchronize()
    a = oracle.align_permute(local, E_l, block_m)
    n = int(npad.item())
    assert n == a["num_padded"]
    assert np.array_equal(sp.cpu().numpy()[:n], a["sorted_pairs"])
    assert np.all(sp.cpu().numpy()[n:] == -1)
    nbe = len(a["block_expert"])
    assert np.array_equal(be.cpu().numpy()[:nbe], a["block_expert"])
    assert np.array_equal(pr.cpu().numpy(), a["pair_row"])


# Experts whose last row block holds 1, 17, 31, 32, 33 or 44 real rows (the gate/up tiles skip
# the MFMAs of their padding-only 32-row groups), at gate/up widths whose tiles are 256 wide
# (I = 128) or 128 wide (I = 192), with an even and an odd number of K steps.
# (H, I, activation, expert-bias std)
SPARSE = {
    "silu_w256": (256, 128, "silu", 0.0),
    "silu_w128": (320, 192, "silu", 0.0),
    "oai_bias_w256": (320, 128, "swigluoai", 1.0),
    "oai_bias_w128": (256, 192, "swigluoai", 1.0),
}


@pytest.mark.parametrize("bm", [256, 0])
@pytest.mark.parametrize("case", sorted(SPARSE))
def test_sparse_last_blocks(case, bm):
    """Nearly empty last row blocks of the sorted gate/up (granule 256), and the same counts as
    variable row blocks (granule 0: blocks of 288, 320, 256 and 64 rows where the shapes allow
    them): every token's output vs the oracle."""
    H, I, act, bstd = SPARSE[case]
    if bm == 0 and not (H % 256 == 0 and I % 128 == 0):
        pytest.skip("variable row blocks need H % 256 == 0 and 2I % 256 == 0")
    counts = (257, 273, 287, 288, 289, 256, 300, 40)
    k = 2
    E = len(counts)
    T = sum(counts) // k
    w = W(f"sparse_{case}", 60 + sorted(SPARSE).index(case), "sparse last blocks", "bf16", (T,),
          H, E, I, k, True, activation=act, expert_bias_std=bstd)
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    flat = np.repeat(np.arange(E, dtype=np.int32), counts)
    ids = np.stack([flat[j * T:(j + 1) * T] for j in range(k)], axis=1)
    assert all(len(set(r)) == k for r in ids.tolist())
    rng = np.random.default_rng(11)
    tw_h = rng.uniform(0.25, 1.0, size=(T, k)).astype(np.float32)
    local = dev_tensor(ids)
    tw = dev_tensor(tw_h)
    ws = torch.empty(moe.moe_workspace_size(p, T, bm), dtype=torch.uint8, device=dev)
    cap = moe.moe_sorted_capacity(p, T, bm)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p, T, bm), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, bm, sp, be, pr, npad, ws)
    y = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, bm, y, ws, b13=d["b13"],
                        b2=d["b2"])
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    moe.moe_combine(p, T, y, pr, tw, None, out)
    torch.cuda.synchronize()
    want = layer.oracle_out(np.arange(T), ids, tw_h, with_shared=False)
    err = rel_err(out.float().cpu().numpy(), want)
    print(f"[sparse {case}] T={T} rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL["bf16"], err


@pytest.mark.parametrize("overlap", [False, True], ids=["serial", "overlap"])
@pytest.mark.parametrize("case", ["ds_s", "skew_s1", "mix_m"])
def test_graph_replay_matches_eager(case, overlap):
    """moe_forward (or moe_forward_overlap, whose side stream forks and joins inside the capture)
    captured in a HIP graph: every replay, with eager work and host syncs in between,
    reproduces the eager output and routing bit for bit."""
    w, T = SMALL[case]
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    out = torch.empty(T, w.hidden_size, dtype=d["x"].dtype, device=dev)
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, w.top_k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)

    side = moe.make_side_stream(*_side(dev)) if overlap else None

    def call():
        if overlap:
            moe.moe_forward_overlap(p, side, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"],
                                    d["w2"], d["sw13"], d["sw2"], out, ids, tw, ws,
                                    score_bias=d["sbias"])
        else:
            moe.moe_forward(p, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"], d["w2"],
                            d["sw13"], d["sw2"], out, ids, tw, ws, score_bias=d["sbias"])

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), ids.clone(), tw.clone())
    if overlap:  # the overlapped layer equals the serial one
        serial = layer.forward()
        assert np.array_equal(out.float().cpu().numpy(), serial[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(4):
        out.zero_()
        ids.zero_()
        ws.zero_()  # the replay must not rely on workspace contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(ids, ref[1]) and torch.equal(tw, ref[2]), r
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), r


# Largest parameters the kernels take: 256 experts, all local (E_l = 256: the alignment's
# one-slot-per-thread tables), top-64 (one wave's ballot in the top-k and the combine), plain
# and grouped.
MAXED = {
    "e256_k64": (W("e256_k64", 41, "E 256, top-64, all local", "bf16", (300,), 128, 256, 64, 64,
                   True), 300),
    "e256_k64_grp": (W("e256_k64_grp", 42, "E 256, top-64, grouped", "bf16", (90,), 128, 256, 64,
                       64, False, use_grouped_topk=True, num_expert_group=64, topk_group=32,
                       routed_scaling_factor=2.0), 90),
    "e256_k1": (W("e256_k1", 43, "E 256, top-1", "bf16", (1000,), 256, 256, 64, 1, True,
                  ep_size=2, ep_rank=1), 1000),
}


@pytest.mark.parametrize("case", sorted(MAXED))
def test_forward_largest_parameters(case):
    w, T = MAXED[case]
    _full_check(Layer(w, T))


@pytest.mark.parametrize("ep", [1, 4, 256])
def test_exchange_largest_parameters(ep):
    """The exchange at top-64 over 256 experts: dispatch bit for bit against the oracle."""
    from test_gpu_exchange import _check_dispatch
    w, T = MAXED["e256_k64"]
    rng = np.random.default_rng(44)
    ids = np.argsort(rng.random((T, 256)), axis=1)[:, :64].astype(np.int32)
    tw = rng.random((T, 64)).astype(np.float32)
    _check_dispatch(w, T, ep, ids, tw, dev_tensor(wl.x(w, T)))


@pytest.mark.parametrize("case", ["ds_s", "skew_s7", "e256_k64"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5])
def test_decode_forward_equals_split_path(case, T):
    """Decode-sized moe_forward (shared expert on the side stream) equals, bit for bit, the
    split entry points (route -> align_permute -> grouped MLP -> shared MLP -> combine) at the
    same granule."""
    w, _ = {**SMALL, **MAXED}[case]
    layer = Layer(w, T)
    out_f, ids_f, tw_f = layer.forward()
    p = params(w)
    d = layer.d
    dev = d["x"].device
    k, H = w.top_k, w.hidden_size
    bm = moe.moe_pick_block_m(p, T)
    ws = torch.empty(moe.moe_workspace_size(p, T, bm), dtype=torch.uint8, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    local = torch.empty(T, k, dtype=torch.int32, device=dev)
    moe.moe_route(p, T, d["x"], d["gate"], d["bias"], d["emap"], ids, tw, local, ws,
                  score_bias=d["sbias"])
    cap = moe.moe_sorted_capacity(p, T, bm)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p, T, bm), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, bm, sp, be, pr, npad, ws)
    y = torch.empty(cap, H, dtype=d["x"].dtype, device=dev)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, bm, y, ws)
    sy = None
    if d["sw13"] is not None:
        sy = torch.empty(T, H, dtype=d["x"].dtype, device=dev)
        moe.moe_shared_mlp(p, T, d["x"], d["sw13"], d["sw2"], sy, ws)
    out = torch.empty(T, H, dtype=d["x"].dtype, device=dev)
    moe.moe_combine(p, T, y, pr, tw, sy, out)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_f) and np.array_equal(tw.cpu().numpy(), tw_f)
    assert np.array_equal(out.float().cpu().numpy(), out_f)
