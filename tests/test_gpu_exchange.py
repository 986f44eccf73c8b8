"""GPU parity of the expert-parallel exchange (dispatch plan, send buffers, combine unpack)
against the oracle, and the exchange wrapped around the share path on one GPU.

The dispatch is integer and byte work: send_pos, the rank offsets and counts, send_token,
send_local, send_w and send_x are compared bit for bit. The combine sums rows in fp32 and
rounds once, so it is held to the output tolerance of ``moe_case``. The end-to-end case runs
every rank's share on the rows the dispatch sent it and compares the unpacked result with the
oracle's layer on the same routing.
"""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import oracle
import workloads as wl
from moe_case import OUT_TOL, Layer, dev_tensor, params, rel_err, torch_dtype

pytestmark = pytest.mark.gpu

W = wl.Workload


def _random_ids(seed, T, E, k, invalid=0.0):
    """Seeded routing: k distinct experts per token; a fraction of slots set to -1."""
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if invalid:
        ids[rng.random((T, k)) < invalid] = -1
    return ids


def _dispatch(w, T, ep, ids, tw, x):
    """moe_ep_dispatch on device tensors; returns the outputs as device tensors."""
    p = params(w)
    dev = x.device
    k, H = w.top_k, w.hidden_size
    R = moe.moe_ep_send_capacity(p, T, ep)
    assert R == T * min(k, ep)
    out = {
        "send_pos": torch.full((T * k,), 99, dtype=torch.int32, device=dev),
        "rank_meta": torch.full((2 * ep + 2,), 99, dtype=torch.int32, device=dev),
        "send_token": torch.full((max(R, 1),), 99, dtype=torch.int32, device=dev),
        "send_x": torch.zeros(max(R, 1), H, dtype=x.dtype, device=dev),
        "send_local": torch.full((max(R, 1), k), 99, dtype=torch.int32, device=dev),
        "send_w": torch.zeros(max(R, 1), k, dtype=torch.float32, device=dev),
    }
    ws = torch.empty(max(moe.moe_ep_workspace_size(p, T, ep), 1), dtype=torch.uint8, device=dev)
    moe.moe_ep_dispatch(p, T, ep, ids, tw, x, out["send_pos"], out["rank_meta"], out["send_token"],
                        out["send_x"], out["send_local"], out["send_w"], ws)
    torch.cuda.synchronize()
    return out


def _check_dispatch(w, T, ep, ids_h, tw_h, x_d, ids_d=None, tw_d=None):
    """Every dispatch output bit for bit against oracle.ep_dispatch / ep_pack."""
    k = w.top_k
    ids_d = dev_tensor(ids_h) if ids_d is None else ids_d
    tw_d = dev_tensor(tw_h) if tw_d is None else tw_d
    got = _dispatch(w, T, ep, ids_d, tw_d, x_d)
    plan = oracle.ep_dispatch(ids_h, k, w.num_experts, ep)
    # the oracle's pack is only asked for the slot and weight columns; the hidden rows are
    # compared by gathering x on the device with the oracle's send_token
    pk = oracle.ep_pack(plan, np.zeros((T, 1), np.float32), ids_h, tw_h, k, w.num_experts, ep)
    meta = got["rank_meta"].cpu().numpy()
    n = plan["n_send"]
    assert meta[0] == n
    assert np.array_equal(meta[1:ep + 2], plan["offsets"])
    assert np.array_equal(meta[ep + 2:2 * ep + 2], plan["counts"])
    assert np.array_equal(got["send_pos"].cpu().numpy(), plan["send_pos"])
    assert np.array_equal(got["send_token"].cpu().numpy()[:n], plan["send_token"])
    assert np.array_equal(got["send_local"].cpu().numpy()[:n], pk["send_local"])
    assert np.array_equal(got["send_w"].cpu().numpy()[:n], pk["send_w"])
    tok = torch.from_numpy(plan["send_token"].astype(np.int64)).to(x_d.device)
    assert torch.equal(got["send_x"][:n], x_d[tok])
    print(f"[dispatch T={T} E={w.num_experts} k={k} ep={ep}] n_send={n} "
          f"counts={plan['counts'].tolist()[:8]}", flush=True)
    return got, plan


SMALL = {
    # (workload, T, ep): multi-chunk (T > 256) and single-chunk alignment, k = 1, ep = 1, ep = E
    "ep_s_r4": (W("ep_s", 12, "small EP layer", "bf16", (300,), 256, 64, 128, 8, True), 300, 4),
    "ep_s_r64": (W("ep_s", 12, "small EP layer", "bf16", (300,), 256, 64, 128, 8, True), 300, 64),
    "ep_s_r1": (W("ep_s", 12, "small EP layer", "bf16", (300,), 256, 64, 128, 8, True), 300, 1),
    "tiny_f32_r8": (W("tiny_ragged", 1, "tiny fp32", "f32", (37,), 128, 8, 256, 2, True), 37, 8),
    "k1_r4": (W("k1", 18, "top-1", "bf16", (777,), 192, 16, 128, 1, True), 777, 4),
    "dsv2_s_r8": (W("ds_s", 13, "small grouped", "bf16", (1000,), 320, 32, 192, 6, False,
                    use_grouped_topk=True, num_expert_group=8, topk_group=3,
                    routed_scaling_factor=16.0), 1000, 8),
    "decode_r8": (W("dec", 19, "decode", "bf16", (3,), 256, 64, 128, 8, True), 3, 8),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_ep_dispatch_small(case):
    w, T, ep = SMALL[case]
    ids = _random_ids(w.cid, T, w.num_experts, w.top_k)
    tw = np.random.default_rng(w.cid + 1).random((T, w.top_k)).astype(np.float32)
    _check_dispatch(w, T, ep, ids, tw, dev_tensor(wl.x(w, T)))


def test_ep_dispatch_invalid_ids_not_sent():
    """Slots with ids outside [0, E) own no row and do not block a later slot's row."""
    w, T, ep = SMALL["ep_s_r4"]
    ids = _random_ids(7, T, w.num_experts, w.top_k, invalid=0.3)
    ids[::7, :] = -1  # tokens with nothing to send
    ids[1::11, 0] = w.num_experts + 5
    tw = np.random.default_rng(8).random((T, w.top_k)).astype(np.float32)
    _, plan = _check_dispatch(w, T, ep, ids, tw, dev_tensor(wl.x(w, T)))
    assert np.all(plan["send_pos"].reshape(T, -1)[::7] == -1)


FULL = [("ep_share", 8192, 4), ("dsv2", 4096, 8), ("skewed", 16384, 8), ("mixtral", 4096, 8),
        ("skewed", 1, 8)]


@pytest.mark.parametrize("key,T,ep", FULL, ids=[f"{k}-T{T}-ep{e}" for k, T, e in FULL])
def test_ep_dispatch_full_size(key, T, ep):
    """Dispatch on the routing moe_route produces for the full-size layers (Zipf-skewed where
    the layer is), every output bit for bit."""
    w = wl.WORKLOADS[key]
    p = params(w)
    x = dev_tensor(wl.x(w, T))
    gate = dev_tensor(wl.gate(w))
    b = wl.logit_bias(w)
    bias = None if b is None else dev_tensor(b)
    emap = dev_tensor(wl.expert_map(w))
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=x.device)
    tw = torch.empty(T, w.top_k, dtype=torch.float32, device=x.device)
    local = torch.empty_like(ids)
    ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=x.device)
    moe.moe_route(p, T, x, gate, bias, emap, ids, tw, local, ws)
    torch.cuda.synchronize()
    _check_dispatch(w, T, ep, ids.cpu().numpy(), tw.cpu().numpy(), x, ids, tw)


@pytest.mark.parametrize("case", ["ep_s_r4", "tiny_f32_r8", "k1_r4", "decode_r8"])
def test_ep_combine_small(case):
    """Unpack of seeded returned rows against the oracle's fp64 per-token sum."""
    w, T, ep = SMALL[case]
    ids = _random_ids(w.cid + 2, T, w.num_experts, w.top_k, invalid=0.1)
    plan = oracle.ep_dispatch(ids, w.top_k, w.num_experts, ep)
    n = plan["n_send"]
    recv = wl.normal_rows((w.cid, 90, 1), np.arange(n), w.hidden_size, dtype=w.dtype)
    dev = torch.device("cuda")
    out = torch.full((T, w.hidden_size), 7.0, dtype=torch_dtype(w), device=dev)
    recv_d = dev_tensor(recv) if n else torch.empty(1, w.hidden_size, dtype=out.dtype, device=dev)
    moe.moe_ep_combine(params(w), T, dev_tensor(plan["send_pos"]), recv_d, out)
    torch.cuda.synchronize()
    want = oracle.ep_combine(plan, wl.to_f32(recv), w.top_k)
    got = out.float().cpu().numpy()
    assert np.all(got[np.all(plan["send_pos"].reshape(T, -1) < 0, axis=1)] == 0.0)
    # fp32 accumulation over at most k rows, one rounding to the output dtype
    tol = 2.0 ** -8 if w.dtype == "bf16" else 1e-6
    assert rel_err(got, want) <= tol


E2E = [("ep_s", 4), ("ep_s", 16), ("ds_s", 8), ("tiny", 4), ("skew_s600", 8), ("skew_s7", 8)]


@pytest.mark.parametrize("case,ep", E2E, ids=[f"{c}-ep{e}" for c, e in E2E])
def test_ep_exchange_around_shares(case, ep):
    """dispatch -> each rank's share path on its received rows (align by send_local, expert
    MLPs, combine with send_w) -> unpack: equals the all-local layer on the same routing."""
    from test_gpu_parity import SMALL as LAYERS
    w0, T = LAYERS[case]
    full = Layer(w0.with_share(1, 0), T)
    ids_h, tw_h, _ = full.gpu_route()
    d = full.d
    dev = d["x"].device
    k, H = w0.top_k, w0.hidden_size
    got = _dispatch(full.w, T, ep, dev_tensor(ids_h), dev_tensor(tw_h), d["x"])
    meta = got["rank_meta"].cpu().numpy()
    n_send = int(meta[0])
    offs = meta[1:ep + 2]
    recv_y = torch.empty(max(n_send, 1), H, dtype=d["x"].dtype, device=dev)
    for r in range(ep):
        lo, n = int(offs[r]), int(offs[r + 1] - offs[r])
        if n == 0:
            continue
        share = Layer(w0.with_share(ep, r, shared=False), 1)
        p = params(share.w)
        bm = moe.moe_pick_block_m(p, n)
        ws = torch.empty(moe.moe_workspace_size(p, n, bm), dtype=torch.uint8, device=dev)
        cap = moe.moe_sorted_capacity(p, n, bm)
        sp = torch.empty(cap, dtype=torch.int32, device=dev)
        be = torch.empty(moe.block_expert_len(p, n, bm), dtype=torch.int32, device=dev)
        pr = torch.empty(n * k, dtype=torch.int32, device=dev)
        npad = torch.empty(1, dtype=torch.int32, device=dev)
        xs = got["send_x"][lo:lo + n]
        moe.moe_align_permute(p, n, got["send_local"][lo:lo + n], bm, sp, be, pr, npad, ws)
        y = torch.empty(cap, H, dtype=d["x"].dtype, device=dev)
        moe.moe_grouped_mlp(p, n, xs, share.d["w13"], share.d["w2"], sp, be, npad, bm, y, ws)
        moe.moe_combine(p, n, y, pr, got["send_w"][lo:lo + n], None, recv_y[lo:lo + n])
    out = torch.full((T, H), 3.0, dtype=d["x"].dtype, device=dev)
    moe.moe_ep_combine(params(full.w), T, got["send_pos"], recv_y, out)
    torch.cuda.synchronize()
    want = full.oracle_out(np.arange(T), ids_h, tw_h, with_shared=False)
    err = rel_err(out.float().cpu().numpy(), want)
    print(f"[exchange {case} T={T} ep={ep}] n_send={n_send} rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[w0.dtype]
    # and the exchange agrees with the all-local forward to the same bar
    out_local, ids_l, tw_l = full.forward(with_shared=False)
    assert np.array_equal(ids_l, ids_h) and np.array_equal(tw_l, tw_h)
    assert rel_err(out.float().cpu().numpy(), out_local) <= OUT_TOL[w0.dtype]


def test_exchange_graph_replay_matches_eager():
    """Dispatch and unpack captured in a HIP graph: every replay, with eager work between the
    replays, reproduces the eager outputs bit for bit."""
    w, T, ep = SMALL["ep_s_r4"]
    ids = _random_ids(61, T, w.num_experts, w.top_k)
    tw = np.random.default_rng(62).random((T, w.top_k)).astype(np.float32)
    p = params(w)
    x = dev_tensor(wl.x(w, T))
    ids_d, tw_d = dev_tensor(ids), dev_tensor(tw)
    ref = _dispatch(w, T, ep, ids_d, tw_d, x)
    R = moe.moe_ep_send_capacity(p, T, ep)
    bufs = {kk: torch.empty_like(v) for kk, v in ref.items()}
    ws = torch.empty(moe.moe_ep_workspace_size(p, T, ep), dtype=torch.uint8, device=x.device)
    out = torch.empty(T, w.hidden_size, dtype=x.dtype, device=x.device)
    out_ref = torch.empty_like(out)
    moe.moe_ep_combine(p, T, ref["send_pos"], ref["send_x"], out_ref)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            moe.moe_ep_dispatch(p, T, ep, ids_d, tw_d, x, bufs["send_pos"], bufs["rank_meta"],
                                bufs["send_token"], bufs["send_x"], bufs["send_local"],
                                bufs["send_w"], ws, stream=s)
            moe.moe_ep_combine(p, T, bufs["send_pos"], bufs["send_x"], out, stream=s)
    n = int(ref["rank_meta"][0].item())
    assert n <= R
    for rep in range(3):
        for v in bufs.values():
            v.fill_(0)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["send_pos"], ref["send_pos"])
        assert torch.equal(bufs["rank_meta"], ref["rank_meta"])
        for kk in ("send_token", "send_x", "send_local", "send_w"):
            assert torch.equal(bufs[kk][:n], ref[kk][:n]), (rep, kk)
        assert torch.equal(out, out_ref)
        _ = (x.float() * 2).sum().item()  # eager work between the replays
