"""GPU parity of replicated experts (expert-parallel load balancing) against the oracle.

The replica choice is integer work: each pair's local slot is compared bit for bit with
``oracle.eplb_local_slots`` on the GPU's own routing. The layer outputs of every share of a
replicated placement sum to the all-local layer, checked against the oracle and against
``moe_forward`` with the tolerance of ``moe_case``. The identity placement gives
``moe_forward``'s output bit for bit.
"""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import oracle
import workloads as wl
from moe_case import OUT_TOL, Layer, dev_tensor, params, rel_err, torch_dtype
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _physical_weights(w, p2l_share):
    """w13 [n, 2I, H], w2 [n, H, I] of the share's physical experts (copies of logical ones)."""
    pairs = [wl.expert_weights(w, int(e)) for e in p2l_share]
    return np.stack([a for a, _ in pairs]), np.stack([b for _, b in pairs])


def _share_map(P, ep, r):
    m = np.full(P, -1, np.int32)
    per = P // ep
    m[r * per:(r + 1) * per] = np.arange(per)
    return m


def _tables(E, p2l):
    l2p, cnt = moe.moe_eplb_tables(E, p2l)
    want_l2p, want_cnt = oracle.eplb_tables(p2l, E)
    assert np.array_equal(cnt, want_cnt)
    assert np.array_equal(l2p[:, :want_l2p.shape[1]], want_l2p)
    return l2p, cnt


CASES = [("ep_s", 4, 8), ("ds_s", 8, 8), ("skew_s600", 8, 8), ("tiny", 2, 4), ("skew_s7", 8, 16),
         ("mix_m", 1, 4)]


@pytest.mark.parametrize("case,ep,extra", CASES, ids=[f"{c}-ep{e}-r{x}" for c, e, x in CASES])
def test_eplb_shares_sum_to_layer(case, ep, extra):
    """Placement with `extra` redundant replicas of the most-loaded experts: every share's
    local slots bit for bit vs the oracle, and the shares' outputs sum to the layer."""
    w0, T = SMALL[case]
    full = Layer(w0.with_share(1, 0), T)
    ids_h, tw_h, _ = full.gpu_route()
    E, k = w0.num_experts, w0.top_k
    P = E + extra
    p2l = wl.eplb_placement(np.bincount(ids_h.ravel(), minlength=E) + 1.0, P, ep)
    l2p, cnt = _tables(E, p2l)
    d_l2p, d_cnt = dev_tensor(l2p), dev_tensor(cnt)
    eplb = moe.make_eplb(P, l2p.shape[1], d_l2p, d_cnt)
    per = P // ep
    dev = full.d["x"].device
    total = np.zeros((T, w0.hidden_size))
    for r in range(ep):
        share_w = w0.with_share(1, 0, shared=(r == 0))
        p = params(share_w, num_local_experts=per)
        pmap = _share_map(P, ep, r)
        d_map = dev_tensor(pmap)
        # routing with the replica choice: ids and weights as moe_route, slots vs the oracle
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        tw = torch.empty(T, k, dtype=torch.float32, device=dev)
        local = torch.full((T, k), 99, dtype=torch.int32, device=dev)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
        moe.moe_route_eplb(p, eplb, T, full.d["x"], full.d["gate"], full.d["bias"], d_map, ids, tw,
                           local, ws)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids_h) and np.array_equal(tw.cpu().numpy(), tw_h)
        want_slots = oracle.eplb_local_slots(ids_h, k, l2p, cnt, pmap)
        assert np.array_equal(local.cpu().numpy(), want_slots)
        # the share's forward over its physical experts
        w13, w2 = _physical_weights(w0, p2l[r * per:(r + 1) * per])
        sw13 = full.d["sw13"] if r == 0 else None
        sw2 = full.d["sw2"] if r == 0 else None
        out = torch.empty(T, w0.hidden_size, dtype=torch_dtype(w0), device=dev)
        moe.moe_forward_eplb(p, eplb, T, full.d["x"], full.d["gate"], full.d["bias"], d_map,
                             dev_tensor(w13), dev_tensor(w2), sw13, sw2, out, None, None, ws)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        shw = (wl.to_f32(full.sw13), wl.to_f32(full.sw2)) if (r == 0 and full.sw13 is not None) \
            else (None, None)
        want_r = oracle.moe_forward_given_slots(wl.to_f32(full.x), want_slots, tw_h,
                                                [wl.to_f32(a) for a in w13],
                                                [wl.to_f32(a) for a in w2], *shw)
        assert rel_err(got, want_r) <= OUT_TOL[w0.dtype]
        total += got
    want = full.oracle_out(np.arange(T), ids_h, tw_h)
    err = rel_err(total, want)
    loads = [int(np.sum((oracle.eplb_local_slots(ids_h, k, l2p, cnt, _share_map(P, ep, r)) >= 0)))
             for r in range(ep)]
    print(f"[eplb {case} T={T} ep={ep} P={P}] rel_err={err:.3e} pairs per rank={loads}", flush=True)
    assert err <= OUT_TOL[w0.dtype]
    out_local, _, _ = full.forward()
    assert rel_err(total, out_local) <= OUT_TOL[w0.dtype]


@pytest.mark.parametrize("case,ep", [("ep_s", 4), ("ds_s", 8)])
def test_eplb_identity_placement_is_moe_forward(case, ep):
    """No redundant experts, identity placement: bit for bit the plain share path."""
    w0, T = SMALL[case]
    E = w0.num_experts
    l2p, cnt = _tables(E, np.arange(E, dtype=np.int32))
    d_l2p, d_cnt = dev_tensor(l2p), dev_tensor(cnt)
    eplb = moe.make_eplb(E, 1, d_l2p, d_cnt)
    for r in (0, ep - 1):
        share = Layer(w0.with_share(ep, r), T)
        ref_out, ref_ids, ref_tw = share.forward()
        p = params(share.w)
        d = share.d
        out = torch.empty(T, w0.hidden_size, dtype=torch_dtype(w0), device=d["x"].device)
        ids = torch.empty(T, w0.top_k, dtype=torch.int32, device=d["x"].device)
        tw = torch.empty(T, w0.top_k, dtype=torch.float32, device=d["x"].device)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=d["x"].device)
        moe.moe_forward_eplb(p, eplb, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"], d["w2"],
                             d["sw13"], d["sw2"], out, ids, tw, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), ref_out)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)
        assert np.array_equal(tw.cpu().numpy(), ref_tw)


def test_eplb_table_entries_out_of_range_are_not_local():
    """Replica counts of 0 or above max_replicas and physical ids outside [0, P) make the pair
    non-local; nothing is read out of range."""
    w0, T = SMALL["ep_s"]
    full = Layer(w0.with_share(1, 0), T)
    ids_h, _, _ = full.gpu_route()
    E, k = w0.num_experts, w0.top_k
    P, R = E + 4, 2
    l2p = np.full((E, R), -1, np.int32)
    l2p[:, 0] = np.arange(E)
    cnt = np.ones(E, np.int32)
    cnt[3] = 0          # no replica
    cnt[5] = 3          # more than max_replicas
    l2p[7, 0] = P + 9   # physical id out of range
    l2p[9, 0] = -4
    pmap = np.arange(P, dtype=np.int32)  # one share holds every physical expert
    p = params(w0.with_share(1, 0), num_local_experts=P)
    eplb = moe.make_eplb(P, R, dev_tensor(l2p), dev_tensor(cnt))
    dev = full.d["x"].device
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    local = torch.full((T, k), 99, dtype=torch.int32, device=dev)
    ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
    moe.moe_route_eplb(p, eplb, T, full.d["x"], full.d["gate"], full.d["bias"], dev_tensor(pmap),
                       ids, tw, local, ws)
    torch.cuda.synchronize()
    got = local.cpu().numpy()
    bad = np.isin(ids_h, [3, 5, 7, 9])
    assert bad.any()
    assert np.all(got[bad] == -1)
    assert np.array_equal(got[~bad], ids_h[~bad])


def test_eplb_with_routing_and_mlp_variants():
    """Replicated experts together with sigmoid scores, a selection bias, the clamped SwiGLU and
    expert biases: every share's slots bit for bit, and the shares' sum against the oracle."""
    w0 = wl.Workload("eplb_var", 51, "EPLB + variants", "bf16", (257,), 256, 32, 128, 4, True,
                     use_grouped_topk=True, num_expert_group=4, topk_group=2,
                     routed_scaling_factor=2.5, scoring_func="sigmoid", score_bias_std=0.05,
                     activation="swigluoai", expert_bias_std=1.0)
    T, ep, extra = 257, 4, 8
    full = Layer(w0, T)
    ids_h, tw_h, _ = full.gpu_route()
    E, k = w0.num_experts, w0.top_k
    P = E + extra
    p2l = wl.eplb_placement(np.bincount(ids_h.ravel(), minlength=E) + 1.0, P, ep)
    l2p, cnt = _tables(E, p2l)
    eplb = moe.make_eplb(P, l2p.shape[1], dev_tensor(l2p), dev_tensor(cnt))
    per = P // ep
    dev = full.d["x"].device
    total = np.zeros((T, w0.hidden_size))
    for r in range(ep):
        p = params(w0, num_local_experts=per)
        pmap = _share_map(P, ep, r)
        mine = p2l[r * per:(r + 1) * per]
        w13, w2 = _physical_weights(w0, mine)
        b13, b2 = wl.expert_biases(w0, [int(e) for e in mine])
        out = torch.empty(T, w0.hidden_size, dtype=torch_dtype(w0), device=dev)
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        tw = torch.empty(T, k, dtype=torch.float32, device=dev)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
        moe.moe_forward_eplb(p, eplb, T, full.d["x"], full.d["gate"], full.d["bias"],
                             dev_tensor(pmap), dev_tensor(w13), dev_tensor(w2), None, None, out,
                             ids, tw, ws, score_bias=full.d["sbias"], b13=dev_tensor(b13),
                             b2=dev_tensor(b2))
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids_h) and np.array_equal(tw.cpu().numpy(), tw_h)
        slots = oracle.eplb_local_slots(ids_h, k, l2p, cnt, pmap)
        want_r = oracle.moe_forward_given_slots(wl.to_f32(full.x), slots, tw_h,
                                                [wl.to_f32(a) for a in w13],
                                                [wl.to_f32(a) for a in w2],
                                                activation="swigluoai", b13_local=b13,
                                                b2_local=b2)
        got = out.float().cpu().numpy()
        assert rel_err(got, want_r) <= OUT_TOL[w0.dtype]
        total += got
    want = full.oracle_out(np.arange(T), ids_h, tw_h)
    assert rel_err(total, want) <= OUT_TOL[w0.dtype]
