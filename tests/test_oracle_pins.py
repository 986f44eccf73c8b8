"""Pins of the CPU oracle against things other than itself (CPU only, no GPU).

Each test fixes one part of the oracle with a closed form, a library routine on a
special case, brute force on tiny inputs, a hand-worked example, or an invariant of the
method (the expert-parallel share-sum, the dense-mixture limit, scaling linearity).
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, stream, std=1.0):
    n = int(np.prod(shape))
    return wl.normal(stream, n, std).reshape(shape).astype(np.float64)


def _tiny_layer(E=8, H=24, I=16, T=11, seed=0, shared_I=0):
    x = _rand((T, H), (900, seed, 0))
    wg = _rand((E, H), (900, seed, 1), 1 / math.sqrt(H))
    w13 = _rand((E, 2 * I, H), (900, seed, 2), 1 / math.sqrt(H))
    w2 = _rand((E, H, I), (900, seed, 3), 1 / math.sqrt(I))
    sw13 = sw2 = None
    if shared_I:
        sw13 = _rand((2 * shared_I, H), (900, seed, 4), 1 / math.sqrt(H))
        sw2 = _rand((H, shared_I), (900, seed, 5), 1 / math.sqrt(shared_I))
    return x, wg, w13, w2, sw13, sw2


# ---------------------------------------------------------------- a1 router GEMM
def test_router_logits_brute_force():
    x = _rand((5, 7), (901, 0, 0))
    wg = _rand((4, 7), (901, 0, 1))
    b = _rand((4,), (901, 0, 2)).astype(np.float32)
    got = oracle.router_logits(x, wg, b)
    for t in range(5):
        for e in range(4):
            exact = math.fsum([x[t, h] * wg[e, h] for h in range(7)] + [float(b[e])])
            ref = np.float32(exact)
            assert abs(float(got[t, e]) - float(ref)) <= abs(float(ref)) * 2 ** -23, (t, e)
    got0 = oracle.router_logits(x, wg, None)
    assert abs(float(got0[1, 2]) - math.fsum(x[1] * wg[2])) < 1e-6


def test_router_logits_expert_relabeling():
    x = _rand((9, 16), (901, 1, 0))
    wg = _rand((6, 16), (901, 1, 1))
    perm = np.array([3, 0, 5, 1, 4, 2])
    assert np.array_equal(oracle.router_logits(x, wg[perm]), oracle.router_logits(x, wg)[:, perm])


# ---------------------------------------------------------------- a2 softmax
def test_softmax_matches_library_and_closed_forms():
    l = (_rand((20, 64), (902, 0, 0)) * 3).astype(np.float32)
    p = oracle.softmax_fp32(l)
    ref = scipy.special.softmax(l.astype(np.float64), axis=1)
    assert p.dtype == np.float32
    assert np.max(np.abs(p - ref) / ref) < 1e-6
    assert np.all(np.abs(p.sum(axis=1, dtype=np.float64) - 1.0) < 1e-6)
    # E = 1: exp(0) / exp(0) is exactly 1
    assert np.all(oracle.softmax_fp32(np.array([[3.5], [-70.0]], np.float32)) == 1.0)
    # large logits must not overflow (max subtraction)
    big = oracle.softmax_fp32(np.array([[1000.0, 0.0, 999.0]], np.float32))
    assert np.all(np.isfinite(big))
    assert abs(big[0, 0] - 1 / (1 + math.exp(-1))) < 1e-6 and big[0, 1] == 0.0


# ---------------------------------------------------------------- a3 top-k
def _beats(p, i, j):
    return p[i] > p[j] or (p[i] == p[j] and i < j)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_topk_brute_force_with_ties(k):
    # probabilities quantised to a few levels so that ties are common
    raw = wl.normal((903, k, 0), 40 * 8).reshape(40, 8)
    p = (np.round(np.abs(raw) * 2) / 8).astype(np.float32)
    ids, gap, _ = oracle.select_experts(p, k)
    for t in range(40):
        sets = [S for S in itertools.combinations(range(8), k)
                if all(_beats(p[t], i, j) for i in S for j in range(8) if j not in S)]
        assert len(sets) == 1
        assert sorted(ids[t].tolist()) == list(sets[0])
        # slot order: probability descending, ties to the lower id
        for a, b in zip(ids[t][:-1], ids[t][1:]):
            assert _beats(p[t], a, b)
        rest = [p[t][j] for j in range(8) if j not in sets[0]]
        assert gap[t] == np.float32(min(p[t][list(sets[0])]) - max(rest))


def test_topk_all_experts():
    p = oracle.softmax_fp32(_rand((6, 8), (903, 9, 0)).astype(np.float32))
    ids, gap, _ = oracle.select_experts(p, 8)
    assert all(sorted(r) == list(range(8)) for r in ids.tolist())
    assert np.all(np.isinf(gap))


def test_grouped_topk_reduces_to_plain():
    p = oracle.softmax_fp32(_rand((30, 16), (904, 0, 0)).astype(np.float32))
    plain = oracle.select_experts(p, 3)[0]
    assert np.array_equal(oracle.select_experts(p, 3, True, 1, 1)[0], plain)
    assert np.array_equal(oracle.select_experts(p, 3, True, 4, 4)[0], plain)
    assert np.array_equal(oracle.select_experts(p, 3, True, 16, 16)[0], plain)


def test_grouped_topk_brute_force():
    raw = wl.normal((904, 1, 0), 50 * 8).reshape(50, 8)
    p = (np.round(np.abs(raw) * 3) / 12).astype(np.float32)
    G, keep, k = 4, 2, 3
    ids, gap, ggap = oracle.select_experts(p, k, True, G, keep)
    for t in range(50):
        gs = [max(p[t][2 * g], p[t][2 * g + 1]) for g in range(G)]
        kept = [S for S in itertools.combinations(range(G), keep)
                if all(_beats(gs, a, b) for a in S for b in range(G) if b not in S)]
        assert len(kept) == 1
        cand = [e for g in kept[0] for e in (2 * g, 2 * g + 1)]
        sets = [S for S in itertools.combinations(cand, k)
                if all(_beats(p[t], i, j) for i in S for j in cand if j not in S)]
        assert len(sets) == 1
        assert sorted(ids[t].tolist()) == sorted(sets[0])
        dropped = [gs[g] for g in range(G) if g not in kept[0]]
        assert ggap[t] == np.float32(min(gs[g] for g in kept[0]) - max(dropped))


def test_grouped_topk_golden_example():
    with open(os.path.join(GOLDEN, "grouped_topk_example.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 5
    for ln in rows:
        probs, k, keep, want = [s.strip() for s in ln.split("|")]
        p = np.array([[float(v) for v in probs.split()]], np.float32)
        ids, _, _ = oracle.select_experts(p, int(k), True, 4, int(keep))
        assert ids[0].tolist() == [int(v) for v in want.split()], ln


# ---------------------------------------------------------------- a3 weights
def test_renormalize_and_scaling():
    p = oracle.softmax_fp32(_rand((25, 16), (905, 0, 0)).astype(np.float32))
    ids = oracle.select_experts(p, 4)[0]
    w = oracle.routing_weights(p, ids, True)
    assert np.all(np.abs(w.sum(axis=1, dtype=np.float64) - 1) < 1e-6)
    w_raw = oracle.routing_weights(p, ids, False)
    assert np.array_equal(w_raw, np.take_along_axis(p, ids.astype(np.int64), axis=1))
    # a power-of-two scale is exact in binary floating point
    assert np.array_equal(oracle.routing_weights(p, ids, True, 16.0), 16 * w)
    assert np.array_equal(oracle.routing_weights(p, ids, False, 16.0), 16 * w_raw)
    # top-1 with renormalisation gives weight exactly 1
    ids1 = oracle.select_experts(p, 1)[0]
    assert np.all(oracle.routing_weights(p, ids1, True) == 1.0)


# ---------------------------------------------------------------- a6/a7 expert MLP
def test_gated_mlp_matches_torch_library():
    H, I = 24, 10
    x = _rand((7, H), (906, 0, 0))
    w13 = _rand((2 * I, H), (906, 0, 1))
    w2 = _rand((H, I), (906, 0, 2))
    X, W13, W2 = (torch.from_numpy(a) for a in (x, w13, w2))
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(X, W13[:I])) * F.linear(X, W13[I:]), W2).numpy()
    got = oracle.gated_mlp(x, w13, w2)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_gated_mlp_scalar_hand_computed():
    # H = I = 1: y = w2 * silu(w1 x) * (w3 x), silu(g) = g / (1 + e^-g)
    x, w1, w3, w2 = 0.7, 1.3, -0.4, 2.5
    g = w1 * x
    want = w2 * (g / (1 + math.exp(-g))) * (w3 * x)
    got = oracle.gated_mlp(np.array([[x]]), np.array([[w1], [w3]]), np.array([[w2]]))
    assert abs(got[0, 0] - want) < 1e-15


def test_single_expert_layer_is_plain_mlp():
    x, wg, w13, w2, _, _ = _tiny_layer(E=1)
    out, r = oracle.moe_forward(x, wg, np.array([0], np.int32), w13, w2, 1, True)
    assert np.all(r["weights"] == 1.0) and np.all(r["ids"] == 0)
    F = torch.nn.functional
    X = torch.from_numpy(x)
    I = w13.shape[1] // 2
    W13 = torch.from_numpy(w13[0])
    ref = F.linear(F.silu(F.linear(X, W13[:I])) * F.linear(X, W13[I:]), torch.from_numpy(w2[0]))
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_shared_mlps_concatenate():
    # two shared experts of width I equal one of width 2I (concatenated rows/cols)
    H, I = 16, 8
    x = _rand((5, H), (907, 0, 0))
    a13, b13 = _rand((2 * I, H), (907, 0, 1)), _rand((2 * I, H), (907, 0, 2))
    a2, b2 = _rand((H, I), (907, 0, 3)), _rand((H, I), (907, 0, 4))
    cat13 = np.concatenate([a13[:I], b13[:I], a13[I:], b13[I:]])
    cat2 = np.concatenate([a2, b2], axis=1)
    two = oracle.gated_mlp(x, a13, a2) + oracle.gated_mlp(x, b13, b2)
    assert np.allclose(oracle.gated_mlp(x, cat13, cat2), two, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- a9 combine / whole layer
def test_topk_all_with_renorm_is_dense_mixture():
    E = 6
    x, wg, w13, w2, _, _ = _tiny_layer(E=E, T=9)
    out, _ = oracle.moe_forward(x, wg, np.arange(E, dtype=np.int32), w13, w2, E, True)
    F = torch.nn.functional
    X = torch.from_numpy(x)
    p = torch.softmax(F.linear(X, torch.from_numpy(wg)), dim=1)
    I = w13.shape[1] // 2
    ref = torch.zeros_like(X)
    for e in range(E):
        W13 = torch.from_numpy(w13[e])
        y = F.linear(F.silu(F.linear(X, W13[:I])) * F.linear(X, W13[I:]), torch.from_numpy(w2[e]))
        ref += p[:, e:e + 1] * y
    ref = ref.numpy()
    assert np.max(np.abs(out - ref)) / np.max(np.abs(ref)) < 2e-6


def test_page1_expert_loop_equals_per_token_definition():
    x, wg, w13, w2, sw13, sw2 = _tiny_layer(shared_I=6)
    emap = np.array([-1, 0, 1, -1, 2, -1, 3, -1], np.int32)
    local = [1, 2, 4, 6]
    r = oracle.route(x, wg, 3, True)
    a = oracle.moe_forward_given_routing(x, r["ids"], r["weights"], emap, w13[local], w2[local],
                                         sw13, sw2)
    b = oracle.moe_forward_per_token(x, r["ids"], r["weights"], emap, w13[local], w2[local],
                                     sw13, sw2)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("ep", [2, 4, 8])
def test_share_sum_equals_all_local(ep):
    E = 8
    x, wg, w13, w2, sw13, sw2 = _tiny_layer(E=E, T=17, shared_I=8)
    full, r = oracle.moe_forward(x, wg, np.arange(E, dtype=np.int32), w13, w2, 2, True,
                                 shared_w13=sw13, shared_w2=sw2)
    total = np.zeros_like(full)
    n = E // ep
    for rank in range(ep):
        emap = np.full(E, -1, np.int32)
        emap[rank * n:(rank + 1) * n] = np.arange(n)
        sh = (sw13, sw2) if rank == 0 else (None, None)
        part, r2 = oracle.moe_forward(x, wg, emap, w13[rank * n:(rank + 1) * n],
                                      w2[rank * n:(rank + 1) * n], 2, True,
                                      shared_w13=sh[0], shared_w2=sh[1])
        assert np.array_equal(r2["ids"], r["ids"])
        total += part
    assert np.allclose(total, full, rtol=1e-12, atol=1e-12)


def test_share_without_tokens_is_zero():
    x, wg, w13, w2, _, _ = _tiny_layer(E=8)
    r = oracle.route(x, wg, 2, True)
    unused = sorted(set(range(8)) - set(r["ids"].reshape(-1).tolist()))
    emap = np.full(8, -1, np.int32)
    for s, e in enumerate(unused):
        emap[e] = s
    out = oracle.moe_forward_given_routing(x, r["ids"], r["weights"], emap, w13[unused],
                                           w2[unused])
    assert np.all(out == 0.0)
    out2 = oracle.moe_forward_given_routing(x, r["ids"], r["weights"], np.full(8, -1, np.int32),
                                            w13[:0], w2[:0])
    assert np.all(out2 == 0.0)


def test_routed_scaling_is_linear():
    x, wg, w13, w2, _, _ = _tiny_layer(E=8)
    emap = np.arange(8, dtype=np.int32)
    o1, r1 = oracle.moe_forward(x, wg, emap, w13, w2, 3, False, True, 4, 2, 1.0)
    o16, r16 = oracle.moe_forward(x, wg, emap, w13, w2, 3, False, True, 4, 2, 16.0)
    assert np.array_equal(r1["ids"], r16["ids"])
    assert np.array_equal(o16, 16.0 * o1)


def test_token_permutation_equivariance():
    x, wg, w13, w2, sw13, sw2 = _tiny_layer(E=8, T=13, shared_I=4)
    emap = np.array([0, 1, 2, 3, -1, -1, -1, -1], np.int32)
    perm = np.array([5, 0, 12, 3, 7, 1, 9, 2, 11, 4, 10, 6, 8])
    a, _ = oracle.moe_forward(x, wg, emap, w13[:4], w2[:4], 2, True, shared_w13=sw13, shared_w2=sw2)
    b, _ = oracle.moe_forward(x[perm], wg, emap, w13[:4], w2[:4], 2, True,
                              shared_w13=sw13, shared_w2=sw2)
    assert np.allclose(b, a[perm], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- a5 align / permute
@pytest.mark.parametrize("block_m", [1, 4, 16])
def test_align_permute_brute_force(block_m):
    T, k, E_l = 37, 3, 5
    raw = wl.normal((908, block_m, 0), T * k)
    tl = (np.floor(np.abs(raw) * 3).astype(np.int32) % (E_l + 2)) - 2  # -2/-1 -> non-local
    tl[tl < 0] = -1
    a = oracle.align_permute(tl.reshape(T, k), E_l, block_m)
    flat = tl.reshape(-1)
    counts = [sum(1 for v in flat if v == e) for e in range(E_l)]
    assert a["counts"].tolist() == counts
    off = 0
    for e in range(E_l):
        assert a["offsets"][e] == off
        seg = a["sorted_pairs"][off:off + counts[e]].tolist()
        assert seg == [p for p in range(T * k) if flat[p] == e]  # ascending pair ids
        pad = -(-counts[e] // block_m) * block_m
        assert all(v == -1 for v in a["sorted_pairs"][off + counts[e]:off + pad])
        assert all(v == e for v in a["block_expert"][off // block_m:(off + pad) // block_m])
        off += pad
    assert a["num_padded"] == off and a["offsets"][E_l] == off
    assert off <= sum(counts) + E_l * (block_m - 1)
    for p in range(T * k):
        r = a["pair_row"][p]
        assert (r == -1) == (flat[p] < 0)
        if r >= 0:
            assert a["sorted_pairs"][r] == p


def test_align_permute_empty():
    a = oracle.align_permute(np.full((4, 2), -1, np.int32), 3, 8)
    assert a["num_padded"] == 0 and a["sorted_pairs"].size == 0 and np.all(a["pair_row"] == -1)


# ---------------------------------------------------------------- memory arithmetic
def test_memory_arithmetic_golden():
    with open(os.path.join(GOLDEN, "memory_arithmetic.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    GiB = 2 ** 30
    vals = {}
    for case, n, H, I, b, L, printed, want in rows:
        got = oracle.weight_bytes(int(n), int(H), int(I), int(b), int(L))
        assert got == int(want), case
        vals[case] = got
    assert vals["tp2"] == 22.5 * GiB  # printed 22.5 GiB, exact
    assert vals["ep4"] == 11.25 * GiB  # the page prints 5.6; its formula gives 11.25
    assert vals["full"] == 45 * GiB
    assert vals["ep4"] == vals["full"] // 4 and vals["tp2"] == vals["full"] // 2
    assert abs(vals["ep4"] / GiB - 5.6) > 5  # the printed 5.6 GiB is not reproducible


# ---------------------------------------------------------------- NEXT-1 exchange (dispatch / combine)
def _distinct_ids(T, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def _dispatch_brute(ids, E, R):
    """Rank by rank, token by token: a token goes to rank r once, carried by its first slot
    whose expert lives on r (written independently of the oracle's vectorised form)."""
    T, k = ids.shape
    per = E // R
    send_pos = [-1] * (T * k)
    send_token, counts = [], []
    for r in range(R):
        c = 0
        for t in range(T):
            js = [j for j in range(k) if ids[t, j] // per == r]
            if js:
                send_pos[t * k + js[0]] = len(send_token)
                send_token.append(t)
                c += 1
        counts.append(c)
    return np.array(send_pos), np.array(send_token, dtype=np.int64), np.array(counts)


@pytest.mark.parametrize("T,k,E,R", [(1, 1, 2, 2), (5, 2, 4, 2), (7, 3, 8, 4), (6, 4, 8, 8), (9, 2, 6, 3),
                                     (4, 3, 9, 1)])
def test_ep_dispatch_brute_force(T, k, E, R):
    for seed in range(5):
        ids = _distinct_ids(T, k, E, seed)
        # repeated experts in one token (external routing) must still give one row per rank
        if seed == 4 and k > 1:
            ids[:, 1] = ids[:, 0]
        plan = oracle.ep_dispatch(ids, k, E, R)
        pos, tok, cnt = _dispatch_brute(ids, E, R)
        assert np.array_equal(plan["send_pos"], pos)
        assert np.array_equal(plan["send_token"], tok)
        assert np.array_equal(plan["counts"], cnt)
        assert plan["offsets"][0] == 0 and np.array_equal(np.diff(plan["offsets"]), cnt)
        assert plan["n_send"] == int(cnt.sum())


def test_ep_dispatch_special_cases():
    ids = _distinct_ids(10, 3, 12, 1)
    # one rank: every token is sent once, by its first slot, in token order
    p1 = oracle.ep_dispatch(ids, 3, 12, 1)
    assert np.array_equal(p1["send_token"], np.arange(10))
    assert np.array_equal(p1["send_pos"].reshape(10, 3)[:, 0], np.arange(10))
    assert np.all(p1["send_pos"].reshape(10, 3)[:, 1:] == -1)
    # one slot per token: every pair owns a row, n_send = T
    p2 = oracle.ep_dispatch(ids[:, :1], 1, 12, 4)
    assert p2["n_send"] == 10 and np.all(p2["send_pos"] >= 0)
    # as many ranks as experts: no two distinct experts share a rank, so every pair owns a row
    p3 = oracle.ep_dispatch(ids, 3, 12, 12)
    assert p3["n_send"] == 30 and np.all(p3["send_pos"] >= 0)


def test_ep_pack_rows_and_local_slots():
    T, k, E, R = 13, 3, 12, 4
    per = E // R
    ids = _distinct_ids(T, k, E, 2)
    w = np.random.default_rng(3).uniform(0.1, 1.0, (T, k)).astype(np.float32)
    x = _rand((T, 5), (901, 0, 0))
    plan = oracle.ep_dispatch(ids, k, E, R)
    pk = oracle.ep_pack(plan, x, ids, w, k, E, R)
    for row, t in enumerate(plan["send_token"]):
        r = int(np.searchsorted(plan["offsets"], row, side="right") - 1)
        assert np.array_equal(pk["send_x"][row], x[t])
        assert np.array_equal(pk["send_w"][row], w[t])
        # the local slot of each expert seen from rank r: expert_map of that share
        emap_r = np.full(E, -1)
        emap_r[r * per:(r + 1) * per] = np.arange(per)
        assert np.array_equal(pk["send_local"][row], emap_r[ids[t]])


@pytest.mark.parametrize("R", [1, 2, 4])
def test_ep_exchange_reconstructs_layer(R):
    """dispatch -> each rank's share of the layer on the rows it received -> combine equals
    the all-local layer (the expert-parallel share sum, through the exchange)."""
    E, H, I, T, k = 8, 24, 16, 11, 3
    x, _, w13, w2, _, _ = _tiny_layer(E=E, H=H, I=I, T=T, seed=3)
    ids = _distinct_ids(T, k, E, 7)
    w = np.random.default_rng(8).uniform(0.1, 1.0, (T, k))
    plan = oracle.ep_dispatch(ids, k, E, R)
    pk = oracle.ep_pack(plan, x, ids, w.astype(np.float32), k, E, R)
    per = E // R
    recv = np.zeros((plan["n_send"], H))
    for r in range(R):
        a, b = plan["offsets"][r], plan["offsets"][r + 1]
        emap_r = np.full(E, -1)
        emap_r[r * per:(r + 1) * per] = np.arange(per)
        rows = plan["send_token"][a:b]
        recv[a:b] = oracle.moe_forward_given_routing(pk["send_x"][a:b], ids[rows], pk["send_w"][a:b],
                                                     emap_r, w13[r * per:(r + 1) * per],
                                                     w2[r * per:(r + 1) * per])
    got = oracle.ep_combine(plan, recv, k)
    want = oracle.moe_forward_given_routing(x, ids, w.astype(np.float32), np.arange(E), w13, w2)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- EPLB (replicated experts)
def test_eplb_tables_hand_example():
    """8 physical experts serving 4 logical ones (placement worked by hand)."""
    l2p, cnt = oracle.eplb_tables([0, 1, 2, 3, 0, 2, 0, 1], 4)
    assert l2p.tolist() == [[0, 4, 6], [1, 7, -1], [2, 5, -1], [3, -1, -1]]
    assert cnt.tolist() == [3, 2, 2, 1]
    with pytest.raises(ValueError):
        oracle.eplb_tables([0, 1, 1, 0], 3)  # logical expert 2 has no replica


def test_eplb_local_slots_hand_example():
    """Round robin by token index over the replicas, worked by hand for two ranks of 4
    physical experts (rank 0: logical 0 1 2 3; rank 1: logical 0 2 0 1)."""
    l2p, cnt = oracle.eplb_tables([0, 1, 2, 3, 0, 2, 0, 1], 4)
    ids = np.array([[0, 3], [0, 1], [2, 0], [1, 2]])
    r0 = np.array([0, 1, 2, 3, -1, -1, -1, -1])
    r1 = np.array([-1, -1, -1, -1, 0, 1, 2, 3])
    assert oracle.eplb_local_slots(ids, 2, l2p, cnt, r0).tolist() == \
        [[0, 3], [-1, -1], [2, -1], [-1, -1]]
    assert oracle.eplb_local_slots(ids, 2, l2p, cnt, r1).tolist() == \
        [[-1, -1], [0, 3], [-1, 2], [3, 1]]


def test_eplb_identity_placement_is_the_plain_map():
    """No redundant experts and the identity placement: the slots are expert_map[ids]."""
    E, k, T = 16, 4, 50
    ids = _distinct_ids(T, k, E, 21)
    l2p, cnt = oracle.eplb_tables(np.arange(E), E)
    for R, r in [(1, 0), (4, 1), (4, 3), (16, 5)]:
        per = E // R
        emap = np.full(E, -1)
        emap[r * per:(r + 1) * per] = np.arange(per)
        assert np.array_equal(oracle.eplb_local_slots(ids, k, l2p, cnt, emap), emap[ids])


def test_eplb_split_is_even_over_consecutive_tokens():
    """Consecutive tokens that all pick one logical expert are spread over its replicas with
    counts that differ by at most one."""
    l2p, cnt = oracle.eplb_tables([0, 1, 0, 0, 1, 2, 0, 2, 3], 4)  # logical 0: 4 replicas
    T = 103
    ids = np.zeros((T, 1), np.int64)
    pmap = np.arange(9)  # one rank holds all physical experts; slot = physical id
    slots = oracle.eplb_local_slots(ids, 1, l2p, cnt, pmap).ravel()
    per_rep = np.bincount(slots, minlength=9)[[0, 2, 3, 6]]
    assert per_rep.sum() == T and per_rep.max() - per_rep.min() <= 1


@pytest.mark.parametrize("R", [1, 2, 3])
def test_eplb_share_sum_equals_all_local(R):
    """Every pair lands on exactly one replica, whose weights are its logical expert's: the
    shares of a replicated placement sum to the all-local layer."""
    E, H, I, T, k = 8, 24, 16, 23, 3
    x, _, w13, w2, sw13, sw2 = _tiny_layer(E=E, H=H, I=I, T=T, seed=5, shared_I=8)
    ids = _distinct_ids(T, k, E, 9)
    w = np.random.default_rng(10).uniform(0.1, 1.0, (T, k))
    p2l = np.concatenate([np.arange(E), [0, 0, 3, 5]])  # 12 physical experts
    rng = np.random.default_rng(11)
    p2l = p2l[rng.permutation(p2l.size)]
    P = p2l.size
    l2p, cnt = oracle.eplb_tables(p2l, E)
    per = P // R
    total = np.zeros((T, H))
    for r in range(R):
        pmap = np.full(P, -1)
        pmap[r * per:(r + 1) * per] = np.arange(per)
        slots = oracle.eplb_local_slots(ids, k, l2p, cnt, pmap)
        mine = p2l[r * per:(r + 1) * per]
        sh = (sw13, sw2) if r == 0 else (None, None)
        total += oracle.moe_forward_given_slots(x, slots, w, w13[mine], w2[mine], *sh)
    want = oracle.moe_forward_given_routing(x, ids, w, np.arange(E), w13, w2, sw13, sw2)
    assert np.allclose(total, want, rtol=1e-12, atol=1e-12)


def test_forward_given_slots_matches_per_expert_form():
    """With the slots of a plain expert map, the slot form is the per-expert loop."""
    E, H, I, T, k = 8, 24, 16, 13, 2
    x, _, w13, w2, _, _ = _tiny_layer(E=E, H=H, I=I, T=T, seed=6)
    ids = _distinct_ids(T, k, E, 12)
    w = np.random.default_rng(13).uniform(0.1, 1.0, (T, k))
    emap = np.array([-1, 0, -1, 1, 2, -1, 3, -1])
    loc = [1, 3, 4, 6]
    got = oracle.moe_forward_given_slots(x, emap[ids], w, w13[loc], w2[loc])
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            s = emap[ids[t, j]]
            if s >= 0:
                h = w13[loc[s]] @ x[t]
                a = h[:I] / (1 + np.exp(-h[:I])) * h[I:]
                want[t] += w[t, j] * (w2[loc[s]] @ a)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- routing variants
def test_sigmoid_special_values_and_symmetry():
    s = oracle.sigmoid_fp32(np.array([[0.0, math.log(3.0), -math.log(3.0), 200.0, -200.0]]))
    assert s.dtype == np.float32
    assert s[0, 0] == 0.5 and s[0, 1] == 0.75 and s[0, 2] == 0.25
    assert s[0, 3] == 1.0 and s[0, 4] == 0.0  # exp(200) overflows the fp32 range of 1/(1+e)
    x = _rand((1, 257), (901, 0, 0), 4.0)
    a, b = oracle.sigmoid_fp32(x), oracle.sigmoid_fp32(-x)
    assert np.max(np.abs(a.astype(np.float64) + b - 1.0)) <= 2.0 ** -24
    assert np.all(np.diff(oracle.sigmoid_fp32(np.sort(x, axis=1))) >= 0)


def test_sigmoid_and_softmax_pick_the_same_experts():
    """Both scores are increasing in the logit, so the plain top-k is the same set (tokens
    whose chosen logits are clearly apart)."""
    l = _rand((64, 32), (902, 0, 0), 2.0).astype(np.float32)
    a = oracle.route_from_logits(l, 5, True, scoring_func="softmax")
    b = oracle.route_from_logits(l, 5, True, scoring_func="sigmoid")
    srt = -np.sort(-l, axis=1)
    clear = (srt[:, 4] - srt[:, 5]) > 1e-4
    assert np.array_equal(np.sort(a["ids"], 1)[clear], np.sort(b["ids"], 1)[clear])
    # the sigmoid weights are the scores of the chosen experts, renormalised
    p = 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    pc = np.take_along_axis(p, b["ids"].astype(np.int64), axis=1)
    assert np.allclose(b["weights"], pc / pc.sum(axis=1, keepdims=True), rtol=1e-6)


def _v3_brute(p, b, k, G, keep):
    """Group-limited choice with a selection bias, by plain enumeration on one token."""
    E = len(p)
    per = E // G
    s = [float(np.float32(np.float32(p[e]) + np.float32(b[e]))) for e in range(E)]
    gsc = []
    for g in range(G):
        top = sorted(s[g * per:(g + 1) * per], reverse=True)
        gsc.append(float(np.float32(top[0] + top[1])) if per > 1 else top[0])
    groups = sorted(range(G), key=lambda g: (-gsc[g], g))[:keep]
    cand = [e for e in range(E) if e // per in groups]
    return sorted(sorted(cand, key=lambda e: (-s[e], e))[:k])


@pytest.mark.parametrize("E,G,keep,k", [(8, 4, 2, 3), (12, 3, 1, 2), (16, 8, 3, 4), (6, 6, 6, 2)])
def test_grouped_choice_with_bias_brute_force(E, G, keep, k):
    rng = np.random.default_rng(E * 10 + G)
    for trial in range(40):
        p = oracle.softmax_fp32(rng.normal(size=(1, E)).astype(np.float32))
        b = rng.normal(scale=0.05, size=E).astype(np.float32)
        ids, _, _ = oracle.select_experts(p, k, True, G, keep, score_bias=b)
        assert sorted(ids[0].tolist()) == _v3_brute(p[0], b, k, G, keep), trial


def test_bias_steers_choice_not_weights():
    """A large bias forces an expert into the top-k; its weight is still its own score."""
    l = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -3.0]], np.float32)
    b = np.zeros(6, np.float32)
    b[5] = 10.0
    r = oracle.route_from_logits(l, 2, False, scoring_func="sigmoid", score_bias=b)
    assert sorted(r["ids"][0].tolist()) == [0, 5]
    w = dict(zip(r["ids"][0].tolist(), r["weights"][0].tolist()))
    assert w[5] == np.float32(1.0 / (1.0 + math.exp(3.0)))
    assert w[0] == np.float32(1.0 / (1.0 + math.exp(-2.0)))
    # a bias equal on every expert changes nothing in the plain choice
    l2 = _rand((40, 16), (903, 0, 0)).astype(np.float32)
    r0 = oracle.route_from_logits(l2, 4, True, scoring_func="sigmoid")
    r1 = oracle.route_from_logits(l2, 4, True, scoring_func="sigmoid",
                                  score_bias=np.full(16, 0.125, np.float32))
    assert np.array_equal(r0["ids"], r1["ids"]) and np.array_equal(r0["weights"], r1["weights"])


def test_grouped_with_bias_and_groups_of_one_is_plain_topk():
    l = _rand((30, 16), (904, 0, 0)).astype(np.float32)
    b = (_rand((16,), (904, 0, 1)) * 0.1).astype(np.float32)
    g = oracle.route_from_logits(l, 3, True, True, 16, 16, scoring_func="sigmoid", score_bias=b)
    pl = oracle.route_from_logits(l, 3, True, scoring_func="sigmoid", score_bias=b)
    assert np.array_equal(g["ids"], pl["ids"]) and np.array_equal(g["weights"], pl["weights"])


# ---------------------------------------------------------------- MLP variants
def _unit_mlp(g, u, activation, b13=None, b2=None):
    """One-row MLP whose gate and up pre-activations are the inputs themselves (H = 2, I = 1,
    identity W1/W3 rows), read out through W2 = [1, 0]^T."""
    w13 = np.array([[1.0, 0.0], [0.0, 1.0]])
    w2 = np.array([[1.0], [0.0]])
    return oracle.gated_mlp(np.array([[g, u]]), w13, w2, activation, b13, b2)[0]


def test_swigluoai_closed_forms():
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    assert _unit_mlp(1.0, 0.0, "swigluoai")[0] == pytest.approx(sig(1.702), rel=1e-15)
    assert _unit_mlp(-2.0, 3.0, "swigluoai")[0] == pytest.approx(-2.0 * sig(-3.404) * 4.0, rel=1e-15)
    # gate clamped above at 7, up clamped to [-7, 7]
    assert _unit_mlp(10.0, 9.0, "swigluoai")[0] == pytest.approx(7.0 * sig(7 * 1.702) * 8.0, rel=1e-15)
    assert _unit_mlp(2.0, -9.0, "swigluoai")[0] == pytest.approx(2.0 * sig(3.404) * -6.0, rel=1e-15)
    assert _unit_mlp(-50.0, 1.0, "swigluoai")[0] == pytest.approx(-50.0 * sig(-85.1) * 2.0, rel=1e-12)
    # up = -1 cancels the gate; silu at the same point for contrast
    assert _unit_mlp(3.0, -1.0, "swigluoai")[0] == 0.0
    assert _unit_mlp(1.0, 2.0, "silu")[0] == pytest.approx(sig(1.0) * 2.0, rel=1e-15)
    with pytest.raises(ValueError):
        _unit_mlp(1.0, 1.0, "gelu")


def test_expert_biases_are_affine_shifts():
    """A gate/up bias is a weight column on a constant input of 1; an output bias adds itself."""
    x, _, w13, w2, _, _ = _tiny_layer(E=1, H=24, I=16, T=9, seed=7)
    b13 = _rand((32,), (905, 0, 0))
    b2 = _rand((24,), (905, 0, 1))
    for act in ("silu", "swigluoai"):
        with_b = oracle.gated_mlp(x, w13[0], w2[0], act, b13, None)
        aug = oracle.gated_mlp(np.hstack([x, np.ones((9, 1))]), np.hstack([w13[0], b13[:, None]]),
                               w2[0], act)
        assert np.allclose(with_b, aug, rtol=1e-13, atol=1e-13)
        d = oracle.gated_mlp(x, w13[0], w2[0], act, b13, b2) - with_b
        assert np.allclose(d, np.broadcast_to(b2, d.shape), rtol=0, atol=1e-13)
        zero = oracle.gated_mlp(x, w13[0], w2[0], act, np.zeros(32), np.zeros(24))
        assert np.array_equal(zero, oracle.gated_mlp(x, w13[0], w2[0], act))


@pytest.mark.parametrize("R", [1, 2, 4])
def test_mlp_variants_share_sum_and_per_token_form(R):
    """swigluoai with expert biases: the vectorised per-expert form equals the per-token loop,
    and the shares (shared expert on one of them) sum to the all-local layer."""
    E, H, I, T, k = 8, 24, 16, 10, 3
    x, _, w13, w2, sw13, sw2 = _tiny_layer(E=E, H=H, I=I, T=T, seed=8, shared_I=8)
    x = 3.0 * x  # reach the clamps
    b13 = _rand((E, 2 * I), (906, 0, 0))
    b2 = _rand((E, H), (906, 0, 1))
    ids = _distinct_ids(T, k, E, 14)
    w = np.random.default_rng(15).uniform(0.1, 1.0, (T, k))
    kw = dict(activation="swigluoai", b13_local=b13, b2_local=b2)
    full = oracle.moe_forward_given_routing(x, ids, w, np.arange(E), w13, w2, sw13, sw2, **kw)
    per_tok = oracle.moe_forward_per_token(x, ids, w, np.arange(E), w13, w2, sw13, sw2, **kw)
    assert np.allclose(full, per_tok, rtol=1e-12, atol=1e-12)
    per = E // R
    total = np.zeros((T, H))
    for r in range(R):
        emap = np.full(E, -1)
        emap[r * per:(r + 1) * per] = np.arange(per)
        sl = slice(r * per, (r + 1) * per)
        sh = (sw13, sw2) if r == 0 else (None, None)
        total += oracle.moe_forward_given_routing(x, ids, w, emap, w13[sl], w2[sl], *sh,
                                                  activation="swigluoai", b13_local=b13[sl],
                                                  b2_local=b2[sl])
    assert np.allclose(total, full, rtol=1e-12, atol=1e-12)


def test_align_variable_blocks_hand_worked():
    """Variable row blocks (block_m = 0) on hand-worked counts: padding to 32, blocks of 256,
    a last piece of at most 64 rows kept in the block before it."""
    counts = [1024, 1033, 1055, 974, 0, 1, 300, 330, 256, 288, 290]
    tl = np.concatenate([np.full(c, e) for e, c in enumerate(counts)]).astype(np.int32)
    a = oracle.align_permute(tl.reshape(-1, 1), len(counts), 0)
    pad = [1024, 1056, 1056, 992, 0, 32, 320, 352, 256, 288, 320]
    assert a["num_padded"] == sum(pad)
    # expected blocks per slot (rows): 1024 -> 4 x 256; 1056 -> 3 x 256 + 288; 992 -> 3 x 256 +
    # 224; 32 -> 32; 320 -> 320; 352 -> 256 + 96; 256; 288; 320
    want_rows = [[256] * 4, [256] * 3 + [288], [256] * 3 + [288], [256] * 3 + [224], [], [32],
                 [320], [256, 96], [256], [288], [320]]
    t = a["block_expert"]
    nb = t[0]
    assert nb == sum(len(r) for r in want_rows)
    assert t[1 + 2 * nb] == -1 and t[2 + 2 * nb] == a["num_padded"]
    got = {}
    for b in range(nb):
        got.setdefault(int(t[1 + 2 * b]), []).append(int(t[4 + 2 * b] - t[2 + 2 * b]))
    for e, rows in enumerate(want_rows):
        assert got.get(e, []) == rows, (e, got.get(e))


def test_align_variable_blocks_invariants():
    """Random routings: the blocks tile [0, num_padded) in order, each inside one slot's padded
    segment, 32 .. 320 rows and a multiple of 32; the pairs are those of the fixed granules."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        E_l = int(rng.integers(1, 40))
        T, k = int(rng.integers(1, 3000)), int(rng.integers(1, 5))
        tl = rng.integers(-1, E_l, size=(T, k)).astype(np.int32)
        a = oracle.align_permute(tl, E_l, 0)
        b = oracle.align_permute(tl, E_l, 32)
        assert np.array_equal(a["sorted_pairs"], b["sorted_pairs"])
        assert np.array_equal(a["pair_row"], b["pair_row"])
        t = a["block_expert"]
        nb = int(t[0])
        starts = [int(t[2 + 2 * i]) for i in range(nb + 1)]
        assert starts[0] == 0 or nb == 0
        assert starts[-1] == a["num_padded"]
        off = a["offsets"]
        for i in range(nb):
            e, r0, r1 = int(t[1 + 2 * i]), starts[i], starts[i + 1]
            assert off[e] <= r0 < r1 <= off[e + 1]
            assert 32 <= r1 - r0 <= 320 and (r1 - r0) % 32 == 0
        # every non-empty slot is covered by its blocks, no more blocks than 256-row pieces
        for e in range(E_l):
            mine = [i for i in range(nb) if t[1 + 2 * i] == e]
            seg = off[e + 1] - off[e]
            assert sum(starts[i + 1] - starts[i] for i in mine) == seg
            assert len(mine) <= -(-seg // 256)
