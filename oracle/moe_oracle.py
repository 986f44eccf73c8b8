"""CPU oracle of the fused MoE layer forward on one expert-parallel share.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the test suite, the smoke check of ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` use it. It shares no code with the HIP library and
reads nothing the HIP library wrote.

What it computes is the plain definition of the MoE layer as the pages give it:

* "[Feature] Expert parallelism support" (sglang issue #1435), ``MixtralMoE.forward``:
  router logits from a replicated gate, softmax in fp32, top-k, renormalise, then for
  each local expert the expert MLP weighted by the routing weight, summed; the rank's
  partial sum is all-reduced over ranks, so one share's output is that sum restricted
  to its local experts.
* "ep_fused_moe_patch.py: EP-aware FusedMoE override for vllm 0.6.3", ``_ep_init`` /
  ``_ep_forward``: routing over ALL experts on every rank (``select_experts`` sees the
  global count), local experts at FULL intermediate size, the renormalize /
  grouped-top-k switches, and the per-token sum of the weighted expert rows
  (Step 4, scatter-add by token).
* "vllm.model_executor.models.transformers.moe", ``MoEMixin.recursive_replace``:
  ``routed_scaling_factor``, grouped top-k enabled by ``n_group`` / ``topk_group``,
  the ``silu`` activation, packed ``gate_up_proj`` of shape (E, 2I, H), and shared
  experts that the fused layer adds itself.
* "Expert Parallel" (vllm-omni design doc), Step 5 forward: the shared expert output is
  added to the routed output on every rank.
* "vllm.model_executor.models.transformers.moe", ``update_physical_experts_metadata`` and
  the EPLB settings of ``recursive_replace``: E logical experts are served by
  E + num_redundant_experts physical ones, each rank holding an equal contiguous share of
  the physical experts, and the expert map is rebuilt over physical experts.

Precision. Router logits are the fp32 rounding of the exact (fp64-accumulated) dot
products; softmax, top-k selection and routing weights are fp32, because the pages run
the softmax with ``dtype=torch.float`` and select on those values. The expert MLPs and
the combine run in fp64 on the exact (upcast) input values.

Readings of points the pages leave open (each is listed with its reason in the design
notes): the expert MLP is ``W2 (silu(W1 x) * (W3 x))`` with ``w13`` = [W1 rows; W3 rows];
grouped top-k scores a group by its largest softmax probability, keeps ``topk_group``
groups and picks top-k among their experts; ties go to the lower expert (or group) id;
renormalisation is over all k global picks, before the expert_map mask; the routed
scaling factor multiplies the routing weights after renormalisation and does not touch
the shared expert; the routing weight multiplies the expert output (after W2). The
activation switch ``swigluoai`` is gpt-oss's clamped SwiGLU (alpha 1.702, limit 7) and the
expert biases (``has_bias``) are added to the gate/up pre-activations and to the expert
output; the pages name both without their formulas.

Pins: every function here is checked by the ``not gpu`` tests against closed forms,
library routines on special cases, brute force on tiny inputs and invariants of the
method (see the tests of the oracle). The absolute outputs of the large workloads are
pinned only through those checks.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "router_logits", "softmax_fp32", "sigmoid_fp32", "select_experts", "routing_weights", "route_from_logits",
    "route",
    "gated_mlp", "moe_forward_given_routing", "moe_forward", "moe_forward_per_token",
    "align_permute", "weight_bytes",
    "ep_dispatch", "ep_pack", "ep_combine",
    "eplb_tables", "eplb_local_slots", "moe_forward_given_slots",
]


def router_logits(x, w_gate, logit_bias=None):
    """fp32 router logits [T, E] = x [T, H] . w_gate [E, H]^T (+ bias [E]).

    The replicated gate of ``MixtralMoE`` (``ReplicatedLinear(hidden, num_experts,
    bias=False)``; sglang issue #1435) and of ``HunYuanSparseMoeBlock`` ("Expert
    Parallel", Step 2). The skewed-load workload adds a per-expert bias to the logits.
    Dot products are accumulated in fp64 and rounded once to fp32.
    """
    l = np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, np.float64)[None, :]
    return l.astype(np.float32)


def softmax_fp32(logits):
    """Row softmax in fp32: exp(l - max) / sum exp(l - max).

    ``F.softmax(router_logits, dim=1, dtype=torch.float)`` in ``MixtralMoE.forward``.
    """
    l = np.asarray(logits, np.float32)
    m = l.max(axis=1, keepdims=True)
    with np.errstate(under="ignore"):
        e = np.exp(l - m)
    s = e.sum(axis=1, keepdims=True, dtype=np.float32)
    return (e / s).astype(np.float32)


def sigmoid_fp32(logits):
    """Element-wise logistic scores 1 / (1 + exp(-l)), computed in fp64 and rounded once to fp32.

    ``scoring_func`` of the fused layer (``recursive_replace`` passes it through; softmax is
    the default). The pages name the switch without its formula; sigmoid is the logistic
    function, as DeepSeek-V3 scores its experts.
    """
    l = np.asarray(logits, np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l))).astype(np.float32)


def select_experts(p, top_k, use_grouped_topk=False, num_expert_group=1, topk_group=1,
                   score_bias=None):
    """Top-k expert ids per token, plain or group-limited.

    Plain: the k largest probabilities (``torch.topk`` in ``MixtralMoE.forward``).
    Grouped (``use_grouped_topk`` / ``num_expert_group`` / ``topk_group`` of ``_ep_init``;
    ``n_group`` / ``topk_group`` of ``recursive_replace``): experts form
    ``num_expert_group`` contiguous groups of E/G; a group's score is its largest
    probability; the ``topk_group`` best groups are kept and the top-k is taken among
    their experts only (others are excluded, not zeroed).

    ``score_bias`` (``e_score_correction_bias``, named on the transformers MoE page without
    its use): a per-expert bias added to the scores for the choice only, as DeepSeek-V3
    does: candidates are ranked by the fp32 sum p + b, and a group's score is the fp32 sum
    of its two largest biased scores (the larger first; one score for groups of one). The
    weights still come from p (``routing_weights``).

    Order and ties: slots are sorted by score descending; equal values go to the lower
    expert id (groups: the lower group id).

    Returns ``ids`` int32 [T, k], ``gap`` fp32 [T] = k-th minus (k+1)-th candidate score
    (+inf without a (k+1)-th candidate) and ``ggap`` fp32 [T] = the same gap between the
    last kept and the first dropped group score (+inf when every group is kept).
    """
    p = np.asarray(p, np.float32)
    T, E = p.shape
    if score_bias is not None:
        p = (p + np.asarray(score_bias, np.float32)[None, :]).astype(np.float32)
    ggap = np.full(T, np.inf, np.float32)
    if use_grouped_topk:
        G = int(num_expert_group)
        per = E // G
        grp = p.reshape(T, G, per)
        if score_bias is None:
            gs = grp.max(axis=2)
        else:
            top = -np.sort(-grp, axis=2)
            gs = top[:, :, 0] if per == 1 else (top[:, :, 0] + top[:, :, 1]).astype(np.float32)
        gorder = np.argsort(-gs, axis=1, kind="stable")
        if topk_group < G:
            gsorted = np.take_along_axis(gs, gorder, axis=1)
            ggap = (gsorted[:, topk_group - 1] - gsorted[:, topk_group]).astype(np.float32)
        keep = np.zeros((T, G), bool)
        np.put_along_axis(keep, gorder[:, :topk_group], True, axis=1)
        score = np.where(np.repeat(keep, per, axis=1), p, np.float32(-np.inf))
        ncand = topk_group * per
    else:
        score = p
        ncand = E
    order = np.argsort(-score, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)
    if top_k < ncand:
        ss = np.take_along_axis(score, order[:, top_k - 1:top_k + 1], axis=1)
        gap = (ss[:, 0] - ss[:, 1]).astype(np.float32)
    else:
        gap = np.full(T, np.inf, np.float32)
    return ids, gap, ggap


def routing_weights(p, ids, renormalize, routed_scaling_factor=1.0):
    """fp32 routing weights [T, k] of the chosen experts.

    ``w = p[ids]``; with ``renormalize`` (``routing_weights /= routing_weights.sum(...)``
    in ``MixtralMoE.forward``) divided by their sum, taken in slot order over all k global
    picks; then multiplied by ``routed_scaling_factor`` (``recursive_replace``).
    """
    w = np.take_along_axis(np.asarray(p, np.float32), ids.astype(np.int64), axis=1)
    if renormalize:
        s = w[:, 0].copy()
        for j in range(1, w.shape[1]):
            s = (s + w[:, j]).astype(np.float32)
        w = (w / s[:, None]).astype(np.float32)
    return (w * np.float32(routed_scaling_factor)).astype(np.float32)


def route_from_logits(logits, top_k, renormalize, use_grouped_topk=False, num_expert_group=1,
                      topk_group=1, routed_scaling_factor=1.0, scoring_func="softmax",
                      score_bias=None):
    """Scores (softmax or sigmoid) -> (grouped) top-k -> weights on given fp32 logits (logit
    bias already added); ``score_bias`` steers the choice only."""
    if scoring_func == "softmax":
        p = softmax_fp32(logits)
    elif scoring_func == "sigmoid":
        p = sigmoid_fp32(logits)
    else:
        raise ValueError(scoring_func)
    ids, gap, ggap = select_experts(p, top_k, use_grouped_topk, num_expert_group, topk_group,
                                    score_bias)
    w = routing_weights(p, ids, renormalize, routed_scaling_factor)
    return {"logits": np.asarray(logits, np.float32), "probs": p, "ids": ids, "weights": w,
            "gap": gap, "ggap": ggap}


def route(x, w_gate, top_k, renormalize, use_grouped_topk=False, num_expert_group=1,
          topk_group=1, routed_scaling_factor=1.0, logit_bias=None, scoring_func="softmax",
          score_bias=None):
    """Router: logits -> fp32 scores -> (grouped) top-k -> weights. Returns a dict."""
    return route_from_logits(router_logits(x, w_gate, logit_bias), top_k, renormalize,
                             use_grouped_topk, num_expert_group, topk_group,
                             routed_scaling_factor, scoring_func, score_bias)


SWIGLUOAI_ALPHA = 1.702
SWIGLUOAI_LIMIT = 7.0


def gated_mlp(x, w13, w2, activation="silu", b13=None, b2=None):
    """fp64 gated expert MLP on rows of x: W2 act(W1 x + b1, W3 x + b3) + b2.

    ``w13`` is [2I, H] with the W1 (gate) rows first and the W3 (up) rows after them, the
    packed ``gate_up_proj`` (E, 2I, H) of ``recursive_replace``; ``w2`` is [H, I].
    ``activation`` (``recursive_replace`` picks ``"silu"``, or ``"swigluoai"`` for gpt-oss;
    the page names the switch, not the formula):
      silu:      act(g, u) = g / (1 + exp(-g)) * u
      swigluoai: g' = min(g, 7), u' = clip(u, -7, 7), act = g' / (1 + exp(-1.702 g')) * (u' + 1)
                 (gpt-oss's clamped SwiGLU).
    ``b13`` [2I] (gate biases, then up biases) and ``b2`` [H] are the expert biases
    (``has_bias`` of ``recursive_replace``), or None.
    """
    x64 = np.asarray(x, np.float64)
    w13 = np.asarray(w13, np.float64)
    I = w13.shape[0] // 2
    g = x64 @ w13[:I].T
    u = x64 @ w13[I:].T
    if b13 is not None:
        b = np.asarray(b13, np.float64)
        g = g + b[:I]
        u = u + b[I:]
    with np.errstate(over="ignore"):
        if activation == "silu":
            a = g / (1.0 + np.exp(-g)) * u
        elif activation == "swigluoai":
            g = np.minimum(g, SWIGLUOAI_LIMIT)
            u = np.clip(u, -SWIGLUOAI_LIMIT, SWIGLUOAI_LIMIT)
            a = g / (1.0 + np.exp(-SWIGLUOAI_ALPHA * g)) * (u + 1.0)
        else:
            raise ValueError(activation)
    y = a @ np.asarray(w2, np.float64).T
    if b2 is not None:
        y = y + np.asarray(b2, np.float64)
    return y


def moe_forward_given_routing(x, ids, weights, expert_map, w13_local, w2_local,
                              shared_w13=None, shared_w2=None, activation="silu", b13_local=None,
                              b2_local=None):
    """One share's output [T, H] (fp64) for given routing, as ``MixtralMoE.forward`` does it.

    For each local expert (slot s of ``expert_map``): the per-token weight is the sum over
    the k slots of ``weights * (ids == expert)``; tokens with that expert get
    ``weight * MLP_s(x)`` added. Tokens that did not pick the expert would add 0 * MLP
    (page 1 runs every token through every local expert); they are skipped, which is
    the same value for finite inputs. Experts outside the share (map value -1)
    contribute nothing. The shared expert, if given, is added with weight 1 ("Expert
    Parallel" Step 5). ``w13_local[s]`` / ``w2_local[s]`` may be any per-slot sequence
    of arrays (converted one slot at a time). ``activation`` applies to every expert,
    shared included; the expert biases ``b13_local[s]`` / ``b2_local[s]`` (or None) belong to
    the routed experts, whose weighted output includes them.
    """
    x64 = np.asarray(x, np.float64)
    T, H = x64.shape
    ids = np.asarray(ids)
    wts = np.asarray(weights, np.float64)
    emap = np.asarray(expert_map)
    slots = emap[ids]
    out = np.zeros((T, H), np.float64)
    for s in range(int(emap.max(initial=-1)) + 1):
        hit = slots == s
        rows = np.nonzero(hit.any(axis=1))[0]
        if rows.size == 0:
            continue
        w_tok = (wts * hit).sum(axis=1)
        out[rows] += w_tok[rows, None] * gated_mlp(
            x64[rows], w13_local[s], w2_local[s], activation,
            None if b13_local is None else b13_local[s], None if b2_local is None else b2_local[s])
    if shared_w13 is not None:
        out += gated_mlp(x64, shared_w13, shared_w2, activation)
    return out


def moe_forward(x, w_gate, expert_map, w13_local, w2_local, top_k, renormalize,
                use_grouped_topk=False, num_expert_group=1, topk_group=1,
                routed_scaling_factor=1.0, logit_bias=None, shared_w13=None, shared_w2=None):
    """Route then combine: returns (out fp64 [T, H], routing dict)."""
    r = route(x, w_gate, top_k, renormalize, use_grouped_topk, num_expert_group, topk_group,
              routed_scaling_factor, logit_bias)
    out = moe_forward_given_routing(x, r["ids"], r["weights"], expert_map, w13_local, w2_local,
                                    shared_w13, shared_w2)
    return out, r


def moe_forward_per_token(x, ids, weights, expert_map, w13_local, w2_local,
                          shared_w13=None, shared_w2=None, activation="silu", b13_local=None,
                          b2_local=None):
    """The per-token definition, with Python loops (small inputs only).

    out[t] = sum over slots j whose expert is local of weights[t, j] * MLP(x[t]) (+ shared
    MLP), the per-token sum of weighted expert rows of ``_ep_forward`` Step 4. Each MLP is
    evaluated with explicit per-row dot products.
    """
    x64 = np.asarray(x, np.float64)
    T, H = x64.shape
    out = np.zeros((T, H), np.float64)
    emap = np.asarray(expert_map)

    def mlp_row(xt, w13, w2, b13=None, b2=None):
        w13 = np.asarray(w13, np.float64)
        w2 = np.asarray(w2, np.float64)
        I = w13.shape[0] // 2
        act = np.empty(I)
        for i in range(I):
            g = float(np.dot(w13[i], xt)) + (0.0 if b13 is None else float(b13[i]))
            u = float(np.dot(w13[I + i], xt)) + (0.0 if b13 is None else float(b13[I + i]))
            if activation == "swigluoai":
                g = min(g, SWIGLUOAI_LIMIT)
                u = max(-SWIGLUOAI_LIMIT, min(u, SWIGLUOAI_LIMIT))
                act[i] = g / (1.0 + math.exp(-SWIGLUOAI_ALPHA * g)) * (u + 1.0) \
                    if SWIGLUOAI_ALPHA * g > -700 else 0.0
            else:
                act[i] = g / (1.0 + np.exp(-g)) * u if g > -700 else 0.0
        return np.array([float(np.dot(w2[h], act)) + (0.0 if b2 is None else float(b2[h]))
                         for h in range(w2.shape[0])])

    for t in range(T):
        acc = np.zeros(H)
        for j in range(ids.shape[1]):
            s = int(emap[int(ids[t, j])])
            if s < 0:
                continue
            acc += float(weights[t, j]) * mlp_row(
                x64[t], w13_local[s], w2_local[s], None if b13_local is None else b13_local[s],
                None if b2_local is None else b2_local[s])
        if shared_w13 is not None:
            acc += mlp_row(x64[t], shared_w13, shared_w2)
        out[t] = acc
    return out


def align_permute(topk_local, num_local_experts, block_m):
    """Token-pair permutation by local expert, padded per expert to a multiple of block_m.

    The method's grouping of work by expert (the per-expert loop of ``MixtralMoE.forward``;
    the sort-and-gather before ``fused_experts`` in ``_ep_forward`` Step 2/3), laid out
    for a grouped GEMM. Pair id p = t * k + j. For each local slot e the pairs with
    ``topk_local == e`` are listed in increasing pair id; segment e starts at
    offsets[e] = sum over e' < e of ceil(count[e'] / block_m) * block_m; unused slots of a
    segment hold -1. ``pair_row[p]`` is the position of pair p (-1 if its expert is not
    local); ``block_expert[b]`` is the slot that owns rows [b*block_m, (b+1)*block_m).

    ``block_m == 0`` (variable row blocks): segments are padded to a multiple of 32 and each
    is cut into blocks of 256 rows, except that a last piece of at most 64 rows stays in the
    block before it (so a block has 32 to 320 rows). ``block_expert`` is then the block table:
    the number of blocks nb, then (slot, first row) of each block in row order, then -1 and
    num_padded, so that block b covers rows [table[2 + 2b], table[4 + 2b]).
    """
    tl = np.asarray(topk_local, np.int64).reshape(-1)
    E_l = int(num_local_experts)
    pairs = np.nonzero(tl >= 0)[0]
    order = np.argsort(tl[pairs], kind="stable")
    by_expert = pairs[order]
    counts = np.bincount(tl[pairs], minlength=E_l).astype(np.int64)
    gran = block_m if block_m > 0 else 32
    padded = -(-counts // gran) * gran
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)])
    num_padded = int(offsets[-1])
    sorted_pairs = np.full(num_padded, -1, np.int32)
    pair_row = np.full(tl.shape[0], -1, np.int32)
    for e in range(E_l):
        seg = by_expert[starts[e]:starts[e + 1]]
        sorted_pairs[offsets[e]:offsets[e] + counts[e]] = seg
        pair_row[seg] = offsets[e] + np.arange(counts[e])
    if block_m > 0:
        block_expert = np.repeat(np.arange(E_l, dtype=np.int32), padded // block_m)
    else:
        table = []
        for e in range(E_l):
            q, r = divmod(int(padded[e]), 256)
            n = q if (q >= 1 and r <= 64) else q + (1 if r > 0 else 0)
            table += [v for j in range(n) for v in (e, int(offsets[e]) + 256 * j)]
        block_expert = np.array([len(table) // 2] + table + [-1, num_padded], np.int32)
    return {"sorted_pairs": sorted_pairs, "block_expert": block_expert, "pair_row": pair_row,
            "num_padded": num_padded, "counts": counts.astype(np.int32),
            "offsets": offsets.astype(np.int32)}


def weight_bytes(n_experts, hidden, inter, dtype_bytes, layers=1):
    """Expert-weight bytes on one card: n * (2*I*H + H*I) * bytes * layers.

    The per-card memory arithmetic of the ep_fused_moe_patch.py docstring ("Memory layout
    comparison"): each expert holds a gate/up matrix (2I x H) and a down matrix (H x I)
    at the card's intermediate size.
    """
    return int(n_experts) * (2 * int(inter) * int(hidden) + int(hidden) * int(inter)) \
        * int(dtype_bytes) * int(layers)


def ep_dispatch(topk_ids, top_k, num_experts, ep_size):
    """Dispatch plan of the expert-parallel exchange: one send row per (token, destination rank).

    "ep_fused_moe_patch.py", ``_ep_forward`` Step 2: the destination rank of pair (t, j) is
    ``topk_ids[t, j] // (num_experts / ep_size)`` (contiguous expert shares, as ``_ep_init``
    sets them up); the work items are ordered by destination rank so that each rank's items
    are contiguous for the all-to-all, with a per-rank count. Here a token is sent to each of
    its destination ranks once (the pairs of token t that go to rank r share one row): pair
    (t, j) owns the row when no earlier slot j' < j of t goes to the same rank. Rows of one
    rank follow increasing token index.

    Returns ``send_pos`` [T*k] (the row of pair (t, j) when it owns one, else -1),
    ``send_token`` [n_send], ``counts`` [ep_size] and ``offsets`` [ep_size + 1].
    """
    ids = np.asarray(topk_ids, np.int64).reshape(-1, top_k)
    T = ids.shape[0]
    per = num_experts // ep_size
    dest = ids // per
    owner = np.zeros(ids.shape, bool)
    for j in range(top_k):
        owner[:, j] = np.all(dest[:, :j] != dest[:, j:j + 1], axis=1)
    counts = np.array([int(np.sum(owner & (dest == r))) for r in range(ep_size)], np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    send_pos = np.full(T * top_k, -1, np.int32)
    send_token = np.zeros(int(offsets[-1]), np.int32)
    for r in range(ep_size):
        tt, jj = np.nonzero(owner & (dest == r))  # row-major: increasing token index
        rows = offsets[r] + np.arange(tt.shape[0])
        send_pos[tt * top_k + jj] = rows
        send_token[rows] = tt
    return {"send_pos": send_pos, "send_token": send_token, "counts": counts.astype(np.int32),
            "offsets": offsets.astype(np.int32), "n_send": int(offsets[-1])}


def ep_pack(plan, x, topk_ids, topk_w, top_k, num_experts, ep_size):
    """Send buffers of the exchange, in the order of ``ep_dispatch``.

    ``_ep_forward`` Step 2 gathers each work item's hidden row, expert id and routing weight
    in destination order. A send row carries the token's hidden row, its k routing weights,
    and its k slots seen from the destination rank: the local expert index
    ``id - r * (num_experts / ep_size)`` for the slots that rank r owns, -1 for the others
    (``_ep_forward`` Step 3, ``recv_ids - start_expert``).
    """
    ids = np.asarray(topk_ids, np.int64).reshape(-1, top_k)
    w = np.asarray(topk_w, np.float32).reshape(-1, top_k)
    per = num_experts // ep_size
    tok = plan["send_token"].astype(np.int64)
    rank = np.searchsorted(plan["offsets"], np.arange(tok.shape[0]), side="right") - 1
    send_x = np.asarray(x)[tok]
    local = ids[tok] - rank[:, None] * per
    send_local = np.where((local >= 0) & (local < per), local, -1).astype(np.int32)
    return {"send_x": send_x, "send_local": send_local, "send_w": w[tok], "rank": rank}


def ep_combine(plan, recv_y, top_k):
    """Unpack of the exchange: out[t] = sum of the rows that token t's ranks sent back.

    ``_ep_forward`` Step 4: each rank returns, for every row it received, that token's
    weighted result over its own experts; the results go back to token order and are summed
    per token (the scatter-add). Here the sum runs over token t's send rows in slot order
    (the order of ``send_pos``), in fp64 on the upcast rows.
    """
    pos = plan["send_pos"].reshape(-1, top_k)
    recv = np.asarray(recv_y, np.float64)
    out = np.zeros((pos.shape[0], recv.shape[1] if recv.ndim == 2 else 0), np.float64)
    for j in range(top_k):
        sel = pos[:, j] >= 0
        out[sel] += recv[pos[sel, j]]
    return out


def eplb_tables(physical_to_logical, num_logical):
    """Replica tables of a physical placement (expert-parallel load balancing).

    ``update_physical_experts_metadata`` / ``recursive_replace`` (transformers MoE page):
    the layer has ``num_physical = num_logical + num_redundant`` physical experts, rank r
    holding physical ids ``[r * P_l, (r + 1) * P_l)``. ``physical_to_logical[q]`` is the
    logical expert whose weights physical expert q holds. Returns
    ``logical_to_physical`` [E, max_replicas] (the physical ids holding logical e in
    increasing order, -1 after the last) and ``replica_count`` [E].
    """
    p2l = np.asarray(physical_to_logical, np.int64)
    reps = [[int(q) for q in np.nonzero(p2l == e)[0]] for e in range(num_logical)]
    if any(len(r) == 0 for r in reps):
        raise ValueError("every logical expert needs a replica")
    width = max(len(r) for r in reps)
    l2p = np.full((num_logical, width), -1, np.int32)
    for e, r in enumerate(reps):
        l2p[e, :len(r)] = r
    return l2p, np.array([len(r) for r in reps], np.int32)


def eplb_local_slots(topk_ids, top_k, logical_to_physical, replica_count, phys_expert_map):
    """Local slot of every (token, slot) pair under a replicated placement.

    The pages name the redundant experts but give no rule for splitting a logical expert's
    tokens among its replicas; the reading here is round robin by token index: token t's
    pair with logical expert e goes to replica ``t mod replica_count[e]`` (deterministic,
    and an even split over consecutive tokens). That physical expert's entry of the share's
    physical expert map gives the local slot (-1 when another rank holds it).
    """
    ids = np.asarray(topk_ids, np.int64).reshape(-1, top_k)
    T = ids.shape[0]
    cnt = np.asarray(replica_count, np.int64)
    l2p = np.asarray(logical_to_physical, np.int64)
    pmap = np.asarray(phys_expert_map, np.int64)
    out = np.full(ids.shape, -1, np.int32)
    for t in range(T):
        for j in range(top_k):
            e = ids[t, j]
            q = l2p[e, t % cnt[e]]
            out[t, j] = pmap[q]
    return out


def moe_forward_given_slots(x, slots, weights, w13_local, w2_local, shared_w13=None,
                            shared_w2=None, activation="silu", b13_local=None, b2_local=None):
    """One share's output [T, H] (fp64) given each pair's local slot (-1: not this share).

    The same sum as ``moe_forward_given_routing`` with the slot of each pair given directly
    (a replicated placement picks the slot per token, not per logical expert).
    """
    x64 = np.asarray(x, np.float64)
    T, H = x64.shape
    sl = np.asarray(slots)
    wts = np.asarray(weights, np.float64)
    out = np.zeros((T, H), np.float64)
    for s in range(int(sl.max(initial=-1)) + 1):
        hit = sl == s
        rows = np.nonzero(hit.any(axis=1))[0]
        if rows.size == 0:
            continue
        w_tok = (wts * hit).sum(axis=1)
        out[rows] += w_tok[rows, None] * gated_mlp(
            x64[rows], w13_local[s], w2_local[s], activation,
            None if b13_local is None else b13_local[s], None if b2_local is None else b2_local[s])
    if shared_w13 is not None:
        out += gated_mlp(x64, shared_w13, shared_w2, activation)
    return out
