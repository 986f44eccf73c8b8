"""Helpers of the GPU parity tests: inputs on the device, the HIP path through the C ABI,
and the oracle's reference on the same seeded inputs.

Comparison rules (fixed in the tests, not tuned to the kernels):
  * routing ids are compared per token as sets, bit-exact, and in the oracle's slot order,
    except on tokens whose oracle k-th/(k+1)-th score gap (or, for grouped routing,
    last-kept/first-dropped group gap) is below 1e-6: those are counted (the test summary
    lists them per case), and where their sets differ the GPU's set must lie inside the tie
    band and their outputs are checked against the oracle fed the GPU's ids;
  * the GPU's fp32 router logits against the oracle's within 4 u sqrt(H) sum|x w| + 2 u |l|,
    and the routing weights against the oracle's own within a bound derived from each
    token's measured logit error (see weight_tolerance);
  * outputs: max|out - ref| / max|ref| <= 2e-2 for bf16 and <= 1e-4 for fp32.
"""
from __future__ import annotations

import numpy as np
import torch

import expert_moe_amd as moe
import oracle
import workloads as wl

TIE_GAP = 1e-6
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}
# router logits: multiple of the probabilistic fp32 summation bound u * sqrt(H) * sum |x w|
LOGIT_C = 4.0
# near-tie tokens per checked case: label -> (near-tie tokens, of them with a differing set, T)
NEAR_TIES = {}


def dev_tensor(a: np.ndarray, device="cuda"):
    """numpy workload array -> device tensor (uint16 arrays are bf16 bit patterns)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def torch_dtype(w: wl.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def params(w: wl.Workload, **over) -> moe.moe_params:
    kw = dict(num_experts=w.num_experts, top_k=w.top_k, hidden_size=w.hidden_size,
              intermediate_size=w.intermediate_size, renormalize=w.renormalize,
              use_grouped_topk=w.use_grouped_topk, num_expert_group=w.num_expert_group,
              topk_group=w.topk_group, routed_scaling_factor=w.routed_scaling_factor,
              num_local_experts=w.num_local_experts,
              shared_intermediate_size=w.shared_intermediate_size, dtype=w.dtype,
              scoring_func=w.scoring_func, activation=w.activation)
    kw.update(over)
    return moe.make_params(**kw)


class Layer:
    """Host (numpy) and device copies of one share's inputs for T tokens."""

    def __init__(self, w: wl.Workload, T: int, device="cuda", host_weights=True):
        self.w, self.T = w, T
        self.x = wl.x(w, T)
        self.gate = wl.gate(w)
        self.bias = wl.logit_bias(w)
        self.sbias = wl.score_bias(w)
        self.emap = wl.expert_map(w)
        self.w13, self.w2 = wl.local_expert_weights(w)
        self.sw13, self.sw2 = wl.shared_weights(w)
        self.b13, self.b2 = wl.expert_biases(w)
        self.d = {
            "x": dev_tensor(self.x, device), "gate": dev_tensor(self.gate, device),
            "bias": None if self.bias is None else dev_tensor(self.bias, device),
            "sbias": None if self.sbias is None else dev_tensor(self.sbias, device),
            "emap": dev_tensor(self.emap, device),
            "w13": dev_tensor(self.w13, device), "w2": dev_tensor(self.w2, device),
            "sw13": None if self.sw13 is None else dev_tensor(self.sw13, device),
            "sw2": None if self.sw2 is None else dev_tensor(self.sw2, device),
            "b13": None if self.b13 is None else dev_tensor(self.b13, device),
            "b2": None if self.b2 is None else dev_tensor(self.b2, device),
        }
        if not host_weights:
            self.w13 = self.w2 = None

    def forward(self, p=None, with_shared=True):
        """The HIP path through moe_forward. Returns (out f32 numpy, ids, weights)."""
        w, T, d = self.w, self.T, self.d
        p = p or params(w)
        dev = d["x"].device
        out = torch.empty(T, w.hidden_size, dtype=torch_dtype(w), device=dev)
        ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
        tw = torch.empty(T, w.top_k, dtype=torch.float32, device=dev)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
        sw13 = d["sw13"] if with_shared else None
        sw2 = d["sw2"] if with_shared else None
        moe.moe_forward(p, T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"], d["w2"], sw13, sw2,
                        out, ids, tw, ws, score_bias=d["sbias"], b13=d["b13"], b2=d["b2"])
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), ids.cpu().numpy(), tw.cpu().numpy()

    def gpu_route(self):
        """moe_route on the layer: (ids, weights, logits) as numpy arrays."""
        w, T, d = self.w, self.T, self.d
        p = params(w)
        dev = d["x"].device
        ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
        tw = torch.empty(T, w.top_k, dtype=torch.float32, device=dev)
        local = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
        moe.moe_route(p, T, d["x"], d["gate"], d["bias"], d["emap"], ids, tw, local, ws,
                      score_bias=d["sbias"])
        torch.cuda.synchronize()
        logits = ws[: T * w.num_experts * 4].view(torch.float32).view(T, w.num_experts)
        return ids.cpu().numpy(), tw.cpu().numpy(), logits.cpu().numpy()

    def check_routing(self, ids, tw, ref):
        """Routing rules on the forward's ids/weights, with moe_route's logits for the weights."""
        r_ids, r_tw, logits = self.gpu_route()
        assert np.array_equal(r_ids, ids) and np.array_equal(r_tw, tw), \
            "moe_route and moe_forward disagree"
        return check_routing(self.w, ids, tw, ref, logits, self.x, self.gate, self.bias,
                             label=f"{self.w.key} T={self.T}")

    def oracle_route(self, rows=None):
        w = self.w
        x = wl.to_f32(self.x if rows is None else self.x[rows])
        return oracle.route(x, wl.to_f32(self.gate), w.top_k, w.renormalize, w.use_grouped_topk,
                            w.num_expert_group, w.topk_group, w.routed_scaling_factor, self.bias,
                            w.scoring_func, self.sbias)

    def oracle_out(self, rows, ids, weights, with_shared=True):
        w = self.w
        w13 = _LazyF32(self.w13)
        w2 = _LazyF32(self.w2)
        sh = (wl.to_f32(self.sw13), wl.to_f32(self.sw2)) if (with_shared and self.sw13 is not None) \
            else (None, None)
        return oracle.moe_forward_given_routing(wl.to_f32(self.x[rows]), ids, weights, self.emap,
                                                w13, w2, sh[0], sh[1], w.activation, self.b13,
                                                self.b2)


class _LazyF32:
    """Per-slot float32 view of a packed [E_l, ...] workload array (converted on access)."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, s):
        return wl.to_f32(self.a[s])

    def __len__(self):
        return len(self.a)


def selection_scores(w: wl.Workload, ref):
    """The scores the top-k ranks (the oracle's fp32 p, plus the selection bias when there is one)."""
    sb = wl.score_bias(w)
    p = ref["probs"]
    return p if sb is None else (p + sb[None, :].astype(np.float32)).astype(np.float32)


def _group_scores(w: wl.Workload, s_row):
    """Group scores of one token (largest score, or with a selection bias the sum of the two
    largest), as the oracle's select_experts defines them."""
    grp = s_row.reshape(w.num_expert_group, -1)
    if wl.score_bias(w) is None:
        return grp.max(axis=1)
    top = -np.sort(-grp, axis=1)
    return top[:, 0] if grp.shape[1] == 1 else (top[:, 0] + top[:, 1]).astype(np.float32)


def check_tie_band(w: wl.Workload, t: int, gpu_ids, s_row):
    """A near-tie token whose GPU set differs from the oracle's: the GPU set must be a top-k of
    the oracle's scores under some resolution of the ties within TIE_GAP. Grouped routing: the
    groups the GPU drew from must be keepable (each within TIE_GAP of the last kept group score,
    and every group clearly above it kept), and inside the kept groups no excluded expert may
    beat the weakest chosen one by more than TIE_GAP."""
    E = w.num_experts
    g_ids = np.asarray(gpu_ids, np.int64)
    assert np.unique(g_ids).size == g_ids.size, f"token {t}: repeated expert ids {g_ids}"
    assert np.all((g_ids >= 0) & (g_ids < E)), f"token {t}: expert ids out of range {g_ids}"
    cand = np.ones(E, bool)
    if w.use_grouped_topk:
        per = E // w.num_expert_group
        gsc = _group_scores(w, s_row)
        kth = np.sort(gsc)[::-1][w.topk_group - 1]
        used = np.unique(g_ids // per)
        assert used.size <= w.topk_group, f"token {t}: experts from {used.size} groups"
        assert np.all(gsc[used] >= kth - TIE_GAP), f"token {t}: a dropped group was used"
        forced = np.nonzero(gsc > kth + TIE_GAP)[0]
        kept = list(dict.fromkeys([int(g) for g in forced] + [int(g) for g in used]))
        assert len(kept) <= w.topk_group, f"token {t}: a clearly kept group was dropped"
        # fill with the other keepable groups whose best expert is weakest (the most lenient
        # valid choice for the check below)
        rest = [int(g) for g in np.nonzero(gsc >= kth - TIE_GAP)[0] if int(g) not in kept]
        rest.sort(key=lambda g: float(s_row[g * per:(g + 1) * per].max()))
        kept += rest[:w.topk_group - len(kept)]
        cand = np.zeros(E, bool)
        for g in kept:
            cand[g * per:(g + 1) * per] = True
    assert np.all(cand[g_ids]), f"token {t}: an expert outside the kept groups was chosen"
    chosen = np.zeros(E, bool)
    chosen[g_ids] = True
    weakest = float(s_row[g_ids].min())
    others = s_row[cand & ~chosen]
    if others.size:
        assert float(others.max()) <= weakest + TIE_GAP, \
            f"token {t}: an expert scoring {others.max()} was left out for one scoring {weakest}"


def weight_tolerance(w: wl.Workload, w_ref, dmax):
    """Bound on |w_gpu - w_oracle| per routing weight from the fp32 arithmetic between them.

    With logits off by at most dmax (per token, measured), softmax gives
    |dp_j| / p_j <= |dl_j| + sum_e p_e |dl_e| <= 2 dmax (the sigmoid's (1 - p) dl is smaller),
    and renormalising over the k picks doubles the relative error. Rounding adds, relative to
    the weight: two exp ulps a side, the E-term sum (at most (E - 1) u in any order), the
    division, the k-term renormalising sum and its division, the routed scale: under
    (2E + k + 16) u. So |dw| <= |w| (4 dmax + (2E + k + 16) u), u = 2^-24.
    """
    u = 2.0 ** -24
    rel = 4.0 * dmax[:, None] + (2 * w.num_experts + w.top_k + 16) * u
    return np.abs(w_ref).astype(np.float64) * rel + 1e-30


def check_routing(w: wl.Workload, ids, weights, ref, logits=None, x=None, gate=None, bias=None,
                  label=None):
    """Apply the routing comparison rules. Returns (exempt_mismatch_rows, n_near_ties).

    ids: the GPU's per-token sets equal the oracle's, bit-exact, on every token whose oracle
      k-th/(k+1)-th score gap (and group gap) is at least TIE_GAP. Where the sets agree the slot
      order is the oracle's too (score descending, equal scores to the lower id), except that
      adjacent chosen experts whose oracle scores are within TIE_GAP may come in either order.
      Near-tie tokens whose sets differ are checked against the tie band (check_tie_band).
    logits (needed for the weight checks): the GPU's fp32 logits against the oracle's
      correctly rounded ones, within LOGIT_C * u * sqrt(H) * sum_h |x_h w_eh| + 2 u |l| (the
      probabilistic bound of fp32 summation over H terms, plus the bias add and final rounding).
    weights: against the oracle's own weights (its logits, softmax, top-k, renormalise and
      scale), each within weight_tolerance() of its token's measured logit error; on near-tie
      tokens whose sets differ, against the oracle's weights of the GPU's ids.
    """
    T, k = ids.shape
    near = (ref["gap"] < TIE_GAP) | (ref["ggap"] < TIE_GAP)
    s = selection_scores(w, ref)
    gs = np.sort(ids, axis=1)
    rs = np.sort(ref["ids"], axis=1)
    differ = np.any(gs != rs, axis=1)
    bad = np.nonzero(differ & ~near)[0]
    assert bad.size == 0, f"routing ids differ on {bad.size} tokens with a clear gap, e.g. {bad[:5]}"
    # slot order where the sets agree
    for t in np.nonzero(~differ & np.any(ids != ref["ids"], axis=1))[0]:
        sc = s[t, ids[t]]
        assert np.all(sc[:-1] >= sc[1:] - TIE_GAP), f"token {t}: slots not in score order {ids[t]}"
        eq = sc[:-1] == sc[1:]
        assert np.all(ids[t][:-1][eq] < ids[t][1:][eq]), f"token {t}: equal scores not in id order"
    mism = np.nonzero(differ)[0]
    for t in mism:
        check_tie_band(w, int(t), ids[t], s[t])
    if logits is not None:
        u = 2.0 ** -24
        l_gpu = logits.astype(np.float32)
        if bias is not None:
            l_gpu = (l_gpu + bias[None, :].astype(np.float32)).astype(np.float32)
        l_gpu = l_gpu.astype(np.float64)
        l_ref = ref["logits"].astype(np.float64)
        xs = np.abs(wl.to_f32(x).astype(np.float64))
        gabs = np.abs(wl.to_f32(gate).astype(np.float64))
        bound = LOGIT_C * u * np.sqrt(w.hidden_size) * (xs @ gabs.T) + 2 * u * np.abs(l_ref) + 1e-30
        dl = np.abs(l_gpu - l_ref)
        worst = float(np.max(dl / bound))
        assert worst <= 1.0, f"router logits off by {worst:.3g} x the fp32 summation bound"
        dmax = dl.max(axis=1)
        # expected weights: the oracle's, matched to the GPU's slots by expert id where the sets
        # agree; the oracle's weights of the GPU's own ids on near-tie tokens whose sets differ
        w_exp = np.empty_like(weights)
        agree = np.nonzero(~differ)[0]
        if agree.size:
            pos = np.argsort(ref["ids"][agree], axis=1, kind="stable")
            sorted_ids = np.take_along_axis(ref["ids"][agree], pos, axis=1)
            sorted_w = np.take_along_axis(ref["weights"][agree], pos, axis=1)
            inv = np.argsort(np.argsort(ids[agree], axis=1, kind="stable"), axis=1, kind="stable")
            w_exp[agree] = np.take_along_axis(sorted_w, inv, axis=1)
            assert np.array_equal(np.take_along_axis(sorted_ids, inv, axis=1), ids[agree])
        if mism.size:
            w_exp[mism] = oracle.routing_weights(ref["probs"][mism], ids[mism], w.renormalize,
                                                 w.routed_scaling_factor)
        tol = weight_tolerance(w, w_exp, dmax)
        err = np.abs(weights.astype(np.float64) - w_exp.astype(np.float64))
        over = err / tol
        i = np.unravel_index(int(np.argmax(over)), over.shape)
        assert float(over[i]) <= 1.0, \
            f"routing weight of token {i[0]} slot {i[1]}: |dw| = {err[i]:.3g} > {tol[i]:.3g}"
    n_near = int(near.sum())
    if label is not None:
        NEAR_TIES[label] = (n_near, int(mism.size), int(T))
    return mism, n_near


def reference_routing(w: wl.Workload, ids, ref, mismatch_rows):
    """Oracle routing, with the GPU's ids (and the oracle's weights of those ids) on the near-tie
    tokens whose sets differ."""
    ids_ref = ref["ids"].copy()
    w_ref = ref["weights"].copy()
    if len(mismatch_rows):
        ids_ref[mismatch_rows] = ids[mismatch_rows]
        w_ref[mismatch_rows] = oracle.routing_weights(ref["probs"][mismatch_rows], ids[mismatch_rows],
                                                      w.renormalize, w.routed_scaling_factor)
    return ids_ref, w_ref


def rel_err(out, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(out - ref)) / (den if den > 0 else 1.0))


def sample_rows(ids, emap, T, n=512, seed=0):
    """>= n seeded token rows that cover every local expert routed at least once."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    slots = emap[ids]
    for s in range(int(emap.max()) + 1):
        hit = np.nonzero((slots == s).any(axis=1))[0]
        if hit.size:
            rows.add(int(hit[0]))
            rows.add(int(hit[-1]))
    return np.array(sorted(rows), dtype=np.int64)


def slot_of_row(table, r, block_m):
    """Slot that owns sorted row r (block_m rows per block, or the variable block table)."""
    if block_m > 0:
        return table[r // block_m]
    nb = table[0]
    starts = table[2:3 + 2 * nb:2]
    b = int(np.searchsorted(starts, r, side="right")) - 1
    return table[1 + 2 * b]
