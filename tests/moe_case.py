"""Helpers of the GPU parity tests: inputs on the device, the HIP path through the C ABI,
and the oracle's reference on the same seeded inputs.

Comparison rules (fixed in the tests, not tuned to the kernels):
  * routing ids are compared per token as sets, bit-exact, except on tokens whose oracle
    k-th/(k+1)-th probability gap (or, for grouped routing, last-kept/first-dropped group
    gap) is below 1e-6; those are counted and their outputs are checked against the oracle
    fed the GPU's own ids and weights;
  * routing weights, in two stages derived from the arithmetic (see check_routing): the GPU's
    fp32 logits against the oracle's correctly rounded ones within the recursive-summation
    error bound, then the GPU's weights against the oracle's softmax / top-k / renormalise /
    scale applied to those same GPU logits, |dw| <= 1e-6 * max(1, routed_scaling_factor);
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
        return check_routing(self.w, ids, tw, ref, logits, self.x, self.gate, self.bias)

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


def check_routing(w: wl.Workload, ids, weights, ref, logits=None, x=None, gate=None, bias=None):
    """Apply the routing comparison rules. Returns (exempt_mismatch_rows, n_near_ties).

    ids: GPU ids vs the oracle's, as sets, bit-exact except on near-tie tokens.
    weights (when the GPU logits are given): two stages derived from the arithmetic.
      1. GPU logits vs the oracle's correctly rounded fp32 logits: recursive-summation bound
         |dl| <= H * u * sum_h |x_h w_eh| + 2 u |l| (bias add, final rounding), u = 2^-24.
      2. GPU weights vs the oracle's softmax / top-k / renormalise / scale applied to the GPU's
         own logits: |dw| <= 1e-6 * max(1, rsf) (exp and summation-order rounding only).
    """
    near = (ref["gap"] < TIE_GAP) | (ref["ggap"] < TIE_GAP)
    gs = np.sort(ids, axis=1)
    rs = np.sort(ref["ids"], axis=1)
    differ = np.any(gs != rs, axis=1)
    bad = np.nonzero(differ & ~near)[0]
    assert bad.size == 0, f"routing ids differ on {bad.size} tokens with a clear gap, e.g. {bad[:5]}"
    if logits is not None:
        u = 2.0 ** -24
        l_gpu = logits.astype(np.float64)
        if bias is not None:
            l_gpu = (logits + bias[None, :].astype(np.float32)).astype(np.float64)
        xs = np.abs(wl.to_f32(x).astype(np.float64))
        gabs = np.abs(wl.to_f32(gate).astype(np.float64))
        bound = w.hidden_size * u * (xs @ gabs.T) + 2 * u * np.abs(l_gpu) + 1e-30
        dl = np.abs(l_gpu - ref["logits"].astype(np.float64))
        worst = float(np.max(dl / bound))
        assert worst <= 1.0, f"router logits off by {worst:.3g} x the fp32 summation bound"
        own = oracle.route_from_logits(l_gpu.astype(np.float32), w.top_k, w.renormalize,
                                       w.use_grouped_topk, w.num_expert_group, w.topk_group,
                                       w.routed_scaling_factor, w.scoring_func, wl.score_bias(w))
        near_own = (own["gap"] < TIE_GAP) | (own["ggap"] < TIE_GAP)
        same_own = np.all(np.sort(own["ids"], 1) == gs, axis=1)
        assert np.all(same_own | near_own), "ids differ from the oracle's top-k of the GPU logits"
        sel = same_own
        o_g = np.argsort(ids[sel], axis=1, kind="stable")
        o_r = np.argsort(own["ids"][sel], axis=1, kind="stable")
        wg = np.take_along_axis(weights[sel], o_g, axis=1)
        wr = np.take_along_axis(own["weights"][sel], o_r, axis=1)
        err = float(np.max(np.abs(wg - wr))) if wg.size else 0.0
        tol = TIE_GAP * max(1.0, abs(w.routed_scaling_factor))
        assert err <= tol, f"routing weights differ by {err} > {tol} on the same logits"
    return np.nonzero(differ)[0], int(near.sum())


def reference_routing(ids, weights, ref, mismatch_rows):
    """Oracle routing, with the GPU's routing on exempt mismatched tokens."""
    ids_ref = ref["ids"].copy()
    w_ref = ref["weights"].copy()
    ids_ref[mismatch_rows] = ids[mismatch_rows]
    w_ref[mismatch_rows] = weights[mismatch_rows]
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
