"""The routing comparison rules of the GPU parity tests, exercised on the CPU.

Each case feeds ``moe_case.check_routing`` a routing built from the oracle (standing in for the
GPU's) and checks that rounding-level differences pass and that planted mistakes fail: a weight
off by 1e-4, logits rounded to bf16, a swapped expert on a clear-gap token, a slot order
reversed, and, on near-tie tokens, a choice outside the tie band.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from moe_case import TIE_GAP, check_routing, reference_routing

W = wl.Workload("rules", 31, "routing rules", "bf16", (96,), 256, 16, 64, 4, True)
WG = wl.Workload("rules_g", 32, "grouped routing rules", "bf16", (96,), 256, 32, 64, 6, False,
                 use_grouped_topk=True, num_expert_group=8, topk_group=3,
                 routed_scaling_factor=16.0)


def _case(w, T=96, tie_rows=None):
    x = wl.x(w, T)
    gate = wl.gate(w).copy()
    if tie_rows is not None:  # two experts with the same gate row: their logits tie exactly
        a, b = tie_rows
        gate[b] = gate[a]
    xf, gf = wl.to_f32(x), wl.to_f32(gate)
    ref = oracle.route(xf, gf, w.top_k, w.renormalize, w.use_grouped_topk, w.num_expert_group,
                       w.topk_group, w.routed_scaling_factor)
    return x, gate, ref


def _route(w, logits):
    return oracle.route_from_logits(logits, w.top_k, w.renormalize, w.use_grouped_topk,
                                    w.num_expert_group, w.topk_group, w.routed_scaling_factor)


@pytest.mark.parametrize("w", [W, WG], ids=["plain", "grouped"])
def test_exact_routing_passes(w):
    x, gate, ref = _case(w)
    mism, _ = check_routing(w, ref["ids"], ref["weights"], ref, ref["logits"], x, gate)
    assert mism.size == 0


@pytest.mark.parametrize("w", [W, WG], ids=["plain", "grouped"])
def test_rounding_level_logit_noise_passes(w):
    """Logits a few fp32 ulps off (another summation order) and the weights they give."""
    x, gate, ref = _case(w)
    rng = np.random.default_rng(0)
    l = ref["logits"]
    noisy = (l + l * (rng.standard_normal(l.shape) * 8 * 2.0 ** -24)).astype(np.float32)
    own = _route(w, noisy)
    mism, _ = check_routing(w, own["ids"], own["weights"], ref, noisy, x, gate)
    ids_ref, w_ref = reference_routing(w, own["ids"], ref, mism)
    assert np.array_equal(np.sort(ids_ref, 1), np.sort(own["ids"], 1))


def test_planted_weight_error_fails():
    x, gate, ref = _case(W)
    bad = ref["weights"].copy()
    bad[5, 1] *= 1.0 + 1e-4
    with pytest.raises(AssertionError, match="routing weight"):
        check_routing(W, ref["ids"], bad, ref, ref["logits"], x, gate)


def test_bf16_rounded_logits_fail():
    """A kernel that rounded the router logits to bf16 is caught by the logit bound."""
    x, gate, ref = _case(W)
    l = ref["logits"]
    u = l.view(np.uint32)
    lb = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)
    own = _route(W, lb)
    with pytest.raises(AssertionError):
        check_routing(W, own["ids"], own["weights"], ref, lb, x, gate)


def test_swapped_expert_on_clear_gap_fails():
    x, gate, ref = _case(W)
    t = int(np.nonzero(ref["gap"] > 1e-3)[0][0])
    ids = ref["ids"].copy()
    ids[t, -1] = next(e for e in range(W.num_experts) if e not in ids[t])
    with pytest.raises(AssertionError, match="clear gap"):
        check_routing(W, ids, ref["weights"], ref, ref["logits"], x, gate)


def test_reversed_slot_order_fails():
    x, gate, ref = _case(W)
    p = ref["probs"]
    t = next(t for t in range(len(p)) if p[t, ref["ids"][t, 0]] - p[t, ref["ids"][t, 1]] > 1e-3)
    ids, wts = ref["ids"].copy(), ref["weights"].copy()
    ids[t, [0, 1]] = ids[t, [1, 0]]
    wts[t, [0, 1]] = wts[t, [1, 0]]
    with pytest.raises(AssertionError, match="score order"):
        check_routing(W, ids, wts, ref, ref["logits"], x, gate)


def test_near_tie_inside_the_band_passes_outside_fails():
    """Experts 3 and 5 share a gate row, so every token that picks one of them at the k-th slot
    has the other at exactly the same score: either choice is valid; a weaker one is not."""
    x, gate, ref = _case(W, tie_rows=(3, 5))
    ids = ref["ids"]
    rows = [t for t in range(len(ids)) if ref["gap"][t] < TIE_GAP
            and ids[t, -1] in (3, 5)]
    assert rows, "the duplicated gate row should create k-th/(k+1)-th ties"
    t = rows[0]
    alt = ids.copy()
    alt[t, -1] = 5 if ids[t, -1] == 3 else 3
    w_alt = ref["weights"].copy()
    w_alt[t] = oracle.routing_weights(ref["probs"][t:t + 1], alt[t:t + 1], W.renormalize,
                                      W.routed_scaling_factor)[0]
    mism, near = check_routing(W, alt, w_alt, ref, ref["logits"], x, gate)
    assert t in mism and near >= 1
    weak = ids.copy()
    p = ref["probs"][t]
    weak[t, -1] = int(min((e for e in range(W.num_experts) if e not in ids[t]), key=lambda e: p[e]))
    w_weak = ref["weights"].copy()
    w_weak[t] = oracle.routing_weights(ref["probs"][t:t + 1], weak[t:t + 1], W.renormalize,
                                       W.routed_scaling_factor)[0]
    with pytest.raises(AssertionError, match="left out"):
        check_routing(W, weak, w_weak, ref, ref["logits"], x, gate)


def test_near_tie_weights_must_match_the_chosen_ids():
    """On a differing near-tie token the weights are the oracle's weights of the GPU's ids."""
    x, gate, ref = _case(W, tie_rows=(3, 5))
    ids = ref["ids"]
    t = next(t for t in range(len(ids)) if ref["gap"][t] < TIE_GAP and ids[t, -1] in (3, 5))
    alt = ids.copy()
    alt[t, -1] = 5 if ids[t, -1] == 3 else 3
    bad = ref["weights"].copy()
    bad[t, -1] *= 1.01
    with pytest.raises(AssertionError, match="routing weight"):
        check_routing(W, alt, bad, ref, ref["logits"], x, gate)


def test_grouped_choice_from_a_dropped_group_fails():
    x, gate, ref = _case(WG)
    per = WG.num_experts // WG.num_expert_group
    t = int(np.nonzero((ref["ggap"] > 1e-3) & (ref["gap"] > 1e-3))[0][0])
    kept = set(int(i) // per for i in ref["ids"][t])
    dropped = next(g for g in range(WG.num_expert_group) if g not in kept)
    ids = ref["ids"].copy()
    ids[t, -1] = dropped * per
    with pytest.raises(AssertionError):
        check_routing(WG, ids, ref["weights"], ref, ref["logits"], x, gate)
