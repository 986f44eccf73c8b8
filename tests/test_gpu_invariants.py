"""GPU cases of the method's closed-form invariants (each is also a pin of the oracle):

* top_k = E with renormalisation: every token takes every expert, so the layer is the dense
  softmax-weighted mixture sum_e p_e MLP_e(x) (the per-expert loop of MixtralMoE.forward with
  all experts selected; "[Feature] Expert parallelism support");
* E = 1: one expert with weight exactly 1, so the layer is a plain gated MLP;
* grouped top-k keeping every group (keep = G), or with one group (G = 1): no expert is ever
  excluded, so routing equals plain top-k (the n_group / topk_group switches of
  recursive_replace on "vllm.model_executor.models.transformers.moe").

All through the C ABI, against the oracle, on every token; sizes span several tiles and end
in a ragged tail.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from moe_case import OUT_TOL, Layer, params, reference_routing, rel_err

pytestmark = pytest.mark.gpu

W = wl.Workload


def _forward(w, T):
    layer = Layer(w, T)
    out, ids, tw = layer.forward()
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    return layer, out, ids, tw, ref, mism


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_all_is_dense_mixture(dtype):
    w = W("topk_all_" + dtype, 41, "top-k of all experts", dtype, (203,), 256, 8, 192, 8, True)
    T = 203
    layer, out, ids, tw, ref, mism = _forward(w, T)
    assert mism.size == 0  # no (k+1)-th candidate: no tie can change the set
    assert np.array_equal(np.sort(ids, 1), np.tile(np.arange(8), (T, 1)))
    x = wl.to_f32(layer.x)
    p = oracle.softmax_fp32(oracle.router_logits(x, wl.to_f32(layer.gate))).astype(np.float64)
    mix = np.zeros((T, w.hidden_size))
    for e in range(w.num_experts):
        mix += p[:, e:e + 1] * oracle.gated_mlp(x, wl.to_f32(layer.w13[e]), wl.to_f32(layer.w2[e]))
    err = rel_err(out, mix)
    print(f"[{w.key}] dense-mixture rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[dtype], err


def test_single_expert_is_plain_mlp():
    w = W("one_expert", 42, "one expert", "bf16", (150,), 192, 1, 320, 1, True)
    T = 150
    layer, out, ids, tw, ref, mism = _forward(w, T)
    assert np.all(ids == 0)
    assert np.all(tw == 1.0)
    want = oracle.gated_mlp(wl.to_f32(layer.x), wl.to_f32(layer.w13[0]), wl.to_f32(layer.w2[0]))
    err = rel_err(out, want)
    print(f"[one_expert] plain-MLP rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL["bf16"], err


@pytest.mark.parametrize("groups,keep", [(4, 4), (1, 1), (8, 8)])
def test_grouped_without_exclusion_is_plain_topk(groups, keep):
    base = W("plain_16", 43, "plain top-4 of 16", "bf16", (260,), 256, 16, 128, 4, False,
             routed_scaling_factor=2.5)
    grouped = W(f"grouped_{groups}_{keep}", 43, "grouped, nothing excluded", "bf16", (260,), 256,
                16, 128, 4, False, use_grouped_topk=True, num_expert_group=groups,
                topk_group=keep, routed_scaling_factor=2.5)
    T = 260
    lp, out_p, ids_p, tw_p, ref_p, mism_p = _forward(base, T)
    lg, out_g, ids_g, tw_g, ref_g, mism_g = _forward(grouped, T)
    # same seed and shapes: same inputs; the GPU's grouped routing is its plain routing
    assert np.array_equal(lp.x, lg.x) and np.array_equal(lp.gate, lg.gate)
    assert np.array_equal(ids_g, ids_p) and np.array_equal(tw_g, tw_p)
    assert np.array_equal(out_g, out_p)
    # and the oracle's grouped routing is its plain routing
    assert np.array_equal(ref_g["ids"], ref_p["ids"])
    ids_ref, w_ref = reference_routing(base, ids_p, ref_p, mism_p)
    want = lp.oracle_out(np.arange(T), ids_ref, w_ref)
    err = rel_err(out_p, want)
    print(f"[grouped G={groups} keep={keep}] rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL["bf16"], err
