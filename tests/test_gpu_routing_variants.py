"""GPU parity of the routing variants (sigmoid scores, selection-only score bias, group score
as the sum of the two largest biased scores) against the oracle, through the C ABI.

The comparison rules are those of ``moe_case``: routing ids bit-exact except on near-tie
tokens (the oracle's gaps are taken on the biased selection scores), routing weights within
the derived bounds on the GPU's own logits, outputs within the dtype tolerance.
"""
import numpy as np
import pytest

import workloads as wl
from moe_case import OUT_TOL, Layer, reference_routing, rel_err, sample_rows

pytestmark = pytest.mark.gpu

W = wl.Workload
CASES = {
    # DeepSeek-V3-like: sigmoid, bias, 8 groups keep 4, top-8, rsf 2.5, shared expert, EP share
    "v3_s": (W("v3_s", 21, "small V3-like", "bf16", (300,), 256, 64, 128, 8, True,
               use_grouped_topk=True, num_expert_group=8, topk_group=4,
               routed_scaling_factor=2.5, ep_size=8, ep_rank=0, shared_intermediate_size=256,
               scoring_func="sigmoid", score_bias_std=0.05), 300),
    # 256 experts (four experts per lane), groups of 32
    "v3_e256": (W("v3_e256", 22, "V3-like, 256 experts", "bf16", (200,), 128, 256, 64, 8, True,
                  use_grouped_topk=True, num_expert_group=8, topk_group=4,
                  routed_scaling_factor=2.5, ep_size=32, ep_rank=3,
                  scoring_func="sigmoid", score_bias_std=0.05), 200),
    # sigmoid, plain top-k, no bias, no renormalisation
    "sig_plain": (W("sig_plain", 23, "sigmoid plain", "bf16", (257,), 192, 32, 128, 4, False,
                    scoring_func="sigmoid"), 257),
    # softmax with a selection bias, plain and grouped
    "sm_bias": (W("sm_bias", 24, "softmax + bias", "bf16", (129,), 256, 64, 128, 6, True,
                  ep_size=4, ep_rank=2, score_bias_std=0.01), 129),
    "sm_bias_grp": (W("sm_bias_grp", 25, "softmax + bias, grouped", "bf16", (211,), 256, 64, 128,
                      6, True, use_grouped_topk=True, num_expert_group=8, topk_group=3,
                      score_bias_std=0.01), 211),
    # fp32, groups of two experts (top-2 sum = the whole group)
    "v3_f32": (W("v3_f32", 26, "V3-like fp32", "f32", (45,), 128, 16, 128, 4, True,
                 use_grouped_topk=True, num_expert_group=8, topk_group=3,
                 scoring_func="sigmoid", score_bias_std=0.05), 45),
    # groups of one expert with a bias: the group rule reduces to the plain top-k
    "g1_bias": (W("g1_bias", 27, "groups of one", "bf16", (64,), 128, 16, 64, 3, True,
                  use_grouped_topk=True, num_expert_group=16, topk_group=5,
                  scoring_func="sigmoid", score_bias_std=0.1), 64),
}


def _check(layer, rows=None, with_shared=True):
    w = layer.w
    out, ids, tw = layer.forward(with_shared=with_shared)
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = np.arange(layer.T) if rows is None else rows
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows], with_shared)
    err = rel_err(out[rows], want)
    print(f"[{w.key} T={layer.T}] rel_err={err:.3e} near_ties={near} exempt={mism.size}",
          flush=True)
    assert err <= OUT_TOL[w.dtype], err
    return ids, tw


@pytest.mark.parametrize("case", sorted(CASES))
def test_routing_variant_layer(case):
    w, T = CASES[case]
    _check(Layer(w, T))


@pytest.mark.parametrize("T", [1, 2, 5])
def test_routing_variant_decode_sizes(T):
    w, _ = CASES["v3_s"]
    _check(Layer(w, T))


def test_bias_changes_the_choice():
    """The selection bias is live: with it removed, some tokens pick other experts, and the
    weights of experts picked both ways are unchanged by it (they come from the scores)."""
    w, T = CASES["v3_s"]
    lay_b = Layer(w, T)
    ids_b, tw_b, _ = lay_b.gpu_route()
    w0 = W(**{**w.__dict__, "score_bias_std": 0.0})
    lay_0 = Layer(w0, T)
    ids_0, tw_0, _ = lay_0.gpu_route()
    assert not np.array_equal(np.sort(ids_b, 1), np.sort(ids_0, 1))
    # without renormalisation the weight of a chosen expert is its own scaled score
    wn = W(**{**w.__dict__, "renormalize": False})
    wn0 = W(**{**wn.__dict__, "score_bias_std": 0.0})
    ib, tb, _ = Layer(wn, T).gpu_route()
    i0, t0, _ = Layer(wn0, T).gpu_route()
    for t in range(T):
        a = dict(zip(ib[t].tolist(), tb[t].tolist()))
        b = dict(zip(i0[t].tolist(), t0[t].tolist()))
        for e in set(a) & set(b):
            assert a[e] == b[e]


@pytest.mark.parametrize("T", [32, 4096])
def test_dsv3_full_size(T):
    """The DeepSeek-V3-shaped share: routing on every token, outputs on every token (T=32) or
    on >= 512 sampled rows that cover every local expert (T=4096)."""
    w = wl.WORKLOADS["dsv3"]
    layer = Layer(w, T)
    out, ids, tw = layer.forward()
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = np.arange(T) if T <= 256 else sample_rows(ids, layer.emap, T)
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows])
    err = rel_err(out[rows], want)
    print(f"[dsv3 T={T}] rel_err={err:.3e} near_ties={near} exempt={mism.size} rows={len(rows)}",
          flush=True)
    assert err <= OUT_TOL[w.dtype], err

