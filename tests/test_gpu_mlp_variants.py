"""GPU parity of the MLP variants (gpt-oss's clamped SwiGLU, expert biases on the gate/up
pre-activations and the expert output) against the oracle, through the C ABI: every kernel
family (LDS tiles of 64/128/256 rows with quarter-tile tails, weight-streaming tiles, the fp32
tile) with each epilogue. Comparison rules are those of ``moe_case``.
"""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import oracle
import workloads as wl
from moe_case import OUT_TOL, Layer, params, reference_routing, rel_err, sample_rows, slot_of_row

pytestmark = pytest.mark.gpu

W = wl.Workload
CASES = {
    # clamped SwiGLU with large biases (past the clamps), top-4 of 32, EP share
    "oai_bias": (W("oai_bias", 31, "swigluoai + biases", "bf16", (300,), 256, 32, 128, 4, True,
                   ep_size=2, ep_rank=1, activation="swigluoai", expert_bias_std=3.0), 300),
    # silu with biases and a shared expert (the shared expert has none)
    "silu_bias": (W("silu_bias", 32, "silu + biases", "bf16", (257,), 192, 16, 192, 2, True,
                    shared_intermediate_size=128, expert_bias_std=0.5), 257),
    # clamped SwiGLU without biases, grouped routing
    "oai_grp": (W("oai_grp", 33, "swigluoai, grouped", "bf16", (200,), 320, 32, 192, 6, False,
                  use_grouped_topk=True, num_expert_group=8, topk_group=3,
                  routed_scaling_factor=16.0, ep_size=8, ep_rank=0, shared_intermediate_size=384,
                  activation="swigluoai"), 200),
    # fp32 tile path
    "oai_f32": (W("oai_f32", 34, "swigluoai + biases fp32", "f32", (45,), 128, 8, 256, 2, True,
                  activation="swigluoai", expert_bias_std=2.0), 45),
    # 256-row tiles with odd K steps and quarter-tile tails
    "oai_large": (W("oai_large", 35, "swigluoai + biases, large tiles", "bf16", (2400,), 192, 4,
                    320, 2, True, activation="swigluoai", expert_bias_std=1.0), 2400),
}


def _check(layer, rows=None):
    w = layer.w
    out, ids, tw = layer.forward()
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = np.arange(layer.T) if rows is None else rows
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows])
    err = rel_err(out[rows], want)
    print(f"[{w.key} T={layer.T}] rel_err={err:.3e} near_ties={near} exempt={mism.size}",
          flush=True)
    assert err <= OUT_TOL[w.dtype], err


@pytest.mark.parametrize("case", sorted(CASES))
def test_mlp_variant_layer(case):
    w, T = CASES[case]
    _check(Layer(w, T))


@pytest.mark.parametrize("T", [1, 3, 7])
def test_mlp_variant_decode_sizes(T):
    """Weight-streaming kernels (granule 16) with both epilogues."""
    w, _ = CASES["oai_bias"]
    _check(Layer(w, T))


@pytest.mark.parametrize("block_m", [0, 16, 32, 64, 128, 256])
def test_mlp_variant_split_entry_points(block_m):
    """align -> gate/up (bias, clamped SwiGLU) -> down (bias) -> combine at every granule (0:
    variable row blocks): each stage's rows against the oracle's expert MLP."""
    w, T = CASES["oai_bias"]
    assert w.hidden_size % 256 == 0 and w.intermediate_size % 128 == 0
    layer = Layer(w, T)
    p = params(w)
    d = layer.d
    dev = d["x"].device
    k, H, I = w.top_k, w.hidden_size, w.intermediate_size
    ids_h, tw_h, _ = layer.gpu_route()
    local = torch.from_numpy(layer.emap[ids_h].astype(np.int32)).to(dev)
    ws = torch.empty(moe.moe_workspace_size(p, T, block_m), dtype=torch.uint8, device=dev)
    cap = moe.moe_sorted_capacity(p, T, block_m)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p, T, block_m), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p, T, local, block_m, sp, be, pr, npad, ws)
    act = torch.empty(cap, I, dtype=d["x"].dtype, device=dev)
    y = torch.empty(cap, H, dtype=d["x"].dtype, device=dev)
    moe.moe_expert_gate_up(p, T, d["x"], d["w13"], sp, be, npad, block_m, act, b13=d["b13"])
    moe.moe_expert_down(p, T, act, d["w2"], be, npad, block_m, y, b2=d["b2"])
    y2 = torch.empty_like(y)
    moe.moe_grouped_mlp(p, T, d["x"], d["w13"], d["w2"], sp, be, npad, block_m, y2, ws,
                        b13=d["b13"], b2=d["b2"])
    out = torch.empty(T, H, dtype=d["x"].dtype, device=dev)
    tw_d = torch.from_numpy(tw_h).to(dev)
    moe.moe_combine(p, T, y, pr, tw_d, None, out)
    torch.cuda.synchronize()
    n = int(npad.item())
    real = sp[:n] >= 0  # padding rows of y hold unspecified values
    assert torch.equal(y[:n][real], y2[:n][real]), "grouped_mlp and the two stages disagree"
    a = oracle.align_permute(local.cpu().numpy(), w.num_local_experts, block_m)
    y_h = y.float().cpu().numpy()
    for r in [r for r in range(n) if a["sorted_pairs"][r] >= 0][:: max(1, n // 24)]:
        pid = a["sorted_pairs"][r]
        s = slot_of_row(a["block_expert"], r, block_m)
        want = oracle.gated_mlp(wl.to_f32(layer.x[pid // k])[None], wl.to_f32(layer.w13[s]),
                                wl.to_f32(layer.w2[s]), "swigluoai", layer.b13[s], layer.b2[s])[0]
        assert rel_err(y_h[r], want) <= 2 * OUT_TOL[w.dtype]
    want_out = layer.oracle_out(np.arange(T), ids_h, tw_h, with_shared=False)
    assert rel_err(out.float().cpu().numpy(), want_out) <= OUT_TOL[w.dtype]


@pytest.mark.parametrize("T", [32, 4096])
def test_gptoss_full_size(T):
    """The gpt-oss-shaped share: routing on every token, outputs on every token (T=32) or on
    >= 512 sampled rows that cover every local expert (T=4096)."""
    w = wl.WORKLOADS["gptoss"]
    layer = Layer(w, T)
    out, ids, tw = layer.forward()
    ref = layer.oracle_route()
    mism, near = layer.check_routing(ids, tw, ref)
    rows = np.arange(T) if T <= 256 else sample_rows(ids, layer.emap, T)
    ids_ref, w_ref = reference_routing(w, ids, ref, mism)
    want = layer.oracle_out(rows, ids_ref[rows], w_ref[rows])
    err = rel_err(out[rows], want)
    print(f"[gptoss T={T}] rel_err={err:.3e} near_ties={near} exempt={mism.size}", flush=True)
    assert err <= OUT_TOL[w.dtype], err
