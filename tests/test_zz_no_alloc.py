"""moe_forward_noalloc (the entry point that allocates nothing; its workspace is the library's
own device array) against moe_forward on the same inputs: two calls in a row, the second with
fewer tokens and another layer shape, each bit for bit equal to moe_forward and within the
oracle's tolerance; a call that needs more than the array holds is refused with MOE_ENOSPC."""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import workloads as wl
from moe_case import OUT_TOL, Layer, params, reference_routing, rel_err, torch_dtype

pytestmark = pytest.mark.gpu

W = wl.Workload
# grouped routing, routed scaling, a shared expert, a share of 8; then a plain share at fewer
# tokens
FIRST = (W("noalloc_a", 51, "no-alloc, grouped with shared", "bf16", (300,), 512, 64, 256, 6,
           False, use_grouped_topk=True, num_expert_group=8, topk_group=3,
           routed_scaling_factor=16.0, ep_size=8, ep_rank=0, shared_intermediate_size=512), 300)
SECOND = (W("noalloc_b", 52, "no-alloc, plain", "bf16", (37,), 256, 16, 384, 4, True,
            ep_size=2, ep_rank=1), 37)


def _noalloc(layer):
    w, T, d = layer.w, layer.T, layer.d
    dev = d["x"].device
    out = torch.full((T, w.hidden_size), 7.0, dtype=torch_dtype(w), device=dev)
    ids = torch.full((T, w.top_k), -7, dtype=torch.int32, device=dev)
    tw = torch.full((T, w.top_k), 7.0, dtype=torch.float32, device=dev)
    moe.moe_forward_noalloc(params(w), T, d["x"], d["gate"], d["bias"], d["emap"], d["w13"],
                            d["w2"], d["sw13"], d["sw2"], out, ids, tw, score_bias=d["sbias"],
                            b13=d["b13"], b2=d["b2"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ids.cpu().numpy(), tw.cpu().numpy()


def test_noalloc_matches_forward_twice():
    for w, T in (FIRST, SECOND):
        layer = Layer(w, T)
        p = params(w)
        assert moe.moe_workspace_size(p, T) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        got = _noalloc(layer)
        want = layer.forward()
        for g, r in zip(got, want):
            assert np.array_equal(g, r), w.key
        ref = layer.oracle_route()
        mism, _ = layer.check_routing(got[1], got[2], ref)
        ids_ref, w_ref = reference_routing(w, got[1], ref, mism)
        err = rel_err(got[0], layer.oracle_out(np.arange(T), ids_ref, w_ref))
        print(f"[{w.key} T={T}] no-alloc rel_err={err:.3e}", flush=True)
        assert err <= OUT_TOL[w.dtype], err


def test_noalloc_refuses_what_does_not_fit():
    w = wl.WORKLOADS["mixtral"]
    T = 4096
    p = params(w)
    assert moe.moe_workspace_size(p, T) > moe.MOE_NOALLOC_SCRATCH_BYTES
    F = 1 << 20  # never dereferenced: the size check comes first
    rc = moe.lib().moe_forward_noalloc(
        moe.ctypes.byref(p), T, F, F, None, None, F, F, F, None, None, None, None, F, None, None,
        None)
    assert rc == moe.MOE_ENOSPC
