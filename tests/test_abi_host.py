"""Host-side checks of the C-ABI library (CPU only: nothing here launches a kernel).

The library loads, exports every entry point include/moe.h declares, and its host logic
(parameter checks, shares, memory arithmetic, workspace sizing, argument errors) behaves
as the header states. Entry points are only called on paths that return before any HIP
call (T = 0, invalid arguments, too-small workspaces).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_moe_amd as moe
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-NULL device address that the host never dereferences


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(moe.LIB_PATH):
        from expert_moe_amd.build import build
        build(verbose=False)
    return moe.lib()


def _params(w: wl.Workload, **over):
    kw = dict(num_experts=w.num_experts, top_k=w.top_k, hidden_size=w.hidden_size,
              intermediate_size=w.intermediate_size, renormalize=w.renormalize,
              use_grouped_topk=w.use_grouped_topk, num_expert_group=w.num_expert_group,
              topk_group=w.topk_group, routed_scaling_factor=w.routed_scaling_factor,
              num_local_experts=w.num_local_experts,
              shared_intermediate_size=w.shared_intermediate_size, dtype=w.dtype)
    kw.update(over)
    return moe.make_params(**kw)


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\**\s+\**(moe_[a-z_]+)\(", text, re.M))
    assert declared == set(moe.EXPORTS)
    h = ctypes.CDLL(moe.LIB_PATH)
    for name in declared:
        assert hasattr(h, name), name


def test_strerror():
    assert moe.strerror(0) == "ok"
    for c in (-1, -2, -3, -4, 7):
        assert moe.strerror(c)


@pytest.mark.parametrize("key", sorted(wl.WORKLOADS))
def test_workload_params_valid(key):
    w = wl.WORKLOADS[key]
    p = _params(w)
    assert moe.moe_check_params(p) == moe.MOE_OK
    for T in w.tokens:
        bm = moe.moe_pick_block_m(p, T)
        assert bm in (0, 16, 32, 64, 128, 256)
        gran = bm if bm > 0 else 32
        assert moe.moe_sorted_capacity(p, T, bm) == T * w.top_k + w.num_local_experts * (gran - 1)
        if bm == 0:  # variable row blocks: bf16 with H and 2I multiples of 256
            assert w.dtype == "bf16" and w.hidden_size % 256 == 0 and w.intermediate_size % 128 == 0
        assert moe.moe_workspace_size(p, T) > 0


def test_param_errors():
    w = wl.WORKLOADS["dsv2"]
    E = moe.MOE_EINVAL
    cases = [
        (dict(top_k=0), E), (dict(top_k=161), E), (dict(hidden_size=100), E),
        (dict(intermediate_size=0), E), (dict(renormalize=True, num_local_experts=0), E),
        (dict(num_local_experts=257), moe.MOE_EUNSUPPORTED), (dict(num_expert_group=7), E),
        (dict(topk_group=9), E), (dict(topk_group=0), E), (dict(top_k=61, topk_group=3), E),
        (dict(shared_intermediate_size=100), E),
        (dict(routed_scaling_factor=float("inf")), E),
        (dict(num_experts=320, num_expert_group=8), moe.MOE_EUNSUPPORTED),
    ]
    for over, want in cases:
        p = _params(w, **over)
        assert moe.moe_check_params(p) == want, over
    p = _params(w)
    p.dtype = 7  # the library's own check (the binding refuses such a dtype before it)
    assert moe.moe_check_params(p) == moe.MOE_EUNSUPPORTED
    p = _params(w)
    p.scoring_func = 2  # neither softmax nor sigmoid
    assert moe.moe_check_params(p) == E
    assert moe.moe_check_params(_params(w, scoring_func="sigmoid")) == moe.MOE_OK
    with pytest.raises(ValueError):
        _params(w, scoring_func="tanh")


def test_expert_map_shares():
    for key, w in wl.WORKLOADS.items():
        got = moe.moe_make_expert_map(w.num_experts, w.ep_size, w.ep_rank)
        assert np.array_equal(got, wl.expert_map(w)), key
    # every global expert lands in exactly one share, with consecutive slots
    maps = [moe.moe_make_expert_map(64, 8, r) for r in range(8)]
    owned = np.stack([m >= 0 for m in maps])
    assert np.all(owned.sum(axis=0) == 1)
    for r, m in enumerate(maps):
        assert m[owned[r]].tolist() == list(range(8))
    for bad in [(8, 9, 0), (8, 3, 0), (8, 4, 4), (8, 4, -1), (0, 1, 0), (8, 0, 0)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_make_expert_map(*bad)
        assert ei.value.code == moe.MOE_EINVAL


def test_weight_bytes_matches_page_arithmetic():
    GiB = 2 ** 30
    assert moe.moe_weight_bytes(256, 2048, 256, 2, 30) == 22.5 * GiB
    assert moe.moe_weight_bytes(64, 2048, 512, 2, 30) == 11.25 * GiB
    assert moe.moe_weight_bytes(256, 2048, 512, 2, 30) == 45 * GiB
    assert moe.moe_weight_bytes(-1, 1, 1, 1, 1) == -1


def test_workspace_grows_with_tokens():
    p = _params(wl.WORKLOADS["skewed"])
    sizes = [moe.moe_workspace_size(p, T, 128) for T in (1, 256, 4096, 16384)]
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(p, 16, 48)
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(p, -1)


def test_host_tensor_arguments_are_refused():
    """A tensor in host memory never reaches a kernel as a device address: the binding raises
    before calling the library."""
    import torch
    p = _params(wl.WORKLOADS["mixtral"])
    x = torch.zeros(4, 4096, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        moe.moe_combine(p, 4, x, None, None, None, None, stream=0)
    with pytest.raises(ValueError, match="device memory"):
        moe.moe_forward(p, 4, x, None, None, None, None, None, None, None, None, None, None,
                        None, stream=0)


def test_entry_points_zero_tokens_are_noops():
    p = _params(wl.WORKLOADS["mixtral"])
    moe.moe_forward(p, 0, None, None, None, None, None, None, None, None, None, None, None,
                    None, stream=0)
    moe.moe_route(p, 0, None, None, None, None, None, None, None, None, stream=0)
    moe.moe_align_permute(p, 0, None, 16, None, None, None, None, None, stream=0)
    moe.moe_grouped_mlp(p, 0, None, None, None, None, None, None, 16, None, None, stream=0)
    moe.moe_combine(p, 0, None, None, None, None, None, stream=0)


def _forward_raw(pp, T, ws_bytes, **over):
    """moe_forward through the raw C symbol with every pointer a fake non-NULL address unless
    overridden (only for calls that must fail before launching anything)."""
    F = FAKE
    a = dict(x=F, w_gate=F, logit_bias=None, score_bias=None, expert_map=F, w13=F, w2=F, b13=None,
             b2=None, shared_w13=F, shared_w2=F, out=F, topk_ids=None, topk_w=None, ws=F)
    a.update(over)
    return moe.lib().moe_forward(pp, T, a["x"], a["w_gate"], a["logit_bias"], a["score_bias"],
                                 a["expert_map"], a["w13"], a["w2"], a["b13"], a["b2"],
                                 a["shared_w13"], a["shared_w2"], a["out"], a["topk_ids"],
                                 a["topk_w"], a["ws"], ws_bytes, None)


def test_entry_point_argument_errors():
    p = _params(wl.WORKLOADS["dsv2"])
    L = moe.lib()
    pp = ctypes.byref(p)
    T = 64
    # exactly what moe_forward needs (its own granule), so that one byte less is refused
    ws = moe.moe_workspace_size(p, T, moe.moe_pick_block_m(p, T))
    F = FAKE
    # missing required pointers
    assert _forward_raw(pp, T, ws, x=None) == -1
    assert _forward_raw(pp, T, ws, expert_map=None) == -1
    # only one of the two shared-expert pointers
    assert _forward_raw(pp, T, ws, shared_w2=None) == -1
    # workspace too small
    assert _forward_raw(pp, T, ws - 1) == -3
    # tensor pointers that are not 16-byte aligned
    assert _forward_raw(pp, T, ws, x=F + 2) == -1
    assert _forward_raw(pp, T, ws, out=F + 8) == -1
    assert _forward_raw(pp, T, ws, b13=F + 8) == -1
    assert _forward_raw(pp, T, ws, b2=F + 4) == -1
    assert L.moe_grouped_mlp(pp, T, F, F, F, None, None, F, F, F, 16, F + 4, F, ws, None) == -1
    assert L.moe_grouped_mlp(pp, T, F, F, F, F + 4, None, F, F, F, 16, F, F, ws, None) == -1
    assert L.moe_expert_gate_up(pp, T, F, F, F + 8, F, F, F, 16, F, None) == -1
    assert L.moe_expert_down(pp, T, F, F, F + 8, F, F, 16, F, None) == -1
    assert L.moe_combine(pp, T, F, F, F, F + 2, F, None) == -1
    # negative token count
    assert _forward_raw(pp, -1, ws) == -1
    # bad block_m for the split entry points
    assert L.moe_align_permute(pp, T, F, 48, F, F, F, F, F, ws, None) == -1
    assert L.moe_grouped_mlp(pp, T, F, F, F, None, None, F, F, F, 48, F, F, ws, None) == -1
    assert L.moe_align_permute(pp, T, F, 16, F, F, F, F, F, 8, None) == -3
    assert L.moe_route(pp, T, F, F, None, None, F, F, F, F, F, 8, None) == -3
    # shared MLP on a share without a shared expert
    p2 = _params(wl.WORKLOADS["ep_share"])
    assert L.moe_shared_mlp(ctypes.byref(p2), T, F, F, F, F, F, ws, None) == -1
    # shared expert pointers given but the params say there is none
    assert _forward_raw(ctypes.byref(p2), T, moe.moe_workspace_size(p2, T)) == -1


def test_ep_exchange_host_logic():
    p = _params(wl.WORKLOADS["dsv2"])  # E = 160, k = 6
    L = moe.lib()
    pp = ctypes.byref(p)
    F = FAKE
    # capacity: every token to min(k, ep_size) ranks
    assert moe.moe_ep_send_capacity(p, 100, 8) == 600
    assert moe.moe_ep_send_capacity(p, 100, 4) == 400
    assert moe.moe_ep_send_capacity(p, 100, 160) == 600
    assert moe.moe_ep_send_capacity(p, 0, 1) == 0
    for bad in (0, 3, 320, 257, -1):  # not a divisor of E, or out of range
        assert L.moe_ep_send_capacity(pp, 100, bad) == -1
        with pytest.raises(moe.MoeError):
            moe.moe_ep_workspace_size(p, 100, bad)
    assert L.moe_ep_send_capacity(pp, -1, 8) == -1
    sizes = [moe.moe_ep_workspace_size(p, T, 8) for T in (1, 256, 4096, 16384)]
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]
    T = 64
    ws = moe.moe_ep_workspace_size(p, T, 8)
    # T = 0 returns before any launch
    moe.moe_ep_dispatch(p, 0, 8, None, None, None, None, None, None, None, None, None, None,
                        stream=0)
    moe.moe_ep_combine(p, 0, None, None, None, stream=0)
    ok = [F] * 9
    for i in range(9):  # each required pointer missing
        args = list(ok)
        args[i] = None
        assert L.moe_ep_dispatch(pp, T, 8, *args, F, ws, None) == -1, i
    args = list(ok)
    args[2] = F + 2  # x not 16-byte aligned
    assert L.moe_ep_dispatch(pp, T, 8, *args, F, ws, None) == -1
    args = list(ok)
    args[6] = F + 8  # send_x not 16-byte aligned
    assert L.moe_ep_dispatch(pp, T, 8, *args, F, ws, None) == -1
    assert L.moe_ep_dispatch(pp, T, 8, *ok, F, ws - 1, None) == -3
    assert L.moe_ep_dispatch(pp, T, 7, *ok, F, ws, None) == -1
    assert L.moe_ep_dispatch(pp, -1, 8, *ok, F, ws, None) == -1
    assert L.moe_ep_combine(pp, T, None, F, F, None) == -1
    assert L.moe_ep_combine(pp, T, F, F + 2, F, None) == -1
    assert L.moe_ep_combine(pp, T, F, F, F + 4, None) == -1


def test_eplb_tables_and_argument_errors():
    import oracle
    # tables: the host helper agrees with the oracle on a shuffled placement
    rng = np.random.default_rng(3)
    p2l = np.concatenate([np.arange(16), [0, 0, 5, 9, 9, 9]]).astype(np.int32)
    p2l = p2l[rng.permutation(p2l.size)]
    l2p, cnt = moe.moe_eplb_tables(16, p2l)
    w_l2p, w_cnt = oracle.eplb_tables(p2l, 16)
    assert np.array_equal(cnt, w_cnt) and np.array_equal(l2p, w_l2p)
    for bad_p2l, E in [([0, 1, 1], 3), ([0, 1, 3], 3), ([0, -1, 1], 3), ([0, 1], 3)]:
        with pytest.raises(moe.MoeError):
            moe.moe_eplb_tables(E, bad_p2l)
    with pytest.raises(moe.MoeError):  # logical 0 has 3 replicas, max_replicas 2
        moe.moe_eplb_tables(2, [0, 0, 0, 1], max_replicas=2)
    # entry points: invalid placements are rejected on the host, T = 0 is a no-op
    w = wl.WORKLOADS["ep_share"]  # E = 256
    p = _params(w)
    L = moe.lib()
    F = FAKE
    T = 32
    ws = moe.moe_workspace_size(p, T, moe.moe_pick_block_m(p, T))  # moe_forward's exact need
    good = moe.moe_eplb(264, 2, F, F)
    for e in [moe.moe_eplb(255, 2, F, F), moe.moe_eplb(4097, 2, F, F), moe.moe_eplb(264, 0, F, F),
              moe.moe_eplb(264, 265, F, F), moe.moe_eplb(264, 2, None, F),
              moe.moe_eplb(264, 2, F, None)]:
        assert L.moe_route_eplb(ctypes.byref(p), ctypes.byref(e), T, F, F, None, None, F, F, F, F, F,
                                ws, None) == -1
        assert L.moe_forward_eplb(ctypes.byref(p), ctypes.byref(e), T, F, F, None, None, F, F, F,
                                  None, None, None, None, F, None, None, F, ws, None) == -1
    assert L.moe_route_eplb(ctypes.byref(p), None, T, F, F, None, None, F, F, F, F, F, ws, None) == -1
    assert L.moe_forward_eplb(ctypes.byref(p), ctypes.byref(good), T, F, F, None, None, F, F, F,
                              None, None, None,
                              None, F, None, None, F, ws - 1, None) == -3
    moe.moe_route_eplb(p, good, 0, None, None, None, None, None, None, None, None, stream=0)
    moe.moe_forward_eplb(p, good, 0, None, None, None, None, None, None, None, None, None, None,
                         None, None, stream=0)
    # a share of a replicated placement may hold more slots than there are logical experts
    p2 = _params(wl.WORKLOADS["tiny"], num_local_experts=12)
    assert moe.moe_check_params(p2) == moe.MOE_OK
    assert moe.moe_workspace_size(p2, 64) > 0


def test_make_params_dtype_names():
    import torch
    for d in ("bf16", "bfloat16", torch.bfloat16, moe.MOE_BF16):
        assert moe.make_params(8, 2, 128, 256, dtype=d).dtype == moe.MOE_BF16
    for d in ("f32", "fp32", "float32", torch.float32, moe.MOE_F32):
        assert moe.make_params(8, 2, 128, 256, dtype=d).dtype == moe.MOE_F32
    for d in ("fp16", torch.float16, 2, None):
        with pytest.raises(ValueError, match="dtype"):
            moe.make_params(8, 2, 128, 256, dtype=d)


def test_binding_checks_tensor_dtypes_and_sizes():
    """The binding refuses a tensor of the wrong dtype or with fewer elements than the header's
    shape for the call, before anything reaches the library (host tensors suffice: the checks
    come first)."""
    import torch
    p = _params(wl.WORKLOADS["tiny"])  # fp32, H 128, E 8, I 256, k 2
    T, H = 4, 128
    x32 = torch.zeros(T, H)
    with pytest.raises(ValueError, match="x: dtype"):
        moe.moe_forward(p, T, x32.bfloat16(), None, None, None, None, None, None, None, None,
                        None, None, None, stream=0)
    with pytest.raises(ValueError, match="x: .* elements"):
        moe.moe_forward(p, T, x32[:2], None, None, None, None, None, None, None, None, None, None,
                        None, stream=0)
    with pytest.raises(ValueError, match="expert_map: dtype"):
        moe.moe_route(p, T, x32, None, None, torch.zeros(8, dtype=torch.int64), None, None, None,
                      None, stream=0)
    with pytest.raises(ValueError, match="w13: .* elements"):
        moe.moe_grouped_mlp(p, T, x32, torch.zeros(8, 2 * 256, H - 1), None, None, None, None, 16,
                            None, None, stream=0)
    with pytest.raises(ValueError, match="topk_w: dtype"):
        moe.moe_combine(p, T, x32, None, torch.zeros(T, 2, dtype=torch.float64), None, None,
                        stream=0)
    with pytest.raises(ValueError, match="out: .* elements"):
        moe.moe_combine(p, T, x32, None, None, None, torch.zeros(T, H - 1), stream=0)


def test_forward_overlap_argument_errors():
    """The side stream's events are required, and the side stream must differ from the call's
    stream; those are refused before anything is enqueued (also at T = 0). Without a side
    stream the call is moe_forward (T = 0: a no-op)."""
    p = _params(wl.WORKLOADS["dsv2"])
    L = moe.lib()
    pp = ctypes.byref(p)
    F = FAKE

    def call(side, T=0, stream=None):
        return L.moe_forward_overlap(pp, None, side, T, F, F, None, None, F, F, F, None, None, F, F,
                                     F, None, None, F, 1 << 30, stream)

    assert call(None) == 0
    assert call(ctypes.byref(moe.moe_side_stream(F, None, F))) == -1
    assert call(ctypes.byref(moe.moe_side_stream(F, F, None))) == -1
    assert call(ctypes.byref(moe.moe_side_stream(F, F, F)), stream=F) == -1
    assert call(ctypes.byref(moe.moe_side_stream(F, F, F)), stream=None) == 0


def test_variable_blocks_granule_rules():
    """Granule 0 (variable row blocks) is valid only for bf16 layers with H and 2I multiples of
    256; the workspace of granule 0 covers both moe_forward and the variable split path."""
    ok = _params(wl.WORKLOADS["mixtral"])
    assert moe.moe_sorted_capacity(ok, 100, 0) == 100 * 2 + 8 * 31
    assert moe.block_expert_len(ok, 100, 0) == 2 * ((200 + 248) // 256 + 1 + 8) + 4
    assert moe.moe_workspace_size(ok, 100, 0) >= moe.moe_workspace_size(ok, 100, 16)
    for key in ("tiny", "gptoss"):  # fp32; H = 2880
        p = _params(wl.WORKLOADS[key])
        with pytest.raises(moe.MoeError):
            moe.moe_sorted_capacity(p, 100, 0)
        assert moe.moe_pick_block_m(p, 4096) != 0
        F = FAKE
        assert moe.lib().moe_align_permute(ctypes.byref(p), 100, F, 0, F, F, F, F, F, 1 << 20,
                                           None) == moe.MOE_EINVAL


def test_weight_layout_rules():
    """Packed weights are a bf16 layout (fp32 layers: MOE_EUNSUPPORTED); other values are
    invalid; a zeroed field is the row-major layout."""
    assert moe.make_params(8, 2, 128, 256).weight_layout == moe.MOE_WEIGHTS_ROW_MAJOR
    assert moe.moe_check_params(moe.make_params(8, 2, 128, 256, weight_layout="packed")) == moe.MOE_OK
    p = moe.make_params(8, 2, 128, 256, dtype="f32", weight_layout="packed")
    assert moe.moe_check_params(p) == moe.MOE_EUNSUPPORTED
    p = moe.make_params(8, 2, 128, 256)
    p.weight_layout = 2
    assert moe.moe_check_params(p) == moe.MOE_EINVAL
    with pytest.raises(ValueError, match="weight_layout"):
        moe.make_params(8, 2, 128, 256, weight_layout="tiled")


def test_pack_weights_argument_errors():
    """moe_pack_weights refuses shapes off its 16 x 32 blocks, NULL, misaligned or overlapping
    buffers before it launches anything (fake device addresses are never dereferenced)."""
    lib = moe.lib()
    a, b = 1 << 32, 1 << 33
    assert lib.moe_pack_weights(0, 16, 32, None, None, None) == moe.MOE_OK
    assert lib.moe_pack_weights(-1, 16, 32, a, b, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(1, 8, 32, a, b, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(1, 24, 32, a, b, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(1, 16, 48, a, b, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(1, 16, 32, None, b, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(1, 16, 32, a + 8, b, None) == moe.MOE_EINVAL
    # 1 KiB matrices: dst inside src's range, and src inside dst's
    assert lib.moe_pack_weights(2, 16, 32, a, a + 1024, None) == moe.MOE_EINVAL
    assert lib.moe_pack_weights(2, 16, 32, a + 1024, a, None) == moe.MOE_EINVAL
    # 2^31 chunks of 16 bytes or more
    assert lib.moe_pack_weights(1 << 20, 1024, 1024 * 2, a, b, None) == moe.MOE_EINVAL
    with pytest.raises(ValueError):
        import torch
        moe.moe_pack_weights(torch.zeros(16, 32, dtype=torch.float32))
