"""Packed weight layout (MOE_WEIGHTS_PACKED) on the GPU.

moe_pack_weights is pure data movement: bit-exact against the layout's definition, written
here as a numpy reshape. The packed layout changes only where the kernels read each weight
chunk, not which chunk meets which MFMA, so every result of the layer (routing, rows, output)
must be bit-identical to the row-major run on the same inputs, which the other GPU tests
check against the oracle.
"""
import numpy as np
import pytest
import torch

import expert_moe_amd as moe
import workloads as wl
from moe_case import Layer, params
from test_gpu_parity import SMALL, VAR_SHARED

pytestmark = pytest.mark.gpu


def _packed_reference(a: np.ndarray) -> np.ndarray:
    """[n, rows, cols] -> blocks of 16 rows x 32 columns: panel-major, then column blocks,
    then the block's rows (the layout stated with moe_pack_weights)."""
    n, rows, cols = a.shape
    return (a.reshape(n, rows // 16, 16, cols // 32, 32).transpose(0, 1, 3, 2, 4)
            .reshape(n, rows, cols))


@pytest.mark.parametrize("shape", [(1, 16, 32), (3, 48, 96), (2, 128, 2880), (5, 2880, 64),
                                   (1, 7168 // 4, 2048)])
def test_pack_matches_layout_definition(shape):
    g = torch.Generator().manual_seed(sum(shape))
    bits = torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16)
    src = bits.view(torch.bfloat16).cuda()
    dst = torch.full_like(src, float("nan"))
    moe.moe_pack_weights(src, out=dst)
    torch.cuda.synchronize()
    want = _packed_reference(bits.numpy())
    assert np.array_equal(dst.cpu().view(torch.int16).numpy(), want)
    # the source is left as it was
    assert torch.equal(src.cpu().view(torch.int16), bits)


def _packed_tensors(d):
    return {k: (None if d[k] is None else moe.moe_pack_weights(d[k]))
            for k in ("w13", "w2", "sw13", "sw2")}


def _forward(p, layer, wts, T):
    w, d = layer.w, layer.d
    dev = d["x"].device
    out = torch.empty(T, w.hidden_size, dtype=d["x"].dtype, device=dev)
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, w.top_k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)
    moe.moe_forward(p, T, d["x"], d["gate"], d["bias"], d["emap"], wts["w13"], wts["w2"],
                    wts["sw13"], wts["sw2"], out, ids, tw, ws, score_bias=d["sbias"], b13=d["b13"],
                    b2=d["b2"])
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), ids.cpu().numpy(), tw.cpu().numpy()


BF16_CASES = [(k, SMALL[k]) for k in sorted(SMALL) if SMALL[k][0].dtype == "bf16"]
BF16_CASES += [("var_sh_1200", (VAR_SHARED, 1200)), ("var_sh_3000", (VAR_SHARED, 3000)),
               ("gptoss_T64", (wl.WORKLOADS["gptoss"], 64))]


@pytest.mark.parametrize("case", [c for c, _ in BF16_CASES])
def test_forward_packed_is_bit_identical(case):
    w, T = dict(BF16_CASES)[case]
    layer = Layer(w, T, host_weights=False)
    row = _forward(params(w), layer, layer.d, T)
    packed = _forward(params(w, weight_layout="packed"), layer, _packed_tensors(layer.d), T)
    assert np.array_equal(row[1], packed[1])
    assert np.array_equal(row[2], packed[2])
    assert np.array_equal(row[0], packed[0]), f"{case}: packed and row-major outputs differ"


@pytest.mark.parametrize("block_m", [16, 64, 256, 0])
@pytest.mark.parametrize("case", ["ep_s", "skew_s600", "mix_m"])
def test_grouped_mlp_packed_is_bit_identical(case, block_m):
    """The split entry points at every kernel granule (16: weight streaming, 64/256: LDS tiles,
    0: variable row blocks where the shapes allow them)."""
    w, T = SMALL[case]
    if block_m == 0 and not (w.hidden_size % 256 == 0 and w.intermediate_size % 128 == 0):
        pytest.skip("variable row blocks need H % 256 == 0 and 2I % 256 == 0")
    layer = Layer(w, T, host_weights=False)
    d, dev = layer.d, layer.d["x"].device
    k, H = w.top_k, w.hidden_size
    p_row, p_pk = params(w), params(w, weight_layout="packed")
    ws = torch.empty(moe.moe_workspace_size(p_row, T, block_m), dtype=torch.uint8, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    local = torch.empty(T, k, dtype=torch.int32, device=dev)
    moe.moe_route(p_row, T, d["x"], d["gate"], d["bias"], d["emap"], ids, tw, local, ws,
                  score_bias=d["sbias"])
    cap = moe.moe_sorted_capacity(p_row, T, block_m)
    sp = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(moe.block_expert_len(p_row, T, block_m), dtype=torch.int32, device=dev)
    pr = torch.empty(T * k, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_align_permute(p_row, T, local, block_m, sp, be, pr, npad, ws)
    pk = _packed_tensors(d)
    n = None
    outs = []
    for p, wts in ((p_row, d), (p_pk, pk)):
        y = torch.zeros(cap, H, dtype=d["x"].dtype, device=dev)
        moe.moe_grouped_mlp(p, T, d["x"], wts["w13"], wts["w2"], sp, be, npad, block_m, y, ws)
        torch.cuda.synchronize()
        n = int(npad.item())
        rows = sp[:n].cpu().numpy() >= 0
        outs.append(y[:n].view(torch.int16).cpu().numpy()[rows])
    assert np.array_equal(outs[0], outs[1]), f"{case} block_m={block_m}"


def test_noalloc_packed_is_bit_identical():
    w, T = SMALL["ds_s"]
    layer = Layer(w, T, host_weights=False)
    d, dev = layer.d, layer.d["x"].device
    row = _forward(params(w), layer, d, T)
    p = params(w, weight_layout="packed")
    pk = _packed_tensors(d)
    out = torch.empty(T, w.hidden_size, dtype=d["x"].dtype, device=dev)
    moe.moe_forward_noalloc(p, T, d["x"], d["gate"], d["bias"], d["emap"], pk["w13"], pk["w2"],
                            pk["sw13"], pk["sw2"], out, None, None, score_bias=d["sbias"])
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), row[0])
