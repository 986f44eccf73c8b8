"""Python binding of the gfx950 fused MoE library (``libexpert_moe.so``).

Argument marshalling only: every function here has the name of the C entry point it
calls (declared in ``include/moe.h``), turns tensors into device pointers and the
current torch stream into a ``hipStream_t``, and raises :class:`MoeError` on a negative
return code. All computation happens in the HIP kernels; there is no fallback path, and
importing a function fails loudly when the library has not been built.

Tensor arguments are ``torch`` tensors already on the GPU (bf16 data is passed as
``torch.bfloat16``; fp32 as ``torch.float32``; ids as ``torch.int32``); ``None`` passes
NULL. Before the library is called, each tensor's dtype and element count are checked against
the shapes ``include/moe.h`` states for the call (a raw integer address is passed unchecked).
PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexpert_moe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOSPC, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_ACT_SILU, MOE_ACT_SWIGLUOAI = 0, 1
MOE_WEIGHTS_ROW_MAJOR, MOE_WEIGHTS_PACKED = 0, 1

# every symbol include/moe.h declares
EXPORTS = (
    "moe_strerror", "moe_check_params", "moe_pick_block_m", "moe_sorted_capacity",
    "moe_workspace_size", "moe_make_expert_map", "moe_weight_bytes", "moe_route",
    "moe_align_permute", "moe_grouped_mlp", "moe_expert_gate_up", "moe_expert_down",
    "moe_shared_mlp", "moe_combine", "moe_forward",
    "moe_ep_send_capacity", "moe_ep_workspace_size", "moe_ep_dispatch", "moe_ep_combine",
    "moe_eplb_tables", "moe_route_eplb", "moe_forward_eplb", "moe_forward_overlap",
    "moe_forward_noalloc", "moe_pack_weights",
)

# bytes of the library's own workspace array behind moe_forward_noalloc
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


class moe_params(ctypes.Structure):
    """Mirror of ``struct moe_params`` in include/moe.h."""
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hidden_size", ctypes.c_int32),
        ("intermediate_size", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("use_grouped_topk", ctypes.c_int32),
        ("num_expert_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("num_local_experts", ctypes.c_int32),
        ("shared_intermediate_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scoring_func", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
    ]


class moe_eplb(ctypes.Structure):
    """Mirror of ``struct moe_eplb`` in include/moe.h (device table pointers as integers)."""
    _fields_ = [
        ("num_physical_experts", ctypes.c_int32),
        ("max_replicas", ctypes.c_int32),
        ("logical_to_physical", ctypes.c_void_p),
        ("replica_count", ctypes.c_void_p),
    ]


class moe_side_stream(ctypes.Structure):
    """Mirror of ``struct moe_side_stream`` in include/moe.h (stream and event handles)."""
    _fields_ = [
        ("stream", ctypes.c_void_p),
        ("fork_event", ctypes.c_void_p),
        ("join_event", ctypes.c_void_p),
    ]


def _event(e):
    if e is None or isinstance(e, int):
        return e
    h = e.cuda_event
    if not h:
        raise ValueError("the event has no handle yet (torch creates it on its first record); "
                         "record it once before passing it")
    return h


def make_side_stream(stream, fork_event, join_event) -> moe_side_stream:
    """A ``moe_side_stream`` from a torch stream (or raw handle) and two torch events (or raw
    handles). The struct holds references to its arguments, so they live as long as it does."""
    s = moe_side_stream(_stream(stream), _event(fork_event), _event(join_event))
    s._keep = (stream, fork_event, join_event)
    return s


def make_eplb(num_physical_experts, max_replicas, logical_to_physical, replica_count):
    """A ``moe_eplb`` over device tables (tensors or raw addresses). The returned struct holds
    references to tensor arguments, so they live as long as it does."""
    e = moe_eplb(num_physical_experts, max_replicas, _ptr(logical_to_physical),
                 _ptr(replica_count))
    e._tables = (logical_to_physical, replica_count)
    return e


def make_params(num_experts, top_k, hidden_size, intermediate_size, renormalize=True,
                use_grouped_topk=False, num_expert_group=1, topk_group=1,
                routed_scaling_factor=1.0, num_local_experts=None, shared_intermediate_size=0,
                dtype="bf16", scoring_func="softmax", activation="silu",
                weight_layout="row_major") -> moe_params:
    if scoring_func in ("softmax", MOE_SCORE_SOFTMAX):
        sf = MOE_SCORE_SOFTMAX
    elif scoring_func in ("sigmoid", MOE_SCORE_SIGMOID):
        sf = MOE_SCORE_SIGMOID
    else:
        raise ValueError(f"scoring_func {scoring_func!r}")
    if activation in ("silu", MOE_ACT_SILU):
        act = MOE_ACT_SILU
    elif activation in ("swigluoai", MOE_ACT_SWIGLUOAI):
        act = MOE_ACT_SWIGLUOAI
    else:
        raise ValueError(f"activation {activation!r}")
    if weight_layout in ("row_major", MOE_WEIGHTS_ROW_MAJOR):
        wlay = MOE_WEIGHTS_ROW_MAJOR
    elif weight_layout in ("packed", MOE_WEIGHTS_PACKED):
        wlay = MOE_WEIGHTS_PACKED
    else:
        raise ValueError(f"weight_layout {weight_layout!r}")
    return moe_params(
        int(num_experts), int(top_k), int(hidden_size), int(intermediate_size),
        int(bool(renormalize)), int(bool(use_grouped_topk)), int(num_expert_group),
        int(topk_group), float(routed_scaling_factor),
        int(num_experts if num_local_experts is None else num_local_experts),
        int(shared_intermediate_size), _dtype_code(dtype), sf, act, wlay)


def _dtype_code(dtype) -> int:
    """MOE_BF16 or MOE_F32 from a name, a code or a torch dtype; ValueError otherwise."""
    if isinstance(dtype, str):
        names = {"bf16": MOE_BF16, "bfloat16": MOE_BF16, "f32": MOE_F32, "fp32": MOE_F32,
                 "float32": MOE_F32}
        if dtype in names:
            return names[dtype]
    elif isinstance(dtype, int) and not isinstance(dtype, bool):
        if dtype in (MOE_BF16, MOE_F32):
            return dtype
    else:
        import torch
        if dtype == torch.bfloat16:
            return MOE_BF16
        if dtype == torch.float32:
            return MOE_F32
    raise ValueError(f"dtype {dtype!r}: expected bf16 or f32 (a name, MOE_BF16 / MOE_F32 or a "
                     "torch dtype)")


_lib = None
_P = ctypes.POINTER(moe_params)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_SIGS = {
    "moe_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "moe_check_params": ([_P], ctypes.c_int),
    "moe_pack_weights": ([_i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "moe_pick_block_m": ([_P, _i64, ctypes.POINTER(_i32)], ctypes.c_int),
    "moe_sorted_capacity": ([_P, _i64, _i32], _i64),
    "moe_workspace_size": ([_P, _i64, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "moe_make_expert_map": ([_i32, _i32, _i32, _vp], ctypes.c_int),
    "moe_weight_bytes": ([_i64, _i64, _i64, _i32, _i64], _i64),
    "moe_route": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_align_permute": ([_P, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_grouped_mlp": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz,
                         _vp], ctypes.c_int),
    "moe_expert_gate_up": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp], ctypes.c_int),
    "moe_expert_down": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp], ctypes.c_int),
    "moe_shared_mlp": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_combine": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_forward": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                     _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_ep_send_capacity": ([_P, _i64, _i32], _i64),
    "moe_ep_workspace_size": ([_P, _i64, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "moe_ep_dispatch": ([_P, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                        ctypes.c_int),
    "moe_ep_combine": ([_P, _i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_eplb_tables": ([_i32, _i32, _vp, _i32, _vp, _vp], ctypes.c_int),
    "moe_route_eplb": ([_P, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                       ctypes.c_int),
    "moe_forward_eplb": ([_P, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_forward_noalloc": ([_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp], ctypes.c_int),
    "moe_forward_overlap": ([_P, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
}


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m expert_moe_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def _ptr(t):
    """Device address of a buffer argument: None, an int (taken as a device address as is), or
    a contiguous tensor in device memory. A host tensor is refused here: the kernels would read
    its address as device memory."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must be in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _check_tensors(p, checks):
    """Host-side argument checks before a call: each (name, tensor, kind, min_elements) with
    kind "data" (p's dtype), "f32" or "i32"; None and raw addresses pass. Raises ValueError."""
    import torch
    data = torch.bfloat16 if p.dtype == MOE_BF16 else torch.float32
    want = {"data": data, "f32": torch.float32, "i32": torch.int32}
    for name, t, kind, n in checks:
        if t is None or isinstance(t, int):
            continue
        if t.dtype != want[kind]:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {want[kind]}")
        if t.numel() < n:
            raise ValueError(f"{name}: {t.numel()} elements, at least {n} expected")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def _check(rc, where):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def strerror(code: int) -> str:
    return lib().moe_strerror(int(code)).decode()


def moe_check_params(p: moe_params) -> int:
    return lib().moe_check_params(ctypes.byref(p))


def moe_pack_weights(w, out=None, stream=None):
    """The packed weight layout (MOE_WEIGHTS_PACKED) of a bf16 weight tensor [..., rows, cols]
    (w13 [E_l, 2I, H], w2 [E_l, H, I], shared_w13 [2 I_s, H], shared_w2 [H, I_s]): a new tensor
    of the same shape and dtype (or `out`) holding the rearranged elements."""
    import torch
    if w.dtype != torch.bfloat16 or w.dim() < 2:
        raise ValueError("moe_pack_weights: a bf16 tensor [..., rows, cols] is expected")
    rows, cols = w.shape[-2], w.shape[-1]
    n = w.numel() // (rows * cols) if rows * cols else 0
    if out is None:
        out = torch.empty_like(w)
    elif out.dtype != torch.bfloat16 or out.numel() != w.numel():
        raise ValueError("moe_pack_weights: out must be a bf16 tensor of the same size")
    _check(lib().moe_pack_weights(n, rows, cols, _ptr(w), _ptr(out), _stream(stream)), "moe_pack_weights")
    return out


def moe_pick_block_m(p: moe_params, num_tokens: int) -> int:
    bm = _i32()
    _check(lib().moe_pick_block_m(ctypes.byref(p), num_tokens, ctypes.byref(bm)), "moe_pick_block_m")
    return bm.value


def moe_sorted_capacity(p: moe_params, num_tokens: int, block_m: int) -> int:
    v = lib().moe_sorted_capacity(ctypes.byref(p), num_tokens, block_m)
    if v < 0:
        raise MoeError(MOE_EINVAL, "moe_sorted_capacity")
    return v


def moe_workspace_size(p: moe_params, num_tokens: int, block_m: int = 0) -> int:
    n = _sz()
    _check(lib().moe_workspace_size(ctypes.byref(p), num_tokens, block_m, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def moe_make_expert_map(num_experts: int, ep_size: int, ep_rank: int):
    """Host helper: returns a numpy int32 [E] map (raises on invalid shares)."""
    import numpy as np
    m = np.empty(num_experts if num_experts > 0 else 1, np.int32)
    _check(lib().moe_make_expert_map(num_experts, ep_size, ep_rank, m.ctypes.data),
           "moe_make_expert_map")
    return m


def moe_weight_bytes(n_experts: int, hidden: int, inter: int, dtype_bytes: int, layers: int = 1) -> int:
    return lib().moe_weight_bytes(n_experts, hidden, inter, dtype_bytes, layers)


def _route_checks(p, T, x, w_gate, logit_bias, score_bias, expert_map, n_map):
    E, H = p.num_experts, p.hidden_size
    return [("x", x, "data", T * H), ("w_gate", w_gate, "data", E * H),
            ("logit_bias", logit_bias, "f32", E), ("score_bias", score_bias, "f32", E),
            ("expert_map", expert_map, "i32", n_map)]


def _expert_checks(p, w13, w2, b13, b2):
    El, H, I = p.num_local_experts, p.hidden_size, p.intermediate_size
    return [("w13", w13, "data", El * 2 * I * H), ("w2", w2, "data", El * H * I),
            ("b13", b13, "f32", El * 2 * I), ("b2", b2, "f32", El * H)]


def moe_route(p, num_tokens, x, w_gate, logit_bias, expert_map, topk_ids, topk_w, topk_local,
              ws, stream=None, score_bias=None):
    Tk = num_tokens * p.top_k
    _check_tensors(p, _route_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                    p.num_experts)
                   + [("topk_ids", topk_ids, "i32", Tk), ("topk_w", topk_w, "f32", Tk),
                      ("topk_local", topk_local, "i32", Tk)])
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w_gate), _ptr(logit_bias),
                           _ptr(score_bias), _ptr(expert_map), _ptr(topk_ids), _ptr(topk_w), _ptr(topk_local),
                           wp, wn, _stream(stream)), "moe_route")


def block_expert_len(p, num_tokens: int, block_m: int) -> int:
    """int32 entries that block_expert needs (include/moe.h): one per block_m rows of the
    sorted capacity, or for variable row blocks (block_m = 0) the block table."""
    cap = moe_sorted_capacity(p, num_tokens, block_m)
    if block_m > 0:
        return cap // block_m + 1
    return 2 * (cap // 256 + 1 + p.num_local_experts) + 4


def _be_len(p, num_tokens, block_m):
    try:
        return block_expert_len(p, num_tokens, block_m) - 1
    except MoeError:
        return 0  # the library reports the invalid argument itself


def _sorted_rows(p, num_tokens, block_m):
    try:
        return moe_sorted_capacity(p, num_tokens, block_m)
    except MoeError:
        return 0  # the library reports the invalid argument itself


def moe_align_permute(p, num_tokens, topk_local, block_m, sorted_pairs, block_expert, pair_row,
                      num_padded, ws, stream=None):
    cap = _sorted_rows(p, num_tokens, block_m)
    Tk = num_tokens * p.top_k
    _check_tensors(p, [("topk_local", topk_local, "i32", Tk), ("sorted_pairs", sorted_pairs, "i32", cap),
                       ("block_expert", block_expert, "i32", _be_len(p, num_tokens, block_m)),
                       ("pair_row", pair_row, "i32", Tk), ("num_padded", num_padded, "i32", 1)])
    wp, wn = _ws(ws)
    _check(lib().moe_align_permute(ctypes.byref(p), num_tokens, _ptr(topk_local), block_m,
                                   _ptr(sorted_pairs), _ptr(block_expert), _ptr(pair_row),
                                   _ptr(num_padded), wp, wn, _stream(stream)), "moe_align_permute")


def moe_grouped_mlp(p, num_tokens, x, w13, w2, sorted_pairs, block_expert, num_padded, block_m,
                    y, ws, stream=None, b13=None, b2=None):
    cap = _sorted_rows(p, num_tokens, block_m)
    _check_tensors(p, [("x", x, "data", num_tokens * p.hidden_size)] + _expert_checks(p, w13, w2, b13, b2)
                   + [("sorted_pairs", sorted_pairs, "i32", cap),
                      ("block_expert", block_expert, "i32", _be_len(p, num_tokens, block_m)),
                      ("num_padded", num_padded, "i32", 1), ("y", y, "data", cap * p.hidden_size)])
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_mlp(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w13), _ptr(w2),
                                 _ptr(b13), _ptr(b2), _ptr(sorted_pairs), _ptr(block_expert), _ptr(num_padded),
                                 block_m, _ptr(y), wp, wn, _stream(stream)), "moe_grouped_mlp")


def moe_expert_gate_up(p, num_tokens, x, w13, sorted_pairs, block_expert, num_padded, block_m,
                       act, stream=None, b13=None):
    cap = _sorted_rows(p, num_tokens, block_m)
    _check_tensors(p, [("x", x, "data", num_tokens * p.hidden_size)]
                   + _expert_checks(p, w13, None, b13, None)
                   + [("sorted_pairs", sorted_pairs, "i32", cap),
                      ("block_expert", block_expert, "i32", _be_len(p, num_tokens, block_m)),
                      ("num_padded", num_padded, "i32", 1),
                      ("act", act, "data", cap * p.intermediate_size)])
    _check(lib().moe_expert_gate_up(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w13), _ptr(b13),
                                    _ptr(sorted_pairs), _ptr(block_expert), _ptr(num_padded),
                                    block_m, _ptr(act), _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(p, num_tokens, act, w2, block_expert, num_padded, block_m, y, stream=None,
                    b2=None):
    cap = _sorted_rows(p, num_tokens, block_m)
    _check_tensors(p, [("act", act, "data", cap * p.intermediate_size)]
                   + _expert_checks(p, None, w2, None, b2)
                   + [("block_expert", block_expert, "i32", _be_len(p, num_tokens, block_m)),
                      ("num_padded", num_padded, "i32", 1), ("y", y, "data", cap * p.hidden_size)])
    _check(lib().moe_expert_down(ctypes.byref(p), num_tokens, _ptr(act), _ptr(w2), _ptr(b2),
                                 _ptr(block_expert), _ptr(num_padded), block_m, _ptr(y),
                                 _stream(stream)), "moe_expert_down")


def moe_shared_mlp(p, num_tokens, x, shared_w13, shared_w2, shared_y, ws, stream=None):
    H, Is = p.hidden_size, p.shared_intermediate_size
    _check_tensors(p, [("x", x, "data", num_tokens * H), ("shared_w13", shared_w13, "data", 2 * Is * H),
                       ("shared_w2", shared_w2, "data", H * Is),
                       ("shared_y", shared_y, "data", num_tokens * H)])
    wp, wn = _ws(ws)
    _check(lib().moe_shared_mlp(ctypes.byref(p), num_tokens, _ptr(x), _ptr(shared_w13),
                                _ptr(shared_w2), _ptr(shared_y), wp, wn, _stream(stream)),
           "moe_shared_mlp")


def moe_combine(p, num_tokens, y, pair_row, topk_w, shared_y, out, stream=None):
    Tk, TH = num_tokens * p.top_k, num_tokens * p.hidden_size
    _check_tensors(p, [("y", y, "data", 0), ("pair_row", pair_row, "i32", Tk),
                       ("topk_w", topk_w, "f32", Tk), ("shared_y", shared_y, "data", TH),
                       ("out", out, "data", TH)])
    _check(lib().moe_combine(ctypes.byref(p), num_tokens, _ptr(y), _ptr(pair_row), _ptr(topk_w),
                             _ptr(shared_y), _ptr(out), _stream(stream)), "moe_combine")


def _forward_checks(p, T, x, w_gate, logit_bias, score_bias, expert_map, n_map, w13, w2, b13, b2,
                    shared_w13, shared_w2, out, topk_ids_out, topk_w_out):
    H, Is, Tk = p.hidden_size, p.shared_intermediate_size, T * p.top_k
    return (_route_checks(p, T, x, w_gate, logit_bias, score_bias, expert_map, n_map)
            + _expert_checks(p, w13, w2, b13, b2)
            + [("shared_w13", shared_w13, "data", 2 * Is * H), ("shared_w2", shared_w2, "data", H * Is),
               ("out", out, "data", T * H), ("topk_ids_out", topk_ids_out, "i32", Tk),
               ("topk_w_out", topk_w_out, "f32", Tk)])


def moe_forward(p, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2, shared_w13,
                shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None, score_bias=None,
                b13=None, b2=None):
    _check_tensors(p, _forward_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                      p.num_experts, w13, w2, b13, b2, shared_w13, shared_w2, out,
                                      topk_ids_out, topk_w_out))
    wp, wn = _ws(ws)
    _check(lib().moe_forward(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w_gate), _ptr(logit_bias),
                             _ptr(score_bias), _ptr(expert_map), _ptr(w13), _ptr(w2), _ptr(b13),
                             _ptr(b2), _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                             _ptr(topk_ids_out), _ptr(topk_w_out), wp, wn, _stream(stream)),
           "moe_forward")


def moe_ep_send_capacity(p, num_tokens: int, ep_size: int) -> int:
    n = lib().moe_ep_send_capacity(ctypes.byref(p), num_tokens, ep_size)
    if n < 0:
        raise MoeError(MOE_EINVAL, "moe_ep_send_capacity")
    return n


def moe_ep_workspace_size(p, num_tokens: int, ep_size: int) -> int:
    n = _sz()
    _check(lib().moe_ep_workspace_size(ctypes.byref(p), num_tokens, ep_size, ctypes.byref(n)),
           "moe_ep_workspace_size")
    return n.value


def moe_ep_dispatch(p, num_tokens, ep_size, topk_ids, topk_w, x, send_pos, rank_meta, send_token,
                    send_x, send_local, send_w, ws, stream=None):
    try:
        R = moe_ep_send_capacity(p, num_tokens, ep_size)
    except MoeError:
        R = 0  # the library reports the invalid argument itself
    Tk, k, H = num_tokens * p.top_k, p.top_k, p.hidden_size
    _check_tensors(p, [("topk_ids", topk_ids, "i32", Tk), ("topk_w", topk_w, "f32", Tk),
                       ("x", x, "data", num_tokens * H), ("send_pos", send_pos, "i32", Tk),
                       ("rank_meta", rank_meta, "i32", 2 * ep_size + 2),
                       ("send_token", send_token, "i32", R), ("send_x", send_x, "data", R * H),
                       ("send_local", send_local, "i32", R * k), ("send_w", send_w, "f32", R * k)])
    wp, wn = _ws(ws)
    _check(lib().moe_ep_dispatch(ctypes.byref(p), num_tokens, ep_size, _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(x), _ptr(send_pos), _ptr(rank_meta), _ptr(send_token),
                                 _ptr(send_x), _ptr(send_local), _ptr(send_w), wp, wn,
                                 _stream(stream)), "moe_ep_dispatch")


def moe_ep_combine(p, num_tokens, send_pos, recv_y, out, stream=None):
    _check_tensors(p, [("send_pos", send_pos, "i32", num_tokens * p.top_k),
                       ("recv_y", recv_y, "data", 0),
                       ("out", out, "data", num_tokens * p.hidden_size)])
    _check(lib().moe_ep_combine(ctypes.byref(p), num_tokens, _ptr(send_pos), _ptr(recv_y), _ptr(out),
                                _stream(stream)), "moe_ep_combine")


def moe_eplb_tables(num_logical: int, physical_to_logical, max_replicas: int | None = None):
    """Host helper: (logical_to_physical [E, max_replicas], replica_count [E]) as numpy int32."""
    import numpy as np
    p2l = np.ascontiguousarray(np.asarray(physical_to_logical, np.int32))
    if max_replicas is None:
        max_replicas = int(np.bincount(p2l[p2l >= 0], minlength=1).max()) if p2l.size else 1
    l2p = np.empty((max(num_logical, 1), max(max_replicas, 1)), np.int32)
    cnt = np.empty(max(num_logical, 1), np.int32)
    _check(lib().moe_eplb_tables(num_logical, p2l.size, p2l.ctypes.data, max_replicas,
                                 l2p.ctypes.data, cnt.ctypes.data), "moe_eplb_tables")
    return l2p, cnt


def moe_route_eplb(p, eplb, num_tokens, x, w_gate, logit_bias, expert_map, topk_ids, topk_w,
                   topk_local, ws, stream=None, score_bias=None):
    Tk = num_tokens * p.top_k
    _check_tensors(p, _route_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                    eplb.num_physical_experts)
                   + [("topk_ids", topk_ids, "i32", Tk), ("topk_w", topk_w, "f32", Tk),
                      ("topk_local", topk_local, "i32", Tk)])
    wp, wn = _ws(ws)
    _check(lib().moe_route_eplb(ctypes.byref(p), ctypes.byref(eplb), num_tokens, _ptr(x),
                                _ptr(w_gate), _ptr(logit_bias), _ptr(score_bias), _ptr(expert_map), _ptr(topk_ids),
                                _ptr(topk_w), _ptr(topk_local), wp, wn, _stream(stream)),
           "moe_route_eplb")


def moe_forward_eplb(p, eplb, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2, shared_w13,
                     shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None, score_bias=None,
                     b13=None, b2=None):
    _check_tensors(p, _forward_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                      eplb.num_physical_experts, w13, w2, b13, b2, shared_w13,
                                      shared_w2, out, topk_ids_out, topk_w_out))
    wp, wn = _ws(ws)
    _check(lib().moe_forward_eplb(ctypes.byref(p), ctypes.byref(eplb), num_tokens, _ptr(x),
                                  _ptr(w_gate), _ptr(logit_bias), _ptr(score_bias),
                                  _ptr(expert_map), _ptr(w13), _ptr(w2), _ptr(b13), _ptr(b2),
                                  _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                                  _ptr(topk_ids_out), _ptr(topk_w_out), wp, wn, _stream(stream)),
           "moe_forward_eplb")


def moe_forward_overlap(p, side, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2,
                        shared_w13, shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None,
                        score_bias=None, b13=None, b2=None, eplb=None):
    """moe_forward (or moe_forward_eplb with ``eplb``) with the shared expert on the caller's
    side stream; ``side`` is a ``moe_side_stream`` (see ``make_side_stream``) or None."""
    n_map = eplb.num_physical_experts if eplb is not None else p.num_experts
    _check_tensors(p, _forward_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                      n_map, w13, w2, b13, b2, shared_w13, shared_w2, out,
                                      topk_ids_out, topk_w_out))
    wp, wn = _ws(ws)
    _check(lib().moe_forward_overlap(ctypes.byref(p), ctypes.byref(eplb) if eplb is not None else None,
                                     ctypes.byref(side) if side is not None else None, num_tokens,
                                     _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(score_bias),
                                     _ptr(expert_map), _ptr(w13), _ptr(w2), _ptr(b13), _ptr(b2),
                                     _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                                     _ptr(topk_ids_out), _ptr(topk_w_out), wp, wn, _stream(stream)),
           "moe_forward_overlap")


def moe_forward_noalloc(p, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2, shared_w13,
                        shared_w2, out, topk_ids_out, topk_w_out, stream=None, score_bias=None,
                        b13=None, b2=None):
    """moe_forward on the library's own workspace array (no workspace argument, nothing
    allocated); MoeError(MOE_ENOSPC) when the call needs more than MOE_NOALLOC_SCRATCH_BYTES."""
    _check_tensors(p, _forward_checks(p, num_tokens, x, w_gate, logit_bias, score_bias, expert_map,
                                      p.num_experts, w13, w2, b13, b2, shared_w13, shared_w2, out,
                                      topk_ids_out, topk_w_out))
    _check(lib().moe_forward_noalloc(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w_gate),
                                     _ptr(logit_bias), _ptr(score_bias), _ptr(expert_map),
                                     _ptr(w13), _ptr(w2), _ptr(b13), _ptr(b2), _ptr(shared_w13),
                                     _ptr(shared_w2), _ptr(out), _ptr(topk_ids_out),
                                     _ptr(topk_w_out), _stream(stream)),
           "moe_forward_noalloc")
