"""Python binding of the gfx950 fused MoE library (``libexpert_moe.so``).

Argument marshalling only: every function here has the name of the C entry point it
calls (declared in ``include/moe.h``), turns tensors into device pointers and the
current torch stream into a ``hipStream_t``, and raises :class:`MoeError` on a negative
return code. All computation happens in the HIP kernels; there is no fallback path, and
importing a function fails loudly when the library has not been built.

Tensor arguments are ``torch`` tensors already on the GPU (bf16 data is passed as
``torch.bfloat16``; fp32 as ``torch.float32``; ids as ``torch.int32``); ``None`` passes
NULL. PyTorch is used for device memory and streams only.
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

# every symbol include/moe.h declares
EXPORTS = (
    "moe_strerror", "moe_check_params", "moe_pick_block_m", "moe_sorted_capacity",
    "moe_workspace_size", "moe_make_expert_map", "moe_weight_bytes", "moe_route",
    "moe_align_permute", "moe_grouped_mlp", "moe_expert_gate_up", "moe_expert_down",
    "moe_shared_mlp", "moe_combine", "moe_forward",
    "moe_ep_send_capacity", "moe_ep_workspace_size", "moe_ep_dispatch", "moe_ep_combine",
    "moe_eplb_tables", "moe_route_eplb", "moe_forward_eplb",
)


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
    ]


class moe_eplb(ctypes.Structure):
    """Mirror of ``struct moe_eplb`` in include/moe.h (device table pointers as integers)."""
    _fields_ = [
        ("num_physical_experts", ctypes.c_int32),
        ("max_replicas", ctypes.c_int32),
        ("logical_to_physical", ctypes.c_void_p),
        ("replica_count", ctypes.c_void_p),
    ]


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
                dtype="bf16", scoring_func="softmax", activation="silu") -> moe_params:
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
    return moe_params(
        int(num_experts), int(top_k), int(hidden_size), int(intermediate_size),
        int(bool(renormalize)), int(bool(use_grouped_topk)), int(num_expert_group),
        int(topk_group), float(routed_scaling_factor),
        int(num_experts if num_local_experts is None else num_local_experts),
        int(shared_intermediate_size), MOE_BF16 if dtype in ("bf16", MOE_BF16) else MOE_F32, sf,
        act)


_lib = None
_P = ctypes.POINTER(moe_params)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_SIGS = {
    "moe_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "moe_check_params": ([_P], ctypes.c_int),
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


def moe_route(p, num_tokens, x, w_gate, logit_bias, expert_map, topk_ids, topk_w, topk_local,
              ws, stream=None, score_bias=None):
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w_gate), _ptr(logit_bias),
                           _ptr(score_bias), _ptr(expert_map), _ptr(topk_ids), _ptr(topk_w), _ptr(topk_local),
                           wp, wn, _stream(stream)), "moe_route")


def moe_align_permute(p, num_tokens, topk_local, block_m, sorted_pairs, block_expert, pair_row,
                      num_padded, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_align_permute(ctypes.byref(p), num_tokens, _ptr(topk_local), block_m,
                                   _ptr(sorted_pairs), _ptr(block_expert), _ptr(pair_row),
                                   _ptr(num_padded), wp, wn, _stream(stream)), "moe_align_permute")


def moe_grouped_mlp(p, num_tokens, x, w13, w2, sorted_pairs, block_expert, num_padded, block_m,
                    y, ws, stream=None, b13=None, b2=None):
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_mlp(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w13), _ptr(w2),
                                 _ptr(b13), _ptr(b2), _ptr(sorted_pairs), _ptr(block_expert), _ptr(num_padded),
                                 block_m, _ptr(y), wp, wn, _stream(stream)), "moe_grouped_mlp")


def moe_expert_gate_up(p, num_tokens, x, w13, sorted_pairs, block_expert, num_padded, block_m,
                       act, stream=None, b13=None):
    _check(lib().moe_expert_gate_up(ctypes.byref(p), num_tokens, _ptr(x), _ptr(w13), _ptr(b13),
                                    _ptr(sorted_pairs), _ptr(block_expert), _ptr(num_padded),
                                    block_m, _ptr(act), _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(p, num_tokens, act, w2, block_expert, num_padded, block_m, y, stream=None,
                    b2=None):
    _check(lib().moe_expert_down(ctypes.byref(p), num_tokens, _ptr(act), _ptr(w2), _ptr(b2),
                                 _ptr(block_expert), _ptr(num_padded), block_m, _ptr(y),
                                 _stream(stream)), "moe_expert_down")


def moe_shared_mlp(p, num_tokens, x, shared_w13, shared_w2, shared_y, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_shared_mlp(ctypes.byref(p), num_tokens, _ptr(x), _ptr(shared_w13),
                                _ptr(shared_w2), _ptr(shared_y), wp, wn, _stream(stream)),
           "moe_shared_mlp")


def moe_combine(p, num_tokens, y, pair_row, topk_w, shared_y, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(p), num_tokens, _ptr(y), _ptr(pair_row), _ptr(topk_w),
                             _ptr(shared_y), _ptr(out), _stream(stream)), "moe_combine")


def moe_forward(p, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2, shared_w13,
                shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None, score_bias=None,
                b13=None, b2=None):
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
    wp, wn = _ws(ws)
    _check(lib().moe_ep_dispatch(ctypes.byref(p), num_tokens, ep_size, _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(x), _ptr(send_pos), _ptr(rank_meta), _ptr(send_token),
                                 _ptr(send_x), _ptr(send_local), _ptr(send_w), wp, wn,
                                 _stream(stream)), "moe_ep_dispatch")


def moe_ep_combine(p, num_tokens, send_pos, recv_y, out, stream=None):
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
    wp, wn = _ws(ws)
    _check(lib().moe_route_eplb(ctypes.byref(p), ctypes.byref(eplb), num_tokens, _ptr(x),
                                _ptr(w_gate), _ptr(logit_bias), _ptr(score_bias), _ptr(expert_map), _ptr(topk_ids),
                                _ptr(topk_w), _ptr(topk_local), wp, wn, _stream(stream)),
           "moe_route_eplb")


def moe_forward_eplb(p, eplb, num_tokens, x, w_gate, logit_bias, expert_map, w13, w2, shared_w13,
                     shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None, score_bias=None,
                     b13=None, b2=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward_eplb(ctypes.byref(p), ctypes.byref(eplb), num_tokens, _ptr(x),
                                  _ptr(w_gate), _ptr(logit_bias), _ptr(score_bias),
                                  _ptr(expert_map), _ptr(w13), _ptr(w2), _ptr(b13), _ptr(b2),
                                  _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                                  _ptr(topk_ids_out), _ptr(topk_w_out), wp, wn, _stream(stream)),
           "moe_forward_eplb")
