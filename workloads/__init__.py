"""Synthetic workloads for the fused MoE layer: the five layer shapes and their seeded inputs.

This module holds no part of the MoE computation. It only describes the workload
shapes and draws their input tensors, so that the GPU path (through its tests and
bench) and the CPU oracle receive byte-identical arrays.

Workload shapes. Each one is an expert-parallel rank's share of one MoE layer, in the
vocabulary of the pages: ``num_experts`` (E), ``top_k`` (k), ``hidden_size`` (H),
``intermediate_size`` (I, full size: no tensor-parallel split), ``renormalize``,
``use_grouped_topk`` / ``num_expert_group`` / ``topk_group``, ``routed_scaling_factor``
and the shared expert, as the EP-aware ``FusedMoE`` constructor on the page
"ep_fused_moe_patch.py: EP-aware FusedMoE override for vllm 0.6.3" (``_ep_init``) and
the config-field mapping of ``MoEMixin.recursive_replace`` on the page
"vllm.model_executor.models.transformers.moe" name them.

Input recipe (all draws from the counter-based stream in ``gen.c``):

* x       : role 0, N(0, 1), row-major [T_max, H]; a run with T tokens takes the first
            T rows, so smaller token counts are prefixes of larger ones.
* gate    : role 1, N(0, 1/H), [E, H]; this makes the router logits about N(0, 1).
* experts : role 3, index 3e+0 (W1, gate rows), 3e+1 (W3, up rows), 3e+2 (W2); W1 and W3
            ~ N(0, 1/H) as [I, H], W2 ~ N(0, 1/I) as [H, I]. Seeded by the GLOBAL expert
            id, so a share draws only its own experts and any share is reproducible alone.
* shared  : role 4, index 0/1/2 for Ws1/Ws3/Ws2 with I_s in place of I.
* bias    : the skewed-load layer adds b[e] = -1.2 ln(e + 1) to the router logits, so
            exp(b) is a Zipf(s = 1.2) law over expert rank (expert 0 most popular).

Values are drawn in fp32; bf16 workloads round them to bf16 (round-to-nearest-even)
and both sides consume the rounded values. bf16 arrays are numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwlgen.so")
_lib = None


def build_lib() -> str:
    """Compile gen.c into libwlgen.so next to this file (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        for name in ("wl_normal_f32", "wl_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, i64, i64, ctypes.c_double, ctypes.c_void_p]
            fn.restype = None
        for name in ("wl_normal_rows_f32", "wl_normal_rows_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, ctypes.c_void_p, i64, i64, ctypes.c_double, ctypes.c_void_p]
            fn.restype = None
        _lib = lib
    return _lib


def normal(stream, count, std=1.0, start=0, dtype="f32", out=None):
    """``count`` consecutive draws of a stream (a 3-int tuple), from element ``start``.

    ``out``: optional C-contiguous array of ``count`` elements (float32 / uint16) to fill.
    """
    a, b, c = stream
    want = {"f32": np.float32, "bf16": np.uint16}[dtype]
    if out is None:
        out = np.empty(count, want)
    if out.dtype != want or out.size != count or not out.flags.c_contiguous:
        raise ValueError("out must be a C-contiguous array of the requested type and size")
    fn = _load().wl_normal_f32 if dtype == "f32" else _load().wl_normal_bf16
    fn(a, b, c, start, count, float(std), out.ctypes.data)
    return out


def normal_rows(stream, rows, cols, std=1.0, dtype="f32"):
    """Rows ``rows`` of the stream viewed as a row-major [*, cols] matrix."""
    a, b, c = stream
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    if dtype == "f32":
        out = np.empty((n, cols), np.float32)
        _load().wl_normal_rows_f32(a, b, c, rows.ctypes.data, n, cols, float(std), out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty((n, cols), np.uint16)
        _load().wl_normal_rows_bf16(a, b, c, rows.ctypes.data, n, cols, float(std), out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f32(a: np.ndarray) -> np.ndarray:
    """Values of a workload array as float32 (exact for both storage types)."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


@dataclass(frozen=True)
class Workload:
    key: str
    cid: int
    desc: str
    dtype: str  # "f32" or "bf16"
    tokens: tuple
    hidden_size: int
    num_experts: int
    intermediate_size: int
    top_k: int
    renormalize: bool
    use_grouped_topk: bool = False
    num_expert_group: int = 1
    topk_group: int = 1
    routed_scaling_factor: float = 1.0
    ep_size: int = 1
    ep_rank: int = 0
    shared_intermediate_size: int = 0
    zipf_bias: float = 0.0  # s of the Zipf logit bias; 0 = none
    scoring_func: str = "softmax"  # or "sigmoid"
    score_bias_std: float = 0.0  # std of the seeded selection bias N(0, std^2); 0 = none
    activation: str = "silu"  # or "swigluoai"
    expert_bias_std: float = 0.0  # std of the seeded expert biases N(0, std^2); 0 = none
    extra: dict = field(default_factory=dict)

    @property
    def num_local_experts(self) -> int:
        return self.num_experts // self.ep_size

    @property
    def local_experts(self) -> range:
        n = self.num_local_experts
        return range(self.ep_rank * n, (self.ep_rank + 1) * n)

    def with_share(self, ep_size: int, ep_rank: int, shared: bool | None = None) -> "Workload":
        """The same layer seen from another expert-parallel share.

        The shared expert is carried by rank 0 only (so a sum over shares counts it
        once) unless ``shared`` says otherwise.
        """
        s = self.shared_intermediate_size if (shared if shared is not None else ep_rank == 0) else 0
        return Workload(**{**self.__dict__, "ep_size": ep_size, "ep_rank": ep_rank,
                           "shared_intermediate_size": s if self.shared_intermediate_size else 0})


WORKLOADS = {
    "tiny": Workload("tiny", 1, "tiny MoE layer, fp32", "f32", (64,), 128, 8, 256, 2, True),
    "mixtral": Workload("mixtral", 2, "Mixtral-shaped layer, bf16", "bf16", (32, 4096),
                        4096, 8, 14336, 2, True),
    "ep_share": Workload("ep_share", 3, "fine-grained EP share, bf16 (experts 64..127 of 256)",
                         "bf16", (8192,), 2048, 256, 512, 8, True, ep_size=4, ep_rank=1),
    "dsv2": Workload("dsv2", 4, "DeepSeek-V2-shaped layer, bf16 (experts 0..19 of 160)", "bf16",
                     (4096,), 5120, 160, 1536, 6, False, use_grouped_topk=True,
                     num_expert_group=8, topk_group=3, routed_scaling_factor=16.0,
                     ep_size=8, ep_rank=0, shared_intermediate_size=2 * 1536),
    "skewed": Workload("skewed", 5, "skewed-load layer, bf16 (experts 0..7 of 64)", "bf16",
                       (1, 256, 16384), 4096, 64, 3072, 8, True, ep_size=8, ep_rank=0,
                       shared_intermediate_size=3072, zipf_bias=1.2),
    # routing variants: sigmoid scores, selection-only bias, group score = top-2 sum
    "dsv3": Workload("dsv3", 6, "DeepSeek-V3-shaped layer, bf16 (experts 0..31 of 256, sigmoid "
                     "scores with a selection bias)", "bf16", (32, 4096), 7168, 256, 2048, 8, True,
                     use_grouped_topk=True, num_expert_group=8, topk_group=4,
                     routed_scaling_factor=2.5, ep_size=8, ep_rank=0,
                     shared_intermediate_size=2048, scoring_func="sigmoid", score_bias_std=0.05),
    # MLP variants: gpt-oss's clamped SwiGLU and expert biases
    "gptoss": Workload("gptoss", 7, "gpt-oss-shaped layer, bf16 (experts 0..15 of 128, clamped "
                       "SwiGLU, expert biases)", "bf16", (32, 4096), 2880, 128, 2880, 4, True,
                       ep_size=8, ep_rank=0, activation="swigluoai", expert_bias_std=0.1),
}


def expert_map(w: Workload) -> np.ndarray:
    """int32 [E]: local slot of each global expert for the workload's share, -1 elsewhere.

    Contiguous shares of E/ep_size experts, starting at ep_rank * E/ep_size, as the
    EP-aware ``_ep_init`` on the ep_fused_moe_patch.py page sets them up.
    """
    m = np.full(w.num_experts, -1, np.int32)
    n = w.num_local_experts
    m[w.ep_rank * n:(w.ep_rank + 1) * n] = np.arange(n, dtype=np.int32)
    return m


def x(w: Workload, T: int, start: int = 0) -> np.ndarray:
    """Activations [T, H], rows start..start+T-1 of the token stream."""
    H = w.hidden_size
    return normal((w.cid, 0, 0), T * H, 1.0, start * H, w.dtype).reshape(T, H)


def x_rows(w: Workload, rows) -> np.ndarray:
    return normal_rows((w.cid, 0, 0), rows, w.hidden_size, 1.0, w.dtype)


def gate(w: Workload) -> np.ndarray:
    """Router gate weight [E, H] (replicated on every share)."""
    E, H = w.num_experts, w.hidden_size
    return normal((w.cid, 1, 0), E * H, 1.0 / math.sqrt(H), 0, w.dtype).reshape(E, H)


def logit_bias(w: Workload):
    """fp32 [E] bias added to the router logits, or None."""
    if not w.zipf_bias:
        return None
    e = np.arange(w.num_experts, dtype=np.float64)
    return (-w.zipf_bias * np.log(e + 1.0)).astype(np.float32)


def score_bias(w: Workload):
    """fp32 [E] selection-only score bias (seeded N(0, std^2)), or None."""
    if not w.score_bias_std:
        return None
    return normal((w.cid, 5, 0), w.num_experts, w.score_bias_std).astype(np.float32)


def expert_biases(w: Workload, experts=None):
    """fp32 (b13 [n, 2I], b2 [n, H]) of the given global experts (default: the share's local
    experts), seeded N(0, std^2) per expert; (None, None) when the layer has none."""
    if not w.expert_bias_std:
        return None, None
    experts = list(w.local_experts if experts is None else experts)
    I, H = w.intermediate_size, w.hidden_size
    b13 = np.stack([normal((w.cid, 6, 2 * e), 2 * I, w.expert_bias_std) for e in experts])
    b2 = np.stack([normal((w.cid, 6, 2 * e + 1), H, w.expert_bias_std) for e in experts])
    return b13.astype(np.float32), b2.astype(np.float32)


def _storage(w: Workload):
    return np.uint16 if w.dtype == "bf16" else np.float32


def _fill_mlp(w: Workload, role: int, idx: int, I: int, w13: np.ndarray, w2: np.ndarray):
    """Draw one MLP's weights into w13 [2I, H] (gate rows, then up rows) and w2 [H, I]."""
    H = w.hidden_size
    s1 = 1.0 / math.sqrt(H)
    normal((w.cid, role, 3 * idx + 0), I * H, s1, 0, w.dtype, out=w13[:I].reshape(-1))
    normal((w.cid, role, 3 * idx + 1), I * H, s1, 0, w.dtype, out=w13[I:].reshape(-1))
    normal((w.cid, role, 3 * idx + 2), H * I, 1.0 / math.sqrt(I), 0, w.dtype, out=w2.reshape(-1))


def expert_weights(w: Workload, e: int):
    """(w13 [2I, H] = [W1 rows; W3 rows], w2 [H, I]) of GLOBAL expert e."""
    I, H = w.intermediate_size, w.hidden_size
    w13 = np.empty((2 * I, H), _storage(w))
    w2 = np.empty((H, I), _storage(w))
    _fill_mlp(w, 3, e, I, w13, w2)
    return w13, w2


def local_expert_weights(w: Workload):
    """Packed weights of the share: w13 [E_l, 2I, H], w2 [E_l, H, I]."""
    I, H, n = w.intermediate_size, w.hidden_size, w.num_local_experts
    w13 = np.empty((n, 2 * I, H), _storage(w))
    w2 = np.empty((n, H, I), _storage(w))
    for s, e in enumerate(w.local_experts):
        _fill_mlp(w, 3, e, I, w13[s], w2[s])
    return w13, w2


def shared_weights(w: Workload):
    """(sw13 [2 I_s, H], sw2 [H, I_s]) or (None, None) when the share has no shared expert."""
    if not w.shared_intermediate_size:
        return None, None
    I, H = w.shared_intermediate_size, w.hidden_size
    w13 = np.empty((2 * I, H), _storage(w))
    w2 = np.empty((H, I), _storage(w))
    _fill_mlp(w, 4, 0, I, w13, w2)
    return w13, w2


def eplb_placement(loads, num_physical: int, ep_size: int) -> np.ndarray:
    """A replicated placement for given per-expert loads (an input of the layer, like the
    expert map): physical_to_logical [num_physical], rank r holding ids r*P_l .. (r+1)*P_l-1.

    Greedy: each redundant replica goes to the expert with the most load per replica; then
    the replicas, heaviest first, go to the least-loaded rank with a free slot that does not
    already hold that expert (if any such rank exists).
    """
    loads = np.asarray(loads, np.float64)
    E = loads.shape[0]
    if num_physical < E or num_physical % ep_size:
        raise ValueError("num_physical must be >= E and divisible by ep_size")
    reps = np.ones(E, np.int64)
    for _ in range(num_physical - E):
        reps[int(np.argmax(loads / reps))] += 1
    items = sorted(((loads[e] / reps[e], e) for e in range(E) for _ in range(reps[e])),
                   key=lambda it: (-it[0], it[1]))
    per = num_physical // ep_size
    slots = [[] for _ in range(ep_size)]
    total = np.zeros(ep_size)
    for ld, e in items:
        free = [r for r in range(ep_size) if len(slots[r]) < per]
        fresh = [r for r in free if e not in slots[r]] or free
        r = min(fresh, key=lambda q: (total[q], q))
        slots[r].append(e)
        total[r] += ld
    return np.array([e for r in range(ep_size) for e in slots[r]], np.int32)
