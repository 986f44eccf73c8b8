#!/usr/bin/env python3
"""Benchmark of the fused MoE layer forward on one MI355X.

Metric: MoE-layer tokens/s on one GPU, with the dominant kernel's achieved fraction of
the MI355X roofline (bf16 MFMA peak 2.5 PFLOP/s for large-token shapes, HBM 8 TB/s for
weight-streaming shapes).

Default workload: the Mixtral-shaped layer (bf16, H 4096, 8 experts of I 14336, top-2
renormalised softmax routing, every expert local) at 4096 tokens (prefill); the same
layer at 32 tokens (decode) is reported in the ``decode`` field of the same line. A step
is one ``moe_forward`` over the batch (router GEMM, softmax/top-k, align/permute, grouped
gate/up and down GEMMs, combine); inputs are resident in HBM before timing starts. The
expert-parallel exchange around the path (dispatch and unpack, at the workload's EP degree)
is timed on the step's routing and reported in the ``ep_exchange`` field.

Expert weights are rearranged once at set-up into the packed layout (``moe_pack_weights``,
like a weight load; ``--weight-layout row_major`` keeps the plain one); ``config.weight_layout``
says which. Warm-up: the requested W steps, extended until at least 0.3 s of steps have run
(the GPU clock ramps over the first tens of milliseconds of load; ``warmup_run`` reports the
count). ``timing`` holds hipEvent times of 50 single steps, each after a 512 MB write that
evicts the MALL (median, p10, p90); ``configs`` holds the same for every configuration point of
the layer families, with each point's target and whether it is met.

The dominant kernel's duration comes from HIP events recorded on the launch stream
around ``moe_expert_gate_up`` in a second timed loop that runs the same kernels through
the split entry points. The oracle (CPU, float64 expert MLPs) is timed on a bounded
sample of tokens of the same workload as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]
                       [--tokens T] [--cpu-sample S | --no-cpu-baseline] [--copy-probe]
                       [--no-exchange | --exchange-only | --eplb R]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
# Sources that define the dominant (gate/up) kernel; a traffic figure measured with
# rocprofv3 counters is only reported while these hash to the value recorded with it.
KERNEL_SOURCES = ("expert_moe_amd/csrc/gemm.h", "expert_moe_amd/csrc/mlp.hip",
                  "expert_moe_amd/csrc/common.h")
TRAFFIC_PROFILE = "profiles/mixtral_T4096_hbm_traffic.md"


def kernel_fingerprint() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, T: int):
    """Counter-measured bytes per gate/up launch for the default workload, or None."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if workload != "mixtral" or T != 4096 or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", " ")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_fingerprint():
        return None
    try:
        return int(vals["gate_up_traffic_bytes"])
    except (KeyError, ValueError):
        return None


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 2000 steps: several seconds of timed GPU work on the default layer (2.4 ms a step), long
    # enough for a once-a-second utilisation sampler to see the GPU busy
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--tokens", type=int, default=None, help="token count (default: the largest)")
    ap.add_argument("--decode-tokens", type=int, default=None,
                    help="second, small token count reported as 'decode' (default: the smallest)")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens the oracle is timed on (capped at the workload's token count)")
    ap.add_argument("--no-decode", action="store_true", help="skip the small-token-count line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exchange", action="store_true",
                    help="skip the expert-parallel exchange (dispatch + unpack) measurement")
    ap.add_argument("--exchange-only", action="store_true",
                    help="route once, then time only the exchange (for kernel profiles)")
    ap.add_argument("--eplb", type=int, default=0, metavar="R",
                    help="only: per-rank layer times of the workload's EP group, plain shares "
                         "and with R redundant replicated experts")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the sweep over every configuration point")
    ap.add_argument("--config-steps", type=int, default=50,
                    help="flushed hipEvent steps per configuration point (median, p10, p90)")
    ap.add_argument("--no-slices", action="store_true",
                    help="skip the per-share times of the expert-parallel layers")
    ap.add_argument("--weight-layout", choices=("packed", "row_major"), default="packed",
                    help="expert weights on the device: packed once at set-up (moe_pack_weights, "
                         "bf16 layers) or as row-major tensors")
    return ap.parse_args()


class Bench:
    """Device inputs, outputs and workspace of one (workload, T) point."""

    def __init__(self, w, T, host):
        import torch

        import expert_moe_amd as moe
        self.w, self.T, self.moe, self.torch = w, T, moe, torch
        dev = "cuda"
        self.p = moe.make_params(w.num_experts, w.top_k, w.hidden_size, w.intermediate_size,
                                 w.renormalize, w.use_grouped_topk, w.num_expert_group,
                                 w.topk_group, w.routed_scaling_factor, w.num_local_experts,
                                 w.shared_intermediate_size, w.dtype, w.scoring_func,
                                 w.activation, layout_for(w))
        self.d = host.device_tensors(T)
        dt = self.d["x"].dtype
        k, H = w.top_k, w.hidden_size
        self.out = torch.empty(T, H, dtype=dt, device=dev)
        self.ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.tw = torch.empty(T, k, dtype=torch.float32, device=dev)
        self.ws = torch.empty(moe.moe_workspace_size(self.p, T), dtype=torch.uint8, device=dev)
        # split-path buffers (same kernels as moe_forward)
        self.bm = moe.moe_pick_block_m(self.p, T)
        cap = moe.moe_sorted_capacity(self.p, T, self.bm)
        self.local = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.sp = torch.empty(cap, dtype=torch.int32, device=dev)
        self.be = torch.empty(moe.block_expert_len(self.p, T, self.bm), dtype=torch.int32,
                              device=dev)
        self.pr = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.npad = torch.empty(1, dtype=torch.int32, device=dev)
        self.act = torch.empty(cap, w.intermediate_size, dtype=dt, device=dev)
        self.y = torch.empty(cap, H, dtype=dt, device=dev)
        self.sy = torch.empty(T, H, dtype=dt, device=dev) if w.shared_intermediate_size else None
        self.sws = torch.empty(moe.moe_workspace_size(self.p, T, self.bm), dtype=torch.uint8,
                               device=dev)
        # a shared expert runs beside the routed path on a side stream of ours (default
        # priority), forked and joined by two events
        self.side = None
        if w.shared_intermediate_size:
            st = torch.cuda.Stream(device=dev)
            fork, join = torch.cuda.Event(), torch.cuda.Event()
            fork.record(st)
            join.record(st)
            self.side = moe.make_side_stream(st, fork, join)

    def forward(self):
        d = self.d
        self.moe.moe_forward_overlap(self.p, self.side, self.T, d["x"], d["gate"], d["bias"],
                                     d["emap"], d["w13"], d["w2"], d["sw13"], d["sw2"], self.out,
                                     self.ids, self.tw, self.ws, score_bias=d["sbias"],
                                     b13=d["b13"], b2=d["b2"])

    def route_logits(self):
        """moe_route alone on the step's tokens; its fp32 router logits [T, E] (host numpy), which
        it leaves at the start of its workspace."""
        m, d, p, T = self.moe, self.d, self.p, self.T
        m.moe_route(p, T, d["x"], d["gate"], d["bias"], d["emap"], self.ids, self.tw, self.local,
                    self.sws, score_bias=d["sbias"])
        self.torch.cuda.synchronize()
        E = self.w.num_experts
        return self.sws[: T * E * 4].view(self.torch.float32).view(T, E).cpu().numpy()

    def split_step(self, ev=None):
        """The same kernels as moe_forward through the split entry points; events at stage ends."""
        m, d, p, T = self.moe, self.d, self.p, self.T
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        m.moe_route(p, T, d["x"], d["gate"], d["bias"], d["emap"], self.ids, self.tw, self.local,
                    self.sws, score_bias=d["sbias"])
        rec(1)
        m.moe_align_permute(p, T, self.local, self.bm, self.sp, self.be, self.pr, self.npad, self.sws)
        rec(2)
        m.moe_expert_gate_up(p, T, d["x"], d["w13"], self.sp, self.be, self.npad, self.bm, self.act,
                             b13=d["b13"])
        rec(3)
        m.moe_expert_down(p, T, self.act, d["w2"], self.be, self.npad, self.bm, self.y, b2=d["b2"])
        rec(4)
        if self.sy is not None:
            m.moe_shared_mlp(p, T, d["x"], d["sw13"], d["sw2"], self.sy, self.sws)
        rec(5)
        m.moe_combine(p, T, self.y, self.pr, self.tw, self.sy, self.out)
        rec(6)


# Layout of the expert weights on the device: "packed" (moe_pack_weights, once at set-up like a
# weight load; bf16 layers) or "row_major" (--weight-layout).
WEIGHT_LAYOUT = "packed"


def layout_for(w):
    return "packed" if WEIGHT_LAYOUT == "packed" and w.dtype == "bf16" else "row_major"


class HostLayer:
    """Seeded host inputs of the largest token count; device copies per token count."""

    def __init__(self, w, T_max):
        import workloads as wl
        self.w = w
        self.x = wl.x(w, T_max)
        self.gate = wl.gate(w)
        self.bias = wl.logit_bias(w)
        self.sbias = wl.score_bias(w)
        self.emap = wl.expert_map(w)
        self.w13, self.w2 = wl.local_expert_weights(w)
        self.sw13, self.sw2 = wl.shared_weights(w)
        self.b13, self.b2 = wl.expert_biases(w)
        self._dev = None

    def _weights_on_device(self):
        if self._dev is None:
            self._dev = {k: _dev(getattr(self, k)) for k in
                         ("gate", "bias", "sbias", "emap", "w13", "w2", "sw13", "sw2", "b13",
                          "b2")}
            if layout_for(self.w) == "packed":
                import expert_moe_amd as moe
                for k in ("w13", "w2", "sw13", "sw2"):
                    if self._dev[k] is not None:
                        self._dev[k] = moe.moe_pack_weights(self._dev[k])
        return self._dev

    def device_tensors(self, T):
        d = dict(self._weights_on_device())
        d["x"] = _dev(self.x[:T])
        return d


def _dev(a):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def algorithmic(w, T, ids):
    """Algorithmic work of one step from the actual routing (ids: numpy [T, k])."""
    import numpy as np
    import workloads as wl
    emap = wl.expert_map(w)
    slots = emap[ids]
    A = int((slots >= 0).sum())
    counts = np.bincount(slots[slots >= 0], minlength=w.num_local_experts)
    touched = int((counts > 0).sum())
    H, I, E, Is = w.hidden_size, w.intermediate_size, w.num_experts, w.shared_intermediate_size
    eb = 2 if w.dtype == "bf16" else 4
    flops = 2 * T * H * E + 6 * A * H * I + 6 * T * H * Is
    bytes_ = (touched * 3 * H * I + 3 * H * Is + E * H + 2 * T * H) * eb
    gate_up_flops = 4 * A * H * I
    gate_up_bytes = (touched * 2 * I * H + T * H + A * I) * eb
    return {"assignments": A, "touched_experts": touched, "flops": flops, "bytes": bytes_,
            "gate_up_flops": gate_up_flops, "gate_up_bytes": gate_up_bytes,
            "rows_per_expert_min": int(counts.min()), "rows_per_expert_max": int(counts.max())}


WARM_SECONDS = 0.3


def warm_up(fn, steps):
    """Untimed calls of fn: at least `steps`, and for at least WARM_SECONDS of GPU time. The
    GPU's clock ramps over the first tens of milliseconds of load (and again after an idle
    gap): a Mixtral-shaped step takes 3.4 ms at first and settles at 2.66 ms after about
    30 steps, so a fixed handful of warm-up steps would time the ramp. Returns the count."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < steps or time.perf_counter() - t0 < WARM_SECONDS:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


class SclkSampler:
    """Samples the GPU's current shader clock (the starred line of the DRM pp_dpm_sclk file)
    every 20 ms on a host thread while a timed loop runs; median in MHz, or None where the file
    cannot be read."""

    def __init__(self):
        import glob
        import threading
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if files else None
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().split("M")[0])
        return None

    def _run(self):
        while not self.stop.is_set():
            try:
                v = self._read()
                if v is not None and v > 200:  # deep-sleep readings between launches
                    self.samples.append(v)
            except (OSError, ValueError, IndexError):
                return
            self.stop.wait(0.02)

    def __enter__(self):
        if self.path:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.path:
            self.thread.join()

    def median_mhz(self):
        import statistics
        return statistics.median(self.samples) if self.samples else None


def run_point(host, w, T, steps, warmup):
    import torch
    b = Bench(w, T, host)
    b.warmup_run = warm_up(b.forward, warmup)
    with SclkSampler() as clk:
        t0 = time.perf_counter()
        for _ in range(steps):
            b.forward()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
    b.sclk_mhz = clk.median_mhz()
    ids = b.ids.cpu().numpy()
    alg = algorithmic(w, T, ids)

    # second timed loop: same kernels, HIP events on the launch stream at stage ends
    warm_up(b.split_step, 1)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        b.split_step(evs[i])
    torch.cuda.synchronize()
    split_ms = (time.perf_counter() - t0) * 1e3 / steps
    names = ["route", "align", "gate_up", "down", "shared", "combine"]
    stage = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i, n in enumerate(names)}

    return b, ms, split_ms, stage, alg


def roofline(alg, stage_ms, bound):
    sec = stage_ms["gate_up"] * 1e-3
    if bound == "mfma":
        achieved = alg["gate_up_flops"] / sec / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "moe_expert_gate_up (silu(x W1^T) * (x W3^T), grouped bf16 MFMA)",
                "per_launch": f"4*A*H*I = {alg['gate_up_flops']} FLOP", "avg_ms": round(stage_ms["gate_up"], 4)}
    achieved = alg["gate_up_bytes"] / sec / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
            "kernel": "moe_expert_gate_up (weight-streaming bf16 MFMA)",
            "per_launch": f"touched w13 + x + act = {alg['gate_up_bytes']} B",
            "avg_ms": round(stage_ms["gate_up"], 4)}


def res_frac_at_clock(roof, sclk_mhz):
    """The roofline fraction against the MFMA peak at the measured clock instead of 2.4 GHz."""
    return roof["frac"] * 2400.0 / sclk_mhz


def exchange_ep_size(w):
    """Expert-parallel degree of the exchange measurement: the workload's own, else one expert
    (Mixtral: eight) per rank, at most eight ranks."""
    return w.ep_size if w.ep_size > 1 else min(8, w.num_experts)


def run_exchange(w, T, ep, x, ids, tw, steps, warmup):
    """Dispatch and unpack of the expert-parallel exchange on the step's routing, timed with
    HIP events on the launch stream; algorithmic bytes from the actual send rows."""
    import numpy as np
    import torch

    import expert_moe_amd as moe
    p = moe.make_params(w.num_experts, w.top_k, w.hidden_size, w.intermediate_size, w.renormalize,
                        w.use_grouped_topk, w.num_expert_group, w.topk_group,
                        w.routed_scaling_factor, w.num_local_experts, w.shared_intermediate_size,
                        w.dtype)
    k, H = w.top_k, w.hidden_size
    dev, dt = x.device, x.dtype
    R = max(moe.moe_ep_send_capacity(p, T, ep), 1)
    send_pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    meta = torch.empty(2 * ep + 2, dtype=torch.int32, device=dev)
    send_token = torch.empty(R, dtype=torch.int32, device=dev)
    send_x = torch.empty(R, H, dtype=dt, device=dev)
    send_local = torch.empty(R, k, dtype=torch.int32, device=dev)
    send_w = torch.empty(R, k, dtype=torch.float32, device=dev)
    out = torch.empty(T, H, dtype=dt, device=dev)
    ws = torch.empty(max(moe.moe_ep_workspace_size(p, T, ep), 1), dtype=torch.uint8, device=dev)

    def dispatch():
        moe.moe_ep_dispatch(p, T, ep, ids, tw, x, send_pos, meta, send_token, send_x, send_local,
                            send_w, ws)

    def unpack():  # the returned rows stand in place: send_x plays recv_y
        moe.moe_ep_combine(p, T, send_pos, send_x, out)

    warm_up(lambda: (dispatch(), unpack()), warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        dispatch()
        e[1].record()
        unpack()
        e[2].record()
    torch.cuda.synchronize()
    d_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    c_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    n_send = int(meta[0].item())
    pos = send_pos.view(T, k).cpu().numpy()
    senders = int((pos >= 0).any(axis=1).sum())
    eb = 2 if w.dtype == "bf16" else 4
    # dispatch: ids/weights in, send_pos out, each sending token's row read once, the send rows
    # and their metadata written; unpack: send_pos and the returned rows in, the tokens out
    d_bytes = T * k * 12 + senders * H * eb + n_send * (H * eb + 4 + 8 * k)
    c_bytes = T * k * 4 + n_send * H * eb + T * H * eb
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    return {"ep_size": ep, "n_send": n_send, "rows_per_token": round(n_send / max(T, 1), 3),
            "dispatch_ms": round(d_ms, 4), "dispatch_bytes": d_bytes,
            "dispatch_gbs": round(gbs(d_bytes, d_ms), 1),
            "dispatch_hbm_frac": round(gbs(d_bytes, d_ms) / PEAK_HBM_GBS, 4),
            "unpack_ms": round(c_ms, 4), "unpack_bytes": c_bytes,
            "unpack_gbs": round(gbs(c_bytes, c_ms), 1),
            "unpack_hbm_frac": round(gbs(c_bytes, c_ms) / PEAK_HBM_GBS, 4),
            "counts": np.diff(meta[1:ep + 2].cpu().numpy()).tolist()}


def run_eplb(host, w, T, extra, steps, warmup):
    """Load balance of an expert-parallel group with and without replicated experts.

    Every rank's share of the routed experts (no shared expert) runs in turn on all T tokens,
    first with the plain contiguous shares, then with `extra` redundant replicas placed from
    the step's own expert loads; the group's step time is the slowest rank's."""
    import numpy as np
    import torch

    import expert_moe_amd as moe
    import workloads as wl
    ep, E, k, H = w.ep_size, w.num_experts, w.top_k, w.hidden_size
    dev = "cuda"
    x = _dev(host.x[:T])
    gate = _dev(host.gate)
    bias = _dev(host.bias)
    sbias = _dev(host.sbias)
    dt = x.dtype
    out = torch.empty(T, H, dtype=dt, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    cache = {}

    def expert(e):  # device weights (and biases, or None) of logical expert e, drawn once
        if e not in cache:
            a, b = wl.expert_weights(w, e)
            b13, b2 = wl.expert_biases(w, [e])
            cache[e] = (_dev(a), _dev(b), None if b13 is None else _dev(b13[0]),
                        None if b2 is None else _dev(b2[0]))
        return cache[e]

    def stack(experts, i):
        parts = [expert(int(e))[i] for e in experts]
        return None if parts[0] is None else torch.stack(parts)

    def time_share(p, emap, w13, w2, b13, b2, eplb=None):
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device=dev)

        def call():
            if eplb is None:
                moe.moe_forward(p, T, x, gate, bias, emap, w13, w2, None, None, out, ids, tw, ws,
                                score_bias=sbias, b13=b13, b2=b2)
            else:
                moe.moe_forward_eplb(p, eplb, T, x, gate, bias, emap, w13, w2, None, None, out,
                                     ids, tw, ws, score_bias=sbias, b13=b13, b2=b2)
        warm_up(call, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def params(n_local):
        return moe.make_params(E, k, H, w.intermediate_size, w.renormalize, w.use_grouped_topk,
                               w.num_expert_group, w.topk_group, w.routed_scaling_factor, n_local,
                               0, w.dtype, w.scoring_func, w.activation)

    per = E // ep
    plain_ms, plain_pairs = [], []
    for r in range(ep):
        emap = torch.from_numpy(moe.moe_make_expert_map(E, ep, r)).to(dev)
        mine = range(r * per, (r + 1) * per)
        plain_ms.append(time_share(params(per), emap, stack(mine, 0), stack(mine, 1),
                                   stack(mine, 2), stack(mine, 3)))
    ids_h = ids.cpu().numpy()
    loads = np.bincount(ids_h.ravel(), minlength=E)
    plain_pairs = [int(loads[r * per:(r + 1) * per].sum()) for r in range(ep)]
    P = E + extra
    p2l = wl.eplb_placement(loads + 1.0, P, ep)
    l2p, cnt = moe.moe_eplb_tables(E, p2l)
    eplb = moe.make_eplb(P, l2p.shape[1], torch.from_numpy(l2p).to(dev),
                         torch.from_numpy(cnt).to(dev))
    pp = P // ep
    eplb_ms, eplb_pairs = [], []
    for r in range(ep):
        pmap = np.full(P, -1, np.int32)
        pmap[r * pp:(r + 1) * pp] = np.arange(pp)
        mine = p2l[r * pp:(r + 1) * pp]
        eplb_ms.append(time_share(params(pp), torch.from_numpy(pmap).to(dev), stack(mine, 0),
                                  stack(mine, 1), stack(mine, 2), stack(mine, 3), eplb))
        # pairs that landed on this rank (replica t mod count of each pair's logical expert)
        t = np.arange(T)[:, None]
        phys = l2p[ids_h, t % cnt[ids_h]]
        eplb_pairs.append(int(((phys >= r * pp) & (phys < (r + 1) * pp)).sum()))
    return {"ep_size": ep, "redundant_experts": extra, "physical_experts": P,
            "placement": p2l.tolist(),
            "rank_ms_plain": [round(v, 4) for v in plain_ms],
            "rank_ms_eplb": [round(v, 4) for v in eplb_ms],
            "group_ms_plain": round(max(plain_ms), 4), "group_ms_eplb": round(max(eplb_ms), 4),
            "rank_pairs_plain": plain_pairs, "rank_pairs_eplb": eplb_pairs,
            "note": "routed experts only (no shared expert); each rank's share runs on all T "
                    "tokens in turn on one GPU; group time = slowest rank"}


# Every configuration point of the layer, with the roof it is graded on: prefill-shaped (large
# token count) points on bf16 MFMA (>= 50% of peak), decode-shaped (weight-streaming) points on
# HBM (>= 60%); the tiny fp32 layer is checked for parity only.
CONFIG_POINTS = (
    ("tiny", 64, None), ("mixtral", 32, "hbm"), ("mixtral", 4096, "mfma"),
    ("ep_share", 8192, "mfma"), ("dsv2", 4096, "mfma"),
    ("skewed", 1, "hbm"), ("skewed", 256, "hbm"), ("skewed", 16384, "mfma"),
)
TARGET_FRAC = {"mfma": 0.50, "hbm": 0.60}
TIE_GAP = 1e-6
FLUSH_BYTES = 512 << 20  # more than the 256 MB MALL


class Flusher:
    """Writes a 512 MB buffer, so the next step finds its weights in HBM, not in the MALL."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i)


def event_protocol(fn, steps, flush, warm=10):
    """hipEvent times of `steps` single steps (ms), each after a cache flush outside the timed
    region, following `warm` untimed steps: median, p10, p90."""
    import numpy as np
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": round(float(np.median(t)), 4), "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4), "steps": steps, "flush_bytes": FLUSH_BYTES}


def near_ties(w, logits, bias):
    """Tokens whose k-th/(k+1)-th selection-score gap (or, grouped, last kept / first dropped
    group gap) is below TIE_GAP, from the GPU's fp32 router logits (scores recomputed on the host
    for this report only)."""
    import numpy as np
    import workloads as wl
    l = logits.astype(np.float32)
    if bias is not None:
        l = (l + bias[None, :]).astype(np.float32)
    if w.scoring_func == "sigmoid":
        p = (1.0 / (1.0 + np.exp(-l.astype(np.float64)))).astype(np.float32)
    else:
        e = np.exp((l - l.max(axis=1, keepdims=True)).astype(np.float64))
        p = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    sb = wl.score_bias(w)
    s = p if sb is None else (p + sb[None, :]).astype(np.float32)
    T, E, k = s.shape[0], s.shape[1], w.top_k
    near = np.zeros(T, bool)
    if w.use_grouped_topk:
        G, keep = w.num_expert_group, w.topk_group
        grp = s.reshape(T, G, E // G)
        gs = grp.max(axis=2) if sb is None else np.sort(grp, axis=2)[:, :, -2:].sum(axis=2)
        order = np.argsort(-gs, axis=1, kind="stable")
        if keep < G:
            srt = np.take_along_axis(gs, order, axis=1)
            near |= (srt[:, keep - 1] - srt[:, keep]) < TIE_GAP
        mask = np.zeros((T, G), bool)
        np.put_along_axis(mask, order[:, :keep], True, axis=1)
        s = np.where(np.repeat(mask, E // G, axis=1), s, -np.inf)
        ncand = keep * (E // G)
    else:
        ncand = E
    if k < ncand:
        srt = -np.sort(-s, axis=1)
        near |= (srt[:, k - 1] - srt[:, k]) < TIE_GAP
    return int(near.sum())


def target(alg, bound):
    """Time a point may take at the graded fraction of its roof (ms), and its roof's peak."""
    if bound == "mfma":
        return alg["flops"] / (TARGET_FRAC["mfma"] * PEAK_BF16_TFLOPS * 1e12) * 1e3
    return alg["bytes"] / (TARGET_FRAC["hbm"] * PEAK_HBM_GBS * 1e9) * 1e3


def share_slices(host, w, T, base, steps, flush):
    """Every expert-parallel share of the layer in turn on one GPU (the routing is replicated,
    so every share sees the same tokens): each share's layer time, their sum and the slowest.
    The named share runs on its seeded weights; the other shares' experts are drawn on the GPU
    from the same distributions (their values do not change the time)."""
    import math
    import numpy as np
    import torch

    import expert_moe_amd as moe
    ep = w.ep_size
    E, El, H, I = w.num_experts, w.num_local_experts, w.hidden_size, w.intermediate_size
    ms = []
    d = base.d
    for r in range(ep):
        emap = torch.from_numpy(moe.moe_make_expert_map(E, ep, r)).cuda()
        if r == w.ep_rank:
            w13, w2 = d["w13"], d["w2"]
        else:
            g = torch.Generator(device="cuda").manual_seed(1000 + r)
            w13 = (torch.randn(El, 2 * I, H, device="cuda", generator=g) / math.sqrt(H)).bfloat16()
            w2 = (torch.randn(El, H, I, device="cuda", generator=g) / math.sqrt(I)).bfloat16()
        # the shared expert lives on rank 0's share
        sh = r == 0 and w.shared_intermediate_size > 0
        p = moe.make_params(E, w.top_k, H, I, w.renormalize, w.use_grouped_topk,
                            w.num_expert_group, w.topk_group, w.routed_scaling_factor, El,
                            w.shared_intermediate_size if sh else 0, w.dtype, w.scoring_func,
                            w.activation, layout_for(w))
        ws = torch.empty(moe.moe_workspace_size(p, T), dtype=torch.uint8, device="cuda")
        side = base.side if sh else None

        def call():
            moe.moe_forward_overlap(p, side, T, d["x"], d["gate"], d["bias"], emap, w13, w2,
                                    d["sw13"] if sh else None, d["sw2"] if sh else None, base.out,
                                    base.ids, base.tw, ws, score_bias=d["sbias"])
        ms.append(event_protocol(call, steps, flush, warm=5)["median_ms"])
        del ws, w13, w2
    return {"ep_size": ep, "share_ms": ms, "sum_ms": round(float(np.sum(ms)), 4),
            "max_ms": round(float(np.max(ms)), 4), "graded_share": w.ep_rank,
            "note": "each share in turn on one GPU, median of flushed hipEvent steps; the group's "
                    "step would take the slowest share (plus the exchange between ranks)"}


def run_configs(steps, flush, slices=True):
    """Every configuration point: layer time (flushed hipEvent median / p10 / p90), tokens/s,
    algorithmic FLOPs and bytes of the actual routing, the fraction of the graded roof, the
    target time and whether it is met, near-tie tokens, per-share times of the shared layers."""
    import numpy as np
    import torch

    import workloads as wl
    out = []
    hosts = {}
    for key, T, bound in CONFIG_POINTS:
        w = wl.WORKLOADS[key]
        print(f"[bench] config {key} T={T}", file=sys.stderr, flush=True)
        if key not in hosts:
            hosts.clear()
            torch.cuda.empty_cache()
            hosts[key] = HostLayer(w, max(w.tokens))
        b = Bench(w, T, hosts[key])
        warm_up(b.forward, 5)
        prot = event_protocol(b.forward, steps, flush)
        # back to back (no flush; weights may stay in the MALL where they fit)
        warm_up(b.forward, 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            b.forward()
        e1.record()
        torch.cuda.synchronize()
        b2b = e0.elapsed_time(e1) / steps
        ids = b.ids.cpu().numpy()
        alg = algorithmic(w, T, ids)
        nt = near_ties(w, b.route_logits(), hosts[key].bias)
        ms = prot["median_ms"]
        rec = {"workload": f"{w.desc}, T={T}", "key": key, "tokens": T, **prot,
               "back_to_back_ms": round(b2b, 4),
               "tokens_per_s": round(T / (ms * 1e-3), 1),
               "tflops": round(alg["flops"] / (ms * 1e-3) / 1e12, 2),
               "gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
               "assignments": alg["assignments"], "touched_experts": alg["touched_experts"],
               "rows_per_expert": [alg["rows_per_expert_min"], alg["rows_per_expert_max"]],
               "flops": alg["flops"], "bytes": alg["bytes"], "near_ties": nt}
        if bound is None:
            rec.update(bound=None, target_ms=None, met=None, note="parity only (fp32)")
        else:
            tgt = target(alg, bound)
            frac = (alg["flops"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if bound == "mfma"
                    else alg["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
            rec.update(bound=bound, frac=round(frac, 4), target_frac=TARGET_FRAC[bound],
                       target_ms=round(tgt, 4), met=bool(ms <= tgt),
                       met_back_to_back=bool(b2b <= tgt))
        if slices and w.ep_size > 1:
            rec["shares"] = share_slices(hosts[key], w, T, b, max(10, steps // 3), flush)
        out.append(rec)
        del b
    hosts.clear()
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(host, w, sample):
    """The oracle, as it stands, on `sample` tokens of the workload (CPU, float64 MLPs)."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    x = wl.to_f32(host.x[:sample])
    t0 = time.perf_counter()
    r = oracle.route(x, wl.to_f32(host.gate), w.top_k, w.renormalize, w.use_grouped_topk,
                     w.num_expert_group, w.topk_group, w.routed_scaling_factor, host.bias,
                     w.scoring_func, host.sbias)

    class Lazy:
        def __init__(self, a):
            self.a = a

        def __getitem__(self, s):
            return wl.to_f32(self.a[s])

    sh = (wl.to_f32(host.sw13), wl.to_f32(host.sw2)) if host.sw13 is not None else (None, None)
    oracle.moe_forward_given_routing(x, r["ids"], r["weights"], host.emap, Lazy(host.w13),
                                     Lazy(host.w2), sh[0], sh[1], w.activation, host.b13, host.b2)
    dt = time.perf_counter() - t0
    res = {"value": round(sample / dt, 3), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle", "seconds": round(dt, 2),
           "sample": f"first {sample} tokens of the same layer (routing + every local expert MLP "
                     f"in float64), whole-step time",
           "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}
    # the same oracle on one core (BLAS limited to one thread), on a smaller sample
    try:
        from threadpoolctl import threadpool_limits
        n1 = max(1, min(sample, 256))
        x1 = wl.to_f32(host.x[:n1])
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            r1 = oracle.route(x1, wl.to_f32(host.gate), w.top_k, w.renormalize, w.use_grouped_topk,
                              w.num_expert_group, w.topk_group, w.routed_scaling_factor, host.bias,
                              w.scoring_func, host.sbias)
            oracle.moe_forward_given_routing(x1, r1["ids"], r1["weights"], host.emap,
                                             Lazy(host.w13), Lazy(host.w2), sh[0], sh[1],
                                             w.activation, host.b13, host.b2)
            d1 = time.perf_counter() - t0
        res["single_core"] = {"value": round(n1 / d1, 3), "unit": "tokens/s", "cores": 1,
                              "sample": f"first {n1} tokens", "seconds": round(d1, 2)}
    except ImportError:  # pragma: no cover
        pass
    return res


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: each expert-parallel share is benchmarked on its own GPU.",
              file=sys.stderr)
        sys.exit(2)
    global WEIGHT_LAYOUT
    WEIGHT_LAYOUT = args.weight_layout
    import torch

    import workloads as wl
    w = wl.WORKLOADS[args.workload]
    T = args.tokens or max(w.tokens)
    Td = args.decode_tokens or min(w.tokens)
    print(f"[bench] generating inputs for {w.key} (T={T})", file=sys.stderr, flush=True)
    host = HostLayer(w, max(T, Td))
    torch.cuda.init()
    if args.eplb:
        print(json.dumps({"workload": f"{w.desc}, T={T}",
                          "eplb": run_eplb(host, w, T, args.eplb, args.steps, args.warmup)}))
        return
    if args.exchange_only:
        b = Bench(w, T, host)
        b.forward()
        torch.cuda.synchronize()
        print(json.dumps({"workload": f"{w.desc}, T={T}",
                          "ep_exchange": run_exchange(w, T, exchange_ep_size(w), b.d["x"], b.ids,
                                                      b.tw, args.steps, args.warmup)}))
        return
    print("[bench] timing", file=sys.stderr, flush=True)
    b, ms, split_ms, stage, alg = run_point(host, w, T, args.steps, args.warmup)
    bound = "mfma" if alg["gate_up_flops"] / max(alg["gate_up_bytes"], 1) > 312 else "hbm"
    flush = Flusher()
    timing = event_protocol(b.forward, max(50, args.config_steps), flush)
    n_near = near_ties(w, b.route_logits(), host.bias)
    res = {
        "metric": "MoE-layer tokens/s on 1 MI355X",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": b.warmup_run,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": f"{w.desc}, T={T}", "tokens": T, "hidden": w.hidden_size,
                   "experts": w.num_experts, "local_experts": w.num_local_experts,
                   "intermediate": w.intermediate_size, "top_k": w.top_k,
                   "shared_intermediate": w.shared_intermediate_size, "block_m": b.bm,
                   "weight_layout": layout_for(w)},
        "achieved_tflops": round(alg["flops"] / (ms * 1e-3) / 1e12, 2),
        "achieved_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
        "roofline": dict(roofline(alg, stage, bound), traffic=measured_traffic(w.key, T)),
        # the shader clock during the timed loop (median of 20 ms samples) and the dominant
        # kernel's fraction of the MFMA peak at that clock (the peak scales with it; 2.4 GHz)
        "sclk_mhz": b.sclk_mhz,
        "frac_at_clock": (round(res_frac_at_clock(roofline(alg, stage, bound), b.sclk_mhz), 4)
                          if b.sclk_mhz and bound == "mfma" else None),
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "split_path_ms_per_step": round(split_ms, 4),
        "timing": dict(timing, note="single steps timed with hipEvents after a 512 MB cache "
                                    "flush each; ms_per_step is the back-to-back wall-clock mean"),
        "near_ties": n_near,
        "work": alg,
    }
    if not args.no_exchange:
        print("[bench] timing the expert-parallel exchange", file=sys.stderr, flush=True)
        res["ep_exchange"] = run_exchange(w, T, exchange_ep_size(w), b.d["x"], b.ids, b.tw,
                                          max(args.steps, 20), args.warmup)
    del b
    if Td != T and not args.no_decode:
        bd, msd, split_d, stage_d, alg_d = run_point(host, w, Td, max(args.steps, 20), args.warmup)
        bound_d = "mfma" if alg_d["gate_up_flops"] / max(alg_d["gate_up_bytes"], 1) > 312 else "hbm"
        res["decode"] = {"tokens": Td, "value": round(Td / (msd * 1e-3), 1), "unit": "tokens/s",
                         "ms_per_step": round(msd, 4),
                         "achieved_gbs": round(alg_d["bytes"] / (msd * 1e-3) / 1e9, 1),
                         "hbm_frac_whole_step": round(alg_d["bytes"] / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "roofline": roofline(alg_d, stage_d, bound_d),
                         "stages_ms": {k: round(v, 4) for k, v in stage_d.items()}, "work": alg_d}
        del bd
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(host, w, min(args.cpu_sample, T))
    if not args.no_configs:
        del host
        res["configs"] = run_configs(args.config_steps, flush, slices=not args.no_slices)
        met = [c for c in res["configs"] if c.get("met") is not None]
        res["configs_met"] = f"{sum(c['met'] for c in met)} of {len(met)}"
    print(json.dumps(res))


if __name__ == "__main__":
    main()
