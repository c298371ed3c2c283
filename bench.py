#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel hot path on one MI355X.

One step = one pass of the whole path over one batch: dispatch layout ->
dispatch -> combine (expert outputs are a resident bf16 N(0,1) buffer in
receive-row order).  Inputs are seeded, synthetic and resident in HBM before
the timed region.  Several independent buffer sets (identical inputs) are
used in rotation (``rotation_sets``): between two uses of one set's source
rows the other sets' source rows cover twice the 256 MB last-level cache.

Timed region (``ms_per_step``, ``value``): exactly K steps (default 200, after
100 warm-up steps) of layout -> dispatch -> combine, replayed from HIP graphs
that each hold 16 consecutive steps on the buffer sets in rotation (every step
runs all three kernels), bracketed by a synchronize on both sides.  ``value`` = whole-step algorithmic bytes / step
time.  Graphs remove the host launch gaps that dominate at decode sizes; the
same K steps as eager launches give ``ms_per_step_eager``, with HIP events
between the ops for the per-op times (``us_mean``...).  Each op is also timed
as a graph of back-to-back launches of that op alone (``us_kernel``);
``layout+dispatch`` is the send side end to end (both ops, same timings);
``layout_dispatch_one_call`` is the same work through moe_layout_dispatch (one
kernel for batches up to 1024 tokens), and ``ms_per_step_one_call`` the step
replayed with it in place of the two calls.

    python bench.py [--steps K] [--warmup W] [--workload prefill|decode|...]

Algorithmic bytes (what the method must move once; distinct rows once):
  layout   = T*k*4 + T*R + 4*(R + E)
  dispatch = T*H*2 + T*k*8 + T*R + N*(H*b + S + 4 + 8*k) + T*R*4
             (b = 2, S = 0 for bf16; b = 1, S = 4*H/128 for FP8)
  combine  = N*H*2 + T*k*8 + T*R*4 + T*H*2
with N = number of receive rows.  The low-latency (per-expert) path, also
measured on the decode workload:
  dispatch_ll = T*H*2 + T*k*4 + N'*(H*b + S + 4) + E*4 + T*k*4
  combine_ll  = N'*H*2 + T*k*12 + T*H*2
with N' = rows written into the per-expert buffers.  The backward (training)
ops, measured on the main workload:
  combine_backward  = T*H*2 + N*H*2 + T*k*8 + T*R*4 + N*H*2 + T*k*4
  dispatch_backward = N*H*2 + T*R*4 + N*k*4 + T*k*4 + T*H*2 + T*k*4
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch/combine achieved HBM GB/s + µs/call, 128-tok decode & 4096-tok prefill"
HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
ROTATION_BYTES = 1 << 30  # buffer sets in rotation cover at least this much memory
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
MAX_SETS = 16
OPS = ("layout", "dispatch", "combine")
FUSED = "layout_dispatch_one_call"  # moe_layout_dispatch: layout and dispatch in one call
STEPS_PER_GRAPH = 16  # consecutive steps captured in one graph for the timed replays


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, n_recv: int) -> dict:
    T, H, k, E, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    fp8 = cfg.dispatch_dtype == "fp8"
    b, S = (1, 4 * H // 128) if fp8 else (2, 0)
    return {
        "layout": T * k * 4 + T * R + 4 * (R + E),
        "dispatch": T * H * 2 + T * k * 8 + T * R + n_recv * (H * b + S + 4 + 8 * k) + T * R * 4,
        "combine": n_recv * H * 2 + T * k * 8 + T * R * 4 + T * H * 2,
    }


def ll_algorithmic_bytes(cfg, n_rows: int) -> dict:
    T, H, k, E = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts
    b, S = (1, 4 * H // 128) if cfg.dispatch_dtype == "fp8" else (2, 0)
    return {
        "dispatch_ll": T * H * 2 + T * k * 4 + n_rows * (H * b + S + 4) + E * 4 + T * k * 4,
        "combine_ll": n_rows * H * 2 + T * k * 12 + T * H * 2,
    }


def bwd_algorithmic_bytes(cfg, n_recv: int) -> dict:
    T, H, k, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_ranks
    return {
        "combine_backward": T * H * 2 + n_recv * H * 2 + T * k * 8 + T * R * 4 + n_recv * H * 2 + T * k * 4,
        "dispatch_backward": n_recv * H * 2 + T * R * 4 + n_recv * k * 4 + T * k * 4 + T * H * 2 + T * k * 4,
    }


# The sources that decide what an op's kernels do: its kernel header, the shared device helpers
# and the host code that picks launch shapes.
OP_SOURCES = {
    "dispatch": ("dispatch_kernels.h", "device_common.h", "moe_ep.hip"),
    "combine": ("combine_kernels.h", "device_common.h", "moe_ep.hip"),
    "layout": ("layout_kernels.h", "device_common.h", "moe_ep.hip"),
}


def kernel_source_hash(op: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_get_dispatch_07_amd", "csrc")
    for name in sorted(OP_SOURCES[op]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, op: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they match the current kernels."""
    path = os.path.join(PROFILE_DIR, f"traffic_{op}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(op):
        return None
    return rec.get("hbm_bytes_per_launch")


def rotation_sets(footprint: int, source_bytes: int) -> int:
    """Buffer sets in rotation.  Together the sets cover ROTATION_BYTES, and the T x H source rows
    (read once per call) of the other sets add up to at least twice the last-level cache between two
    uses of one set's rows, so that those rows come from HBM whatever cache hint a kernel's loads carry.
    At most MAX_SETS: decode-sized sources stay below that bound (and their loads are nontemporal)."""
    by_total = -(-ROTATION_BYTES // max(footprint, 1))
    by_source = 1 + -(-2 * LLC_BYTES // max(source_bytes, 1))
    return max(3, min(MAX_SETS, max(by_total, by_source)))


class Workload:
    """Device buffers for one configuration: `nsets` rotating sets, each allocated once."""

    def __init__(self, cfg, torch, moe, W, nsets=None):
        import numpy as np

        self.cfg, self.torch, self.moe = cfg, torch, moe
        d = W.make_inputs(cfg)
        self.shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
        x16 = torch.from_numpy(d["x"].view(np.int16))
        first = self._new_set(x16, d)
        # one pass to learn the receive row count, then expert outputs ~ N(0,1) in receive-row order
        moe.run_layout(self.shape, first["idx"], first["lay"])
        moe.run_dispatch(self.shape, cfg.dispatch_dtype, first["x"], first["idx"], first["w"], first["lay"],
                         first["disp"])
        torch.cuda.synchronize()
        self.n_recv = int(first["disp"]["num_recv"].item())
        y16 = torch.from_numpy(W.draw_expert_outputs(W.y_stream(cfg), self.n_recv, cfg.hidden).view(np.int16))
        first["y"] = y16.cuda().view(torch.bfloat16)
        self.bytes = algorithmic_bytes(cfg, self.n_recv)
        footprint = sum(t.numel() * t.element_size() for t in self._tensors(first))
        if nsets is None:
            nsets = rotation_sets(footprint, first["x"].numel() * first["x"].element_size())
        self.sets = [first]
        for _ in range(nsets - 1):
            s = self._new_set(x16, d)
            s["y"] = y16.cuda().view(torch.bfloat16)
            self.sets.append(s)
        self.footprint = footprint

    def _new_set(self, x16, d):
        torch, moe, cfg = self.torch, self.moe, self.cfg
        return {
            "x": x16.cuda().view(torch.bfloat16),
            "idx": torch.from_numpy(d["topk_idx"]).cuda(),
            "w": torch.from_numpy(d["topk_w"]).cuda(),
            "lay": moe.alloc_layout(self.shape),
            "disp": moe.alloc_dispatch(self.shape, cfg.dispatch_dtype),
            "out": torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda"),
        }

    def _tensors(self, s):
        for v in s.values():
            if isinstance(v, dict):
                yield from (t for t in v.values() if isinstance(t, self.torch.Tensor))
            elif isinstance(v, self.torch.Tensor):
                yield v

    def op(self, name, s):
        self.op_on(name, s, None)

    def op_on(self, name, s, stream):
        moe, cfg = self.moe, self.cfg
        if name == "layout+dispatch":  # the end-to-end send side
            self.op_on("layout", s, stream)
            self.op_on("dispatch", s, stream)
            return
        calls = s.setdefault("calls", {})  # each op's arguments checked once per buffer set
        if name not in calls:
            if name == "layout":
                calls[name] = moe.prepare_layout(self.shape, s["idx"], s["lay"])
            elif name == FUSED:  # the same outputs from one call (one kernel for small batches)
                calls[name] = moe.prepare_layout_dispatch(self.shape, cfg.dispatch_dtype, s["x"], s["idx"], s["w"],
                                                          s["lay"], s["disp"])
            elif name == "dispatch":
                calls[name] = moe.prepare_dispatch(self.shape, cfg.dispatch_dtype, s["x"], s["idx"], s["w"],
                                                   s["lay"], s["disp"])
            else:
                calls[name] = moe.prepare_combine(self.shape, s["y"], s["idx"], s["w"], s["disp"]["send_row"],
                                                  s["out"])
        calls[name](stream)

    def time_steps(self, steps: int, warmup: int):
        torch = self.torch
        n = len(self.sets)
        for i in range(warmup):
            for name in OPS:
                self.op(name, self.sets[i % n])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            s, e = self.sets[i % n], ev[i]
            e[0].record()
            self.op("layout", s)
            e[1].record()
            self.op("dispatch", s)
            e[2].record()
            self.op("combine", s)
            e[3].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {name: [e[i].elapsed_time(e[i + 1]) for e in ev] for i, name in enumerate(OPS)}
        return wall, per

    def time_steps_graph(self, steps: int, warmup: int, ops=OPS, per_graph: int = STEPS_PER_GRAPH) -> float:
        """Wall seconds for exactly `steps` steps (`ops` in order), replayed from graphs that each hold
        `per_graph` consecutive steps on the buffer sets in rotation (one more graph holds the
        remainder).  Several steps per replay keep the host's per-replay cost from setting the pace
        of short (decode-sized) steps."""
        torch = self.torch
        stream = torch.cuda.Stream()
        n = len(self.sets)

        def capture(count):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    for name in ops:
                        self.op(name, self.sets[i % n])
            return g

        with torch.cuda.stream(stream):
            for s in self.sets:
                for name in ops:  # warm-up on the capture stream
                    self.op(name, s)
            torch.cuda.synchronize()
            full = capture(per_graph)
            tail = capture(steps % per_graph) if steps % per_graph else None
        for _ in range(-(-warmup // per_graph)):
            full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // per_graph):
            full.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del full, tail
        return wall

    def time_kernels(self, reps: int = 20, repeats: int = 5, ops=OPS) -> dict:
        """Per-op µs from HIP graphs of `reps` back-to-back launches over the rotating sets."""
        torch = self.torch
        stream = torch.cuda.Stream()
        out = {}
        for name in ops:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                for s in self.sets:
                    self.op(name, s)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=stream):
                    for r in range(reps):
                        self.op(name, self.sets[r % len(self.sets)])
            g.replay()
            torch.cuda.synchronize()
            times = []
            for _ in range(repeats):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    e0.record()
                    g.replay()
                    e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / reps)
            out[name] = sorted(times)[len(times) // 2]
            del g
        return out


class LlWorkload(Workload):
    """The low-latency path: dispatch into per-expert buffers [E, T, H], combine from them."""

    OPS_LL = ("dispatch_ll", "combine_ll")

    def __init__(self, cfg, torch, moe, W, nsets=None):
        import numpy as np

        self.cfg, self.torch, self.moe = cfg, torch, moe
        d = W.make_inputs(cfg)
        self.shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
        x16 = torch.from_numpy(d["x"].view(np.int16))
        first = self._new_ll_set(x16, d)
        moe.run_dispatch_ll(self.shape, cfg.dispatch_dtype, first["x"], first["idx"], first["ll"])
        torch.cuda.synchronize()
        count = first["ll"]["recv_count"].cpu().numpy()
        self.n_recv = int(count.sum())
        # expert outputs ~ N(0,1) in the rows that were received, zeros elsewhere
        rows = W.draw_expert_outputs(W.y_stream(cfg), self.n_recv, cfg.hidden)
        y = np.zeros((cfg.num_experts, cfg.num_tokens, cfg.hidden), np.uint16)
        i = 0
        for e, n in enumerate(count):
            y[e, :n] = rows[i:i + n]
            i += n
        y16 = torch.from_numpy(y.view(np.int16))
        first["y"] = y16.cuda().view(torch.bfloat16)
        self.bytes = ll_algorithmic_bytes(cfg, self.n_recv)
        footprint = sum(t.numel() * t.element_size() for t in self._tensors(first))
        if nsets is None:
            nsets = rotation_sets(footprint, first["x"].numel() * first["x"].element_size())
        self.sets = [first]
        for _ in range(nsets - 1):
            s_ = self._new_ll_set(x16, d)
            s_["y"] = y16.cuda().view(torch.bfloat16)
            self.sets.append(s_)
        self.footprint = footprint

    def _new_ll_set(self, x16, d):
        torch, moe, cfg = self.torch, self.moe, self.cfg
        return {
            "x": x16.cuda().view(torch.bfloat16),
            "idx": torch.from_numpy(d["topk_idx"]).cuda(),
            "w": torch.from_numpy(d["topk_w"]).cuda(),
            "ll": moe.alloc_dispatch_ll(self.shape, cfg.dispatch_dtype),
            "out": torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda"),
        }

    def op(self, name, s):
        if name == "dispatch_ll":
            self.moe.run_dispatch_ll(self.shape, self.cfg.dispatch_dtype, s["x"], s["idx"], s["ll"])
        else:
            self.moe.moe_combine_ll(self.shape, s["y"], s["idx"], s["w"], s["ll"]["slot_pos"], s["out"])

    def time_ll(self, steps: int, warmup: int):
        torch = self.torch
        n = len(self.sets)
        for i in range(warmup):
            for name in self.OPS_LL:
                self.op(name, self.sets[i % n])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            s_, e = self.sets[i % n], ev[i]
            e[0].record()
            self.op("dispatch_ll", s_)
            e[1].record()
            self.op("combine_ll", s_)
            e[2].record()
        torch.cuda.synchronize()
        per = {name: [e[i].elapsed_time(e[i + 1]) for e in ev] for i, name in enumerate(self.OPS_LL)}
        kern = self.time_kernels(ops=self.OPS_LL)
        return {o: op_summary(self.bytes[o], per[o], kern[o]) for o in self.OPS_LL}


class BwdWorkload(Workload):
    """Backward of combine and dispatch on the rank layout of the forward workload."""

    OPS_BWD = ("combine_backward", "dispatch_backward")

    def __init__(self, cfg, torch, moe, W, nsets=None):
        super().__init__(cfg, torch, moe, W, nsets)
        import numpy as np

        n, T, H, k = self.n_recv, cfg.num_tokens, cfg.hidden, cfg.num_topk
        g16 = torch.from_numpy(W.draw_expert_outputs(np.random.default_rng(11), T, H).view(np.int16))
        grw = torch.from_numpy(np.random.default_rng(12).standard_normal((n, k)).astype(np.float32))
        for s_ in self.sets:
            self.op("layout", s_)
            self.op("dispatch", s_)
            s_["g"] = g16.cuda().view(torch.bfloat16)
            s_["grad_y"] = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
            s_["grad_w"] = torch.empty((T, k), dtype=torch.float32, device="cuda")
            s_["grad_recv_w"] = grw.cuda()
            s_["grad_x"] = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            s_["grad_topk_w"] = torch.empty((T, k), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.bytes = bwd_algorithmic_bytes(cfg, n)

    def op(self, name, s):
        if name == "combine_backward":
            self.moe.moe_combine_backward(self.shape, s["g"], s["y"], s["idx"], s["w"], s["disp"]["send_row"],
                                          s["grad_y"], s["grad_w"])
        elif name == "dispatch_backward":
            self.moe.moe_dispatch_backward(self.shape, s["y"], s["idx"], s["disp"]["send_row"], s["grad_x"],
                                           s["grad_recv_w"], s["grad_topk_w"])
        else:
            super().op(name, s)

    def time_bwd(self, steps: int, warmup: int):
        torch = self.torch
        n = len(self.sets)
        for i in range(warmup):
            for name in self.OPS_BWD:
                self.op(name, self.sets[i % n])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            s_, e = self.sets[i % n], ev[i]
            e[0].record()
            self.op("combine_backward", s_)
            e[1].record()
            self.op("dispatch_backward", s_)
            e[2].record()
        torch.cuda.synchronize()
        per = {name: [e[i].elapsed_time(e[i + 1]) for e in ev] for i, name in enumerate(self.OPS_BWD)}
        kern = self.time_kernels(ops=self.OPS_BWD)
        return {o: op_summary(self.bytes[o], per[o], kern[o]) for o in self.OPS_BWD}


def graph_us(torch, fn, reps: int = 20, repeats: int = 5) -> float:
    """Median µs per call of `fn(r)` from a HIP graph of `reps` back-to-back calls."""
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for r in range(reps):
            fn(r)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for r in range(reps):
                fn(r)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return sorted(times)[len(times) // 2]


def router_timing(cfg, torch, moe, W, nsets: int = 8) -> dict:
    """Top-k gating fused with the layout against the layout alone on the same ids, and against a
    plain torch gate (topk + softmax/sigmoid, no group limit) for context.  Also the whole send side
    from logits: moe_route_dispatch (one kernel up to 1024 tokens) against moe_route_layout followed
    by moe_dispatch."""
    import numpy as np
    grouped = cfg.routing == "group_limited"
    gate = "sigmoid" if cfg.routing == "sigmoid" else "softmax"
    G, KG = (cfg.num_groups, cfg.topk_groups) if grouped else (1, 1)
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    logits = torch.from_numpy(W.config_logits(cfg)).cuda()
    x = torch.from_numpy(W.make_inputs(cfg)["x"].view(np.int16)).view(torch.bfloat16).cuda()
    dtype = cfg.dispatch_dtype
    sets = []
    for _ in range(nsets):
        lay = moe.alloc_route(shape)
        sets.append({"logits": logits.clone(), "lay": lay, "x": x.clone(), "d": moe.alloc_dispatch(shape, dtype)})
    for s in sets:
        moe.run_route(shape, s["logits"], s["lay"], gate, G, KG)
    torch.cuda.synchronize()

    def route_dispatch(r):
        s = sets[r % nsets]
        moe.run_route_dispatch(shape, dtype, s["logits"], s["x"], s["lay"], s["d"], gate, G, KG)

    def route_then_dispatch(r):
        s = sets[r % nsets]
        moe.run_route(shape, s["logits"], s["lay"], gate, G, KG)
        moe.run_dispatch(shape, dtype, s["x"], s["lay"]["topk_idx"], s["lay"]["topk_w"], s["lay"], s["d"])

    def fused(r):
        s = sets[r % nsets]
        moe.run_route(shape, s["logits"], s["lay"], gate, G, KG)

    def layout_only(r):
        s = sets[r % nsets]
        moe.run_layout(shape, s["lay"]["topk_idx"], s["lay"])

    def torch_gate(r):
        x = sets[r % nsets]["logits"]
        v, _ = torch.topk(x, cfg.num_topk, dim=1)
        w = torch.softmax(v, dim=1) if gate == "softmax" else torch.sigmoid(v)
        if gate == "sigmoid":
            w = w / w.sum(dim=1, keepdim=True)

    T, E, k, R = cfg.num_tokens, cfg.num_experts, cfg.num_topk, cfg.num_ranks
    nbytes = T * E * 4 + T * k * 8 + T * R + T * 8
    out = {"gate": gate, "num_groups": G, "topk_groups": KG,
           "route_layout_us": round(graph_us(torch, fused), 2),
           "layout_only_us": round(graph_us(torch, layout_only), 2),
           "torch_topk_gate_us": round(graph_us(torch, torch_gate), 2),
           "algorithmic_bytes": nbytes,
           "route_dispatch_one_call_us": round(graph_us(torch, route_dispatch), 2),
           "route_then_dispatch_us": round(graph_us(torch, route_then_dispatch), 2),
           "dispatch_dtype": dtype}
    out["route_layout_GB_per_s"] = round(nbytes / (out["route_layout_us"] * 1e-6) / 1e9, 1)
    return out


def cu_sweep(wl: "Workload", torch, moe, budgets=(8, 16, 32, 64, 128, 256), reps: int = 20) -> list:
    """Dispatch and combine on streams restricted to a number of CUs (the analogue of reserving SMs)."""
    rows = []
    n = len(wl.sets)
    for cus in budgets:
        h = moe.stream_create_cu_range(0, cus)
        st = torch.cuda.ExternalStream(h)
        try:
            res = {"num_cus": cus}
            for name in ("dispatch", "combine"):
                for i in range(3):
                    wl.op_on(name, wl.sets[i % n], h)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                st.synchronize()
                e0.record(st)
                for i in range(reps):
                    wl.op_on(name, wl.sets[i % n], h)
                e1.record(st)
                st.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                res[name] = {"us": round(us, 2), "GB_per_s": round(wl.bytes[name] / (us * 1e-6) / 1e9, 1)}
            rows.append(res)
            log(f"cu budget {cus}: {res}")
        finally:
            st.synchronize()
            moe.stream_destroy(h)
    return rows


def overlap(wl: "Workload", torch, moe, comm_cus: int, reps: int = 10) -> dict:
    """Exchange (dispatch + combine) on `comm_cus` CUs while a bf16 GEMM runs on the other CUs."""
    total = torch.cuda.get_device_properties(0).multi_processor_count
    hc = moe.stream_create_cu_range(0, comm_cus)
    hg = moe.stream_create_cu_range(comm_cus, total - comm_cus)
    sc, sg = torch.cuda.ExternalStream(hc), torch.cuda.ExternalStream(hg)
    M = 8192
    a = torch.randn(M, M, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(M, M, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(M, M, device="cuda", dtype=torch.bfloat16)
    n = len(wl.sets)

    def comm():
        for i in range(reps):
            wl.op_on("dispatch", wl.sets[i % n], hc)
            wl.op_on("combine", wl.sets[i % n], hc)

    def gemm():
        with torch.cuda.stream(sg):
            for _ in range(reps):
                torch.matmul(a, b, out=c)

    def timed(fns):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for f in fns:
            f()
        sc.synchronize()
        sg.synchronize()
        return (time.perf_counter() - t0) * 1e3

    try:
        timed([gemm, comm])  # warm-up
        t_gemm, t_comm, t_both = timed([gemm]), timed([comm]), timed([gemm, comm])
    finally:
        torch.cuda.synchronize()
        moe.stream_destroy(hc)
        moe.stream_destroy(hg)
    res = {"comm_cus": comm_cus, "gemm_cus": total - comm_cus, "reps": reps, "gemm": f"bf16 {M}x{M}x{M}",
           "ms_gemm_alone": round(t_gemm, 3), "ms_exchange_alone": round(t_comm, 3), "ms_both": round(t_both, 3),
           "overlap_gain": round((t_gemm + t_comm) / t_both, 3)}
    log(f"overlap: {res}")
    return res


def op_summary(bytes_: int, times_ms, kernel_us: float) -> dict:
    import numpy as np

    t = np.asarray(times_ms)
    mean_us = float(t.mean() * 1e3)
    timed = kernel_us == kernel_us  # NaN: per-launch timing skipped
    return {
        "us_mean": round(mean_us, 3),
        "us_median": round(float(np.median(t) * 1e3), 3),
        "us_p10": round(float(np.percentile(t, 10) * 1e3), 3),
        "us_p90": round(float(np.percentile(t, 90) * 1e3), 3),
        "us_kernel": round(kernel_us, 3) if timed else None,
        "bytes": int(bytes_),
        "GB_per_s": round(bytes_ / (mean_us * 1e-6) / 1e9, 2),
        "GB_per_s_kernel": round(bytes_ / (kernel_us * 1e-6) / 1e9, 2) if timed else None,
        "frac_of_hbm_peak": round(bytes_ / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown cpu"


def _numpy_threads() -> dict:
    """Threads the oracle's numpy can use: element-wise ufuncs run on the calling thread; the BLAS
    pool (not used by the oracle) is reported for completeness."""
    out = {"elementwise": 1}
    try:
        from threadpoolctl import threadpool_info
        out["blas"] = sum(int(p.get("num_threads", 0)) for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:  # threadpoolctl missing or unable to inspect: the element-wise figure stands
        pass
    return out


def cpu_ops(cfg, W, repeats: int = 3) -> dict:
    """The numpy oracle, as it stands, per op on the full workload: µs per call (median of `repeats`)
    and GB/s with the GPU's algorithmic byte formulas.  layout = counts and mask; dispatch = receive
    rows, their metadata and payload (bf16 copy or FP8 quantisation); combine = the weighted sum."""
    import numpy as np

    from oracle import moe_oracle as O

    d = W.make_inputs(cfg)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    E, R = cfg.num_experts, cfg.num_ranks
    _, _, mask0 = O.get_dispatch_layout(idx, E, R)
    y = W.draw_expert_outputs(W.y_stream(cfg), int(mask0.sum()), cfg.hidden)
    state = {}

    def layout():
        state["mask"] = O.get_dispatch_layout(idx, E, R)[2]

    def dispatch():
        _, send_row, n = O.assign_slots(state["mask"])
        src, _, _ = O.dispatch_metadata(idx, w, E, R, send_row, n)
        if cfg.dispatch_dtype == "bf16":
            O.dispatch_rows_bf16(x, src)
        else:
            O.dispatch_rows_fp8(x, src)
        state["send_row"], state["n"] = send_row, n

    def combine():
        O.combine(y, idx, w, state["send_row"], E, R)

    out = {}
    for name, fn in (("layout", layout), ("dispatch", dispatch), ("combine", combine)):
        times = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        out[name] = float(np.median(times))
    b = algorithmic_bytes(cfg, state["n"])
    return {op: {"us": round(out[op] * 1e6, 1), "GB_per_s": round(b[op] / out[op] / 1e9, 3)} for op in out}


def cpu_baseline(cfg, W, secondary=None) -> dict:
    """The numpy oracle timed on the host cores: per op on the main workload (and on `secondary`),
    with `value` the whole step's algorithmic bytes over the summed per-op medians."""
    ops = cpu_ops(cfg, W)
    step_s = sum(op["us"] for op in ops.values()) * 1e-6
    d = W.make_inputs(cfg)
    from oracle import moe_oracle as O
    _, _, mask = O.get_dispatch_layout(d["topk_idx"], cfg.num_experts, cfg.num_ranks)
    b = algorithmic_bytes(cfg, int(mask.sum()))
    threads = _numpy_threads()
    out = {
        "value": round((b["layout"] + b["dispatch"] + b["combine"]) / step_s / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"full {cfg.name} workload, layout, dispatch and combine each timed as the median of 3 "
                  f"calls ({step_s:.2f} s per step); numpy element-wise work runs on one core",
        "ops": ops,
        "cpu_model": _cpu_model(),
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
        "numpy_threads": threads,
    }
    if secondary is not None:
        out["secondary"] = {"workload": secondary.name, "ops": cpu_ops(secondary, W)}
    return out


def copy_reference(torch, nbytes: int = 512 << 20, reps: int = 10) -> dict:
    """A plain 512 MB device-to-device copy in the same run: the achievable-bandwidth reference
    (read + write bytes over the copy time, median of `reps` event-timed copies)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = sorted(times)[len(times) // 2]
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * nbytes, "us": round(us, 1), "GB_per_s": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}


HBM_CEILING = os.path.join(ROOT, "hbm_ceiling")
LAUNCH_FLOOR = os.path.join(ROOT, "liblaunch_floor.so")
# The probe's mix closest to each kernel's read/write mix
CEILING_MIX = {"dispatch": "read1_write5", "combine": "read5_write1",
               "combine_backward": "read5_write5", "dispatch_backward": "read5_write1"}


def hbm_ceiling():
    """Best streaming bandwidth per read/write mix (hbm_ceiling.hip, built by build.py),
    or None when the probe is not built."""
    import subprocess

    if not os.path.exists(HBM_CEILING):
        log("hbm_ceiling is not built; skipping the streaming-bandwidth probe")
        return None
    res = subprocess.run([HBM_CEILING], capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        raise RuntimeError(f"hbm_ceiling failed ({res.returncode}): {res.stderr.strip()}")
    return json.loads(res.stdout)


def launch_floor(torch) -> dict:
    """The shortest launches (launch_floor.hip, built by build.py), timed like the ops' us_kernel:
    graphs of back-to-back launches.  `empty_us`: a one-wave kernel that does nothing;
    `load_store_us`: a one-wave kernel whose lane 0 loads one 16-byte value and stores it, the
    launches of a graph reading 64 addresses 16 MiB apart (1 GiB in all) so that consecutive
    launches touch different lines.  None when the probe is not built."""
    import ctypes

    if not os.path.exists(LAUNCH_FLOOR):
        log("launch_floor is not built; skipping the launch floor")
        return None
    lib = ctypes.CDLL(LAUNCH_FLOOR)
    lib.floor_empty.argtypes = [ctypes.c_void_p]
    lib.floor_load_store.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(64 * 16, dtype=torch.uint8, device="cuda")
    srcs = [src.data_ptr() + r * (16 << 20) for r in range(64)]
    dsts = [dst.data_ptr() + 16 * r for r in range(64)]

    def empty(r):
        if lib.floor_empty(torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("floor_empty launch failed")

    def load_store(r):
        if lib.floor_load_store(srcs[r % 64], dsts[r % 64], torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("floor_load_store launch failed")

    out = {"empty_us": round(graph_us(torch, empty), 3), "load_store_us": round(graph_us(torch, load_store, reps=64), 3)}
    del src
    return out


def copy_calibration(torch, nbytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain device copy of known size, so counter runs can scale FETCH/WRITE_SIZE."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--secondary", default="decode", help="second workload measured in the same run ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true", help="skip the graph-replay per-op timing")
    ap.add_argument("--copy-calibration", action="store_true", help="also run a 1 GiB device copy (counter runs)")
    ap.add_argument("--no-hbm-ceiling", action="store_true", help="skip the streaming-bandwidth probe")
    ap.add_argument("--no-launch-floor", action="store_true", help="skip the shortest-launch timing")
    ap.add_argument("--no-low-latency", action="store_true", help="skip the per-expert path on decode")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward ops on the main workload")
    ap.add_argument("--no-router", action="store_true", help="skip the fused router + layout timing")
    ap.add_argument("--cu-sweep", action="store_true", help="dispatch/combine on streams limited to 8..256 CUs")
    ap.add_argument("--overlap", type=int, default=0, metavar="CUS",
                    help="exchange on CUS CUs concurrently with a bf16 GEMM on the rest")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: logical EP ranks are segments of one GPU's HBM; "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import combine_get_dispatch_07_amd as moe
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    def measure(name: str) -> dict:
        cfg = W.CONFIG_BY_NAME[name]
        log(f"building workload {name}")
        wl = Workload(cfg, torch, moe, W)
        log(f"timing {args.steps} steps of {name} (N_recv={wl.n_recv}, {len(wl.sets)} rotating sets "
            f"of {wl.footprint / 2**20:.0f} MiB)")
        wall_eager, per = wl.time_steps(args.steps, args.warmup)
        wall = wl.time_steps_graph(args.steps, args.warmup)
        both = "layout+dispatch"
        kern = ({o: float("nan") for o in OPS + (both,)} if args.no_kernel_timing
                else wl.time_kernels(ops=OPS + (both,)))
        per[both] = [a + b for a, b in zip(per["layout"], per["dispatch"])]  # event to event, both ops
        ops = {o: op_summary(wl.bytes[o], per[o], kern[o]) for o in OPS}
        ops[both] = op_summary(wl.bytes["layout"] + wl.bytes["dispatch"], per[both], kern[both])
        # the send side as one call, and the step built on it (graph replays)
        wall_one = wl.time_steps_graph(args.steps, args.warmup, ops=(FUSED, "combine"))
        if not args.no_kernel_timing:
            us = wl.time_kernels(ops=(FUSED,))[FUSED]
            b_send = wl.bytes["layout"] + wl.bytes["dispatch"]
            ops[FUSED] = {"us_kernel": round(us, 3), "bytes": int(b_send),
                          "GB_per_s_kernel": round(b_send / (us * 1e-6) / 1e9, 2)}
        res = {"cfg": cfg, "n_recv": wl.n_recv, "ops": ops, "ms_per_step": wall * 1e3 / args.steps,
               "ms_per_step_eager": wall_eager * 1e3 / args.steps,
               "ms_per_step_one_call": wall_one * 1e3 / args.steps,
               "step_bytes": sum(wl.bytes.values()), "sets": len(wl.sets)}
        if name == args.workload and args.cu_sweep:
            res["cu_budget"] = cu_sweep(wl, torch, moe)
        if name == args.workload and args.overlap:
            res["overlap"] = overlap(wl, torch, moe, args.overlap)
        del wl
        torch.cuda.empty_cache()
        if name == args.workload and not args.no_backward:
            log(f"timing the backward ops on {name}")
            bw = BwdWorkload(cfg, torch, moe, W)
            res["backward"] = {"ops": bw.time_bwd(args.steps, args.warmup)}
            del bw
            torch.cuda.empty_cache()
        if not args.no_router:
            log(f"timing the fused router + layout on {name}")
            res["router"] = router_timing(cfg, torch, moe, W)
            torch.cuda.empty_cache()
        if cfg.name == "decode" and not args.no_low_latency:
            log(f"timing the low-latency path on {name}")
            ll = LlWorkload(cfg, torch, moe, W)
            res["low_latency"] = {"n_rows": ll.n_recv, "ops": ll.time_ll(args.steps, args.warmup)}
            del ll
            torch.cuda.empty_cache()
        return res

    main_res = measure(args.workload)
    cfg = main_res["cfg"]
    sec = measure(args.secondary) if args.secondary and args.secondary != args.workload else None
    if args.copy_calibration:
        copy_calibration(torch)

    ops = main_res["ops"]
    # Per launch: HIP events on the launch stream around graphs of back-to-back launches of the kernel
    # (us_kernel), which is what a kernel trace reports as its duration.  The eager per-op events also
    # hold each launch's gap (~2 us); their rate is reported beside it, and stands in for the
    # per-launch one when that timing is skipped (--no-kernel-timing).
    timed = not args.no_kernel_timing
    dom = max(("dispatch", "combine"), key=lambda o: ops[o]["us_kernel"] if timed else ops[o]["us_mean"])
    achieved = ops[dom]["GB_per_s_kernel"] if timed else ops[dom]["GB_per_s"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload, dom),
                "algorithmic_bytes_per_launch": ops[dom]["bytes"], "launch_us": ops[dom]["us_kernel"],
                "achieved_eager_events": ops[dom]["GB_per_s"]}

    log("timing a 512 MB device copy (achievable-bandwidth reference)")
    copy_ref = copy_reference(torch)
    floor = None
    if not args.no_launch_floor:
        log("timing the shortest launches (launch floor)")
        floor = launch_floor(torch)
    ceiling = None
    if not args.no_hbm_ceiling:
        log("measuring streaming bandwidth per read/write mix")
        ceiling = hbm_ceiling()
    if ceiling is not None:  # the same read/write mix as the dominant kernel, streamed without a gather
        best = ceiling[CEILING_MIX[dom]]["GB_per_s"]
        roofline["streaming_ceiling_same_mix"] = {"mix": CEILING_MIX[dom], "GB_per_s": best,
                                                  "frac": round(achieved / best, 4)}
        for name, op in main_res.get("backward", {}).get("ops", {}).items():
            rate = op.get("GB_per_s_kernel") or op["GB_per_s"]
            best = ceiling.get(CEILING_MIX[name], {}).get("GB_per_s")
            if best:
                op["streaming_ceiling_same_mix"] = {"mix": CEILING_MIX[name], "GB_per_s": best,
                                                    "frac": round(rate / best, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(cfg, W, sec["cfg"] if sec is not None else None)

    value = main_res["step_bytes"] / (main_res["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "ms_per_step_eager": round(main_res["ms_per_step_eager"], 4),
        "ms_per_step_one_call": round(main_res["ms_per_step_one_call"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dispatch_dtype == "bf16" else "fp8-e4m3/bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.num_tokens} H={cfg.hidden} E={cfg.num_experts} "
                               f"top-{cfg.num_topk} R={cfg.num_ranks} {cfg.dispatch_dtype} dispatch, "
                               f"fp32-accumulate combine to bf16",
                   "num_tokens": cfg.num_tokens, "hidden": cfg.hidden, "num_experts": cfg.num_experts,
                   "num_topk": cfg.num_topk, "num_ranks": cfg.num_ranks, "n_recv": main_res["n_recv"],
                   "rotating_sets": main_res["sets"]},
        "ops": ops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "copy_reference": copy_ref,
        "hbm_ceiling": ceiling,
        "launch_floor": floor,
    }
    if sec is not None:
        c2 = sec["cfg"]
        line["secondary"] = {"workload": f"{c2.name}: T={c2.num_tokens} H={c2.hidden} E={c2.num_experts} "
                                         f"top-{c2.num_topk} R={c2.num_ranks} {c2.dispatch_dtype} dispatch",
                             "n_recv": sec["n_recv"], "ms_per_step": round(sec["ms_per_step"], 4),
                             "ms_per_step_eager": round(sec["ms_per_step_eager"], 4),
                             "ms_per_step_one_call": round(sec["ms_per_step_one_call"], 4),
                             "ops": sec["ops"]}
        for key in ("low_latency", "router"):
            if key in sec:
                line["secondary"][key] = sec[key]
    if "low_latency" in main_res:
        line["low_latency"] = main_res["low_latency"]
    for key in ("backward", "cu_budget", "overlap", "router"):
        if key in main_res:
            line[key] = main_res[key]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
