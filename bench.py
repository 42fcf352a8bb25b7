#!/usr/bin/env python3
"""Benchmark of the MoE routing hot path on one MI355X.

One step = the whole path over one batch already resident in HBM:
  moe_route_dispatch (routing + dispatch in one call) -> moe_combine
on the prefill batch (4096 tokens, hidden 7168 bf16, 384 experts, top-8, 48 destination ranks,
bf16 payload and output). The expert outputs combine reads are emulated once before timing
(row * (expert+1)/256), as the grouped GEMM is not part of the path.

Prints ONE JSON line: value = algorithmic HBM bytes of a step / step time (GB/s), ms_per_step =
µs per layer / 1000, per-call times from HIP events on the launch stream, the roofline of the
dominant kernel (combine), and the CPU oracle timed on the host. Two more timed loops run the same
step as route -> moe_dispatch -> combine and as route -> moe_dispatch_layout ->
moe_dispatch_pack -> combine, so the token-order packing kernel gets its own HIP-event timing.

The steps rotate over 8 buffer sets by default, so that every set's activations and logits have
left the 256 MB Infinity Cache when the set comes round again: the numbers are cold. A warm step
(one set) is reported beside them.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs/layer and achieved HBM GB/s (% of peak), 1 MI355X"
PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill.json")
HIP_SRC = os.path.join(ROOT, "combine_moe_route_03_amd", "csrc", "moe_route.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill")
    p.add_argument("--settle-seconds", type=float, default=0.3,
                   help="before the warmup steps, run the plain copy kernel this long so the GPU "
                        "reaches its steady clocks (0 disables it)")
    p.add_argument("--settle-step-seconds", type=float, default=0.04,
                   help="after the copy kernel, run the step itself this long (untimed) before "
                        "the warmup steps, so the timed steps start at the GPU's steady state "
                        "under this workload (0 disables it)")
    p.add_argument("--sets", type=int, default=8,
                   help="buffer sets used in rotation (each set is about 1 GB at prefill). With "
                        "2 sets the activations and logits of a set (65 MB at prefill) are still "
                        "in the 256 MB Infinity Cache when the set comes round again; from 6 sets "
                        "on they are not (measured: the same step time at 6 and 8 sets)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="host time budget of the CPU-oracle baseline (0 disables it)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run the 1 GiB plain copy kernel (for HBM counter calibration)")
    p.add_argument("--other-workloads", type=int, default=1,
                   help="also time the step on the other workloads (tiny, decode, decode_fp8, "
                        "skewed); 0 skips them")
    return p.parse_args()


def algorithmic_bytes(w) -> dict:
    """Bytes each kernel must move (reads + writes of its inputs and outputs, once each)."""
    T, H, E, k, N, R = w.T, w.H, w.E, w.k, w.N, w.rows
    xb = 4 if w.x_dtype == "f32" else 2
    pb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[w.payload]
    yb = 4 if w.y_dtype == "f32" else 2
    ob = 4 if w.out_dtype == "f32" else 2
    scales = R * (H // 128) * 4 if w.payload == "fp8_e4m3" else 0
    return {
        "route": T * E * 4 + R * 8,                                     # logits; ids + weights
        "layout": R * 4 + R * 8 + (2 * E + 2 * N + 2) * 4,              # ids; maps; counts
        "pack": T * H * xb + R * H * pb + scales + R * 4,               # x; rows; token_row
        "combine": R * H * yb + R * 8 + T * H * ob,                     # rows; maps+w; out
    }


class Prepared:
    """A C entry point with its ctypes arguments built once (launch cost only in the loop)."""

    def __init__(self, fn, *args):
        self.fn, self.args = fn, args

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"{self.fn.__name__} returned {st}")


def make_set(w, inp, dev, moe, torch):
    """Device buffers of one step and its four prepared launches."""
    import numpy as np
    lib = moe.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    if w.x_dtype == "bf16":
        x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp["x"]).to(dev)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    buf = moe.alloc_dispatch_out(w.T, w.H, w.E, w.k, w.N, w.payload, dev)
    ws = moe.alloc_workspace(w.T, w.E, w.k, dev)
    out = torch.empty((w.T, w.H), dtype=moe.TORCH_DTYPES[w.out_dtype], device=dev)
    struct = buf.as_struct()
    code = moe.DTYPE_CODES
    s = {"x": x, "logits": logits, "idx": idx, "w": wt, "buf": buf, "ws": ws, "out": out,
         "struct": struct}
    s["route"] = Prepared(lib.moe_route_topk, P(logits.data_ptr()), w.T, w.E, w.k,
                          P(idx.data_ptr()), P(wt.data_ptr()), stream)
    s["layout"] = Prepared(lib.moe_dispatch_layout, P(idx.data_ptr()), w.T, w.k, w.E, w.N,
                           ctypes.byref(struct), P(ws.data_ptr()), ws.numel(), stream)
    s["pack"] = Prepared(lib.moe_dispatch_pack, P(x.data_ptr()), code[w.x_dtype], w.T, w.H, w.k,
                         P(buf.token_row.data_ptr()), code[w.payload], P(buf.recv.data_ptr()),
                         P(buf.recv_scales.data_ptr() if buf.recv_scales is not None else 0),
                         stream)
    s["dispatch"] = Prepared(lib.moe_dispatch, P(x.data_ptr()), code[w.x_dtype], w.T, w.H,
                             P(idx.data_ptr()), w.k, w.E, w.N, code[w.payload],
                             ctypes.byref(struct), P(ws.data_ptr()), ws.numel(), stream)
    s["route_dispatch"] = Prepared(lib.moe_route_dispatch, P(logits.data_ptr()), P(x.data_ptr()),
                                   code[w.x_dtype], w.T, w.H, w.E, w.k, w.N, code[w.payload],
                                   P(idx.data_ptr()), P(wt.data_ptr()), ctypes.byref(struct),
                                   P(ws.data_ptr()), ws.numel(), stream)
    # one untimed pass, then the emulated expert outputs y = row * (expert+1)/256 (or identity)
    s["route"]()
    s["layout"]()
    s["pack"]()
    torch.cuda.synchronize()
    counts = buf.expert_counts.long()
    e_row = torch.repeat_interleave(torch.arange(w.E, device=dev), counts)
    if w.payload == "fp8_e4m3":
        val = buf.recv.view(torch.float8_e4m3fn).float() * \
            buf.recv_scales.repeat_interleave(128, dim=1)
    else:
        val = buf.recv.float()
    if w.experts == "scale":
        val = val * ((e_row + 1).float() / 256.0)[:, None]
    y = val.to(moe.TORCH_DTYPES[w.y_dtype]).contiguous()
    del val
    s["y"] = y
    s["combine"] = Prepared(lib.moe_combine, P(y.data_ptr()), code[w.y_dtype], w.T, w.H, w.k,
                            P(buf.token_row.data_ptr()), P(wt.data_ptr()), P(out.data_ptr()),
                            code[w.out_dtype], stream)
    return s


def copy_ceiling(torch, gib: float = 1.0, iters: int = 10):
    """GB/s of the plain 16-byte streaming copy over `gib` GiB (read + write counted)."""
    from combine_moe_route_03_amd import build as b
    lib = ctypes.CDLL(b.BENCH_LIB)
    lib.bench_stream_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p]
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):
        assert lib.bench_stream_copy16(src.data_ptr(), dst.data_ptr(), n, stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        assert lib.bench_stream_copy16(src.data_ptr(), dst.data_ptr(), n, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return {"bytes_per_launch": 2 * n, "us": ms * 1e3, "GBps": 2 * n / (ms * 1e-3) / 1e9}


def settle_clocks(torch, seconds: float) -> float:
    """Run the plain copy kernel over 256 MiB for about `seconds` of wall time, so that the timed
    loop does not start while the GPU is still raising its clocks; returns the seconds spent."""
    if seconds <= 0:
        return 0.0
    from combine_moe_route_03_amd import build as b
    lib = ctypes.CDLL(b.BENCH_LIB)
    lib.bench_stream_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p]
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            assert lib.bench_stream_copy16(src.data_ptr(), dst.data_ptr(), n, stream) == 0
        torch.cuda.synchronize()
    del src, dst
    return time.perf_counter() - t0


def settle_steps(torch, sets, phases, seconds: float) -> int:
    """After settle_clocks, run the step itself back to back over the buffer sets for about
    `seconds` (untimed), keeping the launch queue fed: the host waits only for the chunk before
    the last. Measured at prefill (8 sets, blocks of 20 steps after the copy kernel): the step
    takes 190, 190, 187, 186 us in the first four blocks and 185 us from about step 100 on; after
    150 steps of this settle the first block is already at 185 us. Without the copy kernel first,
    150 steps are not enough (195, 201, 193 us). Returns the number of steps run."""
    if seconds <= 0:
        return 0
    chunk, pending, n = 16, [], 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(chunk):
            for ph in phases:
                sets[n % len(sets)][ph]()
            n += 1
        ev = torch.cuda.Event()
        ev.record()
        pending.append(ev)
        if len(pending) > 1:
            pending.pop(0).synchronize()
    torch.cuda.synchronize()
    return n


def hbm_traffic(kernel_pattern: str):
    """Counter-measured HBM bytes per launch of the kernel whose name (template arguments
    included) matches `kernel_pattern`, from the committed profile: (name, bytes), or
    (None, None) when the kernels changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    with open(HIP_SRC, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("source_sha256"):
            return None, None
    for name, k in rec["kernels"].items():
        if re.fullmatch(kernel_pattern, name):
            return name, int(round(k["fetch_kib"] * 1024 * rec["copy_calibration"]["read_factor"]
                                   + k["write_kib"] * 1024 *
                                   rec["copy_calibration"]["write_factor"]))
    return None, None


def cpu_baseline(w, seconds: float, alg_total: int):
    """The CPU oracle, single-threaded, on the same batch: route + dispatch + combine passes
    repeated until `seconds` of work have been timed (expert emulation untimed)."""
    import oracle
    from combine_moe_route_03_amd.workloads import make_inputs
    inp = make_inputs(w)
    idx, wt = oracle.route(inp["logits"], w.k)
    d = oracle.dispatch(inp["x"], w.x_dtype, idx, w.E, w.N, w.payload)
    y = oracle.experts(d["recv"], w.payload, d["recv_scales"], d["expert_offsets"], w.experts,
                       w.y_dtype)
    del d
    busy, n = 0.0, 0
    while busy < seconds or n == 0:
        t0 = time.perf_counter()
        idx, wt = oracle.route(inp["logits"], w.k)
        d = oracle.dispatch(inp["x"], w.x_dtype, idx, w.E, w.N, w.payload)
        oracle.combine(y, w.y_dtype, d["token_row"], wt, w.out_dtype)
        busy += time.perf_counter() - t0
        n += 1
        del d
    return {"value": round(alg_total * n / busy / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} full passes of route+dispatch+combine over the {w.T}-token batch "
                      f"({busy:.1f} s, single thread)",
            "ms_per_step": round(busy / n * 1e3, 1), "host_cpus": os.cpu_count(),
            "host_cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


_PREROLL = {}


def preroll(torch):
    """Keep the GPU busy for about 20 us with the plain copy kernel (64 MiB) while the host
    enqueues the first timed launches: after a synchronize the GPU would otherwise sit idle
    between the start event and the first kernel, and that host latency (about 10 us) would be
    counted in the timed steps. Runs before the start event, outside the timed region."""
    if "lib" not in _PREROLL:
        from combine_moe_route_03_amd import build as b
        lib = ctypes.CDLL(b.BENCH_LIB)
        lib.bench_stream_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p]
        n = 64 << 20
        _PREROLL.update(lib=lib, n=n, src=torch.zeros(n, dtype=torch.uint8, device="cuda"),
                        dst=torch.empty(n, dtype=torch.uint8, device="cuda"))
    p = _PREROLL
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert p["lib"].bench_stream_copy16(p["src"].data_ptr(), p["dst"].data_ptr(), p["n"],
                                        stream) == 0


def timed(torch, sets, phases, K, per_call_events):
    """K steps of `phases` (rotating over the buffer sets) between two HIP events on the launch
    stream; with per_call_events, also an event after every call (each costs a few us of GPU
    idle, so the headline loop records none). Returns (ms per step, {phase: us} or None,
    per-step ms list or None)."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
          for _ in range(K)] if per_call_events else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    preroll(torch)
    start.record()
    for i in range(K):
        s = sets[i % len(sets)]
        if ev is None:
            for ph in phases:
                s[ph]()
        else:
            e = ev[i]
            e[0].record()
            for p, ph in enumerate(phases):
                s[ph]()
                e[p + 1].record()
    end.record()
    torch.cuda.synchronize()
    per = steps = None
    if ev is not None:
        per = {ph: sum(ev[i][p].elapsed_time(ev[i][p + 1]) for i in range(K)) / K * 1e3
               for p, ph in enumerate(phases)}
        steps = [ev[i][0].elapsed_time(ev[i][-1]) for i in range(K)]
    return start.elapsed_time(end) / K, per, steps


HEADLINE = ("route_dispatch", "combine")


def other_workloads(torch, moe, dev, names, K, n_sets, settle_s, settle_step_s):
    """The headline step on the smaller workloads (latency-bound ones are reported in us), over
    n_sets buffer sets in rotation, each after the same settle as the headline workload."""
    from combine_moe_route_03_amd.workloads import WORKLOADS, make_inputs
    res = {}
    for name in names:
        w = WORKLOADS[name]
        inp = make_inputs(w)
        sets = [make_set(w, inp, dev, moe, torch) for _ in range(n_sets)]
        settle_clocks(torch, settle_s)
        settle_steps(torch, sets, HEADLINE, settle_step_s)
        for i in range(10):
            for ph in HEADLINE:
                sets[i % n_sets][ph]()
        ms, _, _ = timed(torch, sets, HEADLINE, K, False)
        _, per, steps = timed(torch, sets, HEADLINE, K, True)
        alg = sum(algorithmic_bytes(w).values())
        res[name] = {"us_per_step": round(ms * 1e3, 2),
                     "median_evented_us": round(sorted(steps)[len(steps) // 2] * 1e3, 2),
                     "phases_us": {ph: round(v, 2) for ph, v in per.items()},
                     "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
                     "shape": f"T={w.T} H={w.H} E={w.E} k={w.k} N={w.N} {w.payload}"}
        del sets
        torch.cuda.empty_cache()
    return res


def ep_emulation(torch, moe, dev, K):
    """Expert parallelism over S = N = 8 devices emulated on this GPU, at the prefill batch spread
    512 tokens a device: every source's send, every rank's receive and return, every source's
    combine. Reports the per-call averages (per device: one of each runs on every device), the
    whole emulated step and its algorithmic bytes."""
    import ctypes
    import numpy as np
    from combine_moe_route_03_amd.workloads import EP_WORKLOADS, make_inputs
    w = EP_WORKLOADS["ep_prefill"]
    lib = moe.load()
    inp = make_inputs(w.as_workload())
    S, N, L, cap, T, H, k = w.S, w.N, w.L, w.cap, w.T, w.H, w.k
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    idx, wt = moe.moe_route_topk(logits, k)
    regions = torch.zeros((N * S * cap, H), dtype=torch.bfloat16, device=dev)
    returns = torch.zeros_like(regions)
    counts = torch.zeros((N, S, L), dtype=torch.int32, device=dev)
    rows = [torch.empty(T * k, dtype=torch.int32, device=dev) for _ in range(S)]
    ws = [moe.alloc_workspace(T, w.E, k, dev) for _ in range(S)]
    grouped = [torch.zeros((S * cap, H), dtype=torch.bfloat16, device=dev) for _ in range(N)]
    ec = [torch.empty(L, dtype=torch.int32, device=dev) for _ in range(N)]
    eo = [torch.empty(L + 1, dtype=torch.int32, device=dev) for _ in range(N)]
    gs = [torch.empty(S * cap, dtype=torch.int32, device=dev) for _ in range(N)]
    out = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(S)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P, B = ctypes.c_void_p, moe.DTYPE_CODES["bf16"]
    calls = {"send": [], "recv": [], "return": [], "combine": []}
    for s in range(S):
        calls["send"].append(Prepared(
            lib.moe_ep_send, P(x[s * T:].data_ptr()), B, T, H, P(idx[s * T:].data_ptr()), k, w.E,
            N, s, S, cap, P(regions.data_ptr()), P(counts.data_ptr()), P(rows[s].data_ptr()),
            P(ws[s].data_ptr()), ws[s].numel(), stream))
        calls["combine"].append(Prepared(
            lib.moe_ep_combine, P(returns.data_ptr()), B, T, H, k, P(rows[s].data_ptr()),
            P(wt[s * T:].data_ptr()), N * S * cap, P(out[s].data_ptr()), B, stream))
    for r in range(N):
        calls["recv"].append(Prepared(
            lib.moe_ep_recv, P(regions.data_ptr()), B, H, w.E, N, r, S, cap, P(counts.data_ptr()),
            P(grouped[r].data_ptr()), P(ec[r].data_ptr()), P(eo[r].data_ptr()),
            P(gs[r].data_ptr()), stream))
        # expert outputs: the grouped rows themselves (identity experts; the copy is the point)
        calls["return"].append(Prepared(
            lib.moe_ep_return, P(grouped[r].data_ptr()), B, H, w.E, N, S, cap,
            P(gs[r].data_ptr()), P(eo[r].data_ptr()), P(returns.data_ptr()), stream))
    order = ("send", "recv", "return", "combine")

    def step():
        for ph in order:
            for c in calls[ph]:
                c()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    tot = {ph: 0.0 for ph in order}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / K
    for _ in range(K):
        e[0].record()
        for p, ph in enumerate(order):
            for c in calls[ph]:
                c()
            e[p + 1].record()
        torch.cuda.synchronize()
        for p, ph in enumerate(order):
            tot[ph] += e[p].elapsed_time(e[p + 1])
    # combine with pre-reduction on the expert side: partial-row layout (per source), the partial
    # rows (per rank), the source-side finish; against the return + combine above
    pcap = T
    pc = torch.zeros((N, S), dtype=torch.int32, device=dev)
    prow = [torch.empty((T, N), dtype=torch.int32, device=dev) for _ in range(S)]
    prow_all = torch.empty((S * T, N), dtype=torch.int32, device=dev)
    rows_all = torch.empty(S * T * k, dtype=torch.int32, device=dev)
    partials = torch.zeros((N * S * pcap, H), dtype=torch.bfloat16, device=dev)
    rws = moe.moe_ep_reduce_workspace(S, cap, dev)
    out_red = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(S)]
    red = {"partial_rows": [], "reduce": [], "finish": []}
    for s in range(S):
        red["partial_rows"].append(Prepared(
            lib.moe_ep_partial_rows, P(idx[s * T:].data_ptr()), T, k, w.E, N, s, S, pcap,
            P(prow[s].data_ptr()), P(pc.data_ptr()), stream))
        red["finish"].append(Prepared(
            lib.moe_ep_combine_reduced, P(partials.data_ptr()), B, T, H, N, P(prow[s].data_ptr()),
            N * S * pcap, P(out_red[s].data_ptr()), B, stream))
    for r in range(N):
        red["reduce"].append(Prepared(
            lib.moe_ep_reduce, P(grouped[r].data_ptr()), B, H, w.E, N, r, S, cap,
            P(gs[r].data_ptr()), T, k, P(idx.data_ptr()), P(wt.data_ptr()),
            P(rows_all.data_ptr()), P(prow_all.data_ptr()), pcap, P(partials.data_ptr()),
            P(rws.data_ptr()), rws.numel(), stream))
    for c in red["partial_rows"]:
        c()
    torch.cuda.synchronize()
    torch.cat(prow, out=prow_all)
    torch.cat(rows, out=rows_all)
    rorder = ("partial_rows", "reduce", "finish")
    for ph in rorder:
        for c in red[ph]:
            c()
    torch.cuda.synchronize()
    rtot = {ph: 0.0 for ph in rorder}
    for _ in range(K):
        e[0].record()
        for p, ph in enumerate(rorder):
            for c in red[ph]:
                c()
            e[p + 1].record()
        torch.cuda.synchronize()
        for p, ph in enumerate(rorder):
            rtot[ph] += e[p].elapsed_time(e[p + 1])
    overlap = send_overlap(torch, calls["send"], S * T, H, dev, K)
    full_o = torch.cat(out).view(torch.int16).to(torch.int32)
    red_o = torch.cat(out_red).view(torch.int16).to(torch.int32)
    mono = lambda v: torch.where(v < 0, -(v & 0x7FFF), v)  # noqa: E731
    dist = (mono(full_o) - mono(red_o)).abs()
    rows_back = int(pc.sum().item())
    b = 2
    rows_total = S * T * k
    alg = {"send": S * (T * H * b + T * k * H * b + 8 * T * k),
           "recv": 2 * rows_total * H * b + 4 * rows_total,
           "return": 2 * rows_total * H * b + 4 * rows_total,
           "combine": S * (T * k * H * b + 8 * T * k + T * H * b)}
    per_call = {ph: round(tot[ph] / K / len(calls[ph]) * 1e3, 2) for ph in order}
    return {"workload": f"{w.name}: {S} sources x {T} tokens, hidden {H} bf16, {w.E} experts "
                        f"top-{k}, {N} ranks of {L} experts, regions of {cap} rows",
            "step_us": round(step_ms * 1e3, 1),
            "per_device_us": round(step_ms * 1e3 / S, 1),
            "per_call_us": per_call,
            "phase_GBps": {ph: round(alg[ph] / (tot[ph] / K * 1e-3) / 1e9, 1) for ph in order},
            "algorithmic_bytes": alg,
            "GBps": round(sum(alg.values()) / (step_ms * 1e-3) / 1e9, 1),
            "pre_reduced_combine": {
                "per_call_us": {ph: round(rtot[ph] / K / len(red[ph]) * 1e3, 2) for ph in rorder},
                "rows_back": rows_back, "rows_back_without": rows_total,
                "bytes_back": rows_back * H * b, "bytes_back_without": rows_total * H * b,
                "bytes_saved_frac": round(1 - rows_back / rows_total, 4),
                "vs_receiver_only_max_bf16_codes": int(dist.max().item()),
                "vs_receiver_only_frac_elements_differing": round(
                    float((dist > 0).float().mean().item()), 5)},
            "send_overlap": overlap}


def send_overlap(torch, sends, tokens, H, dev, K, inter=2048):
    """What the sender half leaves free: the S sends (main stream) beside a dense bf16 matmul of the
    same tokens on a second stream (default priority), standing in for a shared expert's first
    projection [tokens, H] x [H, inter]. Times each alone and both together, forked and joined by
    events; `hidden_us` is how much of the shorter one the overlap hides."""
    a = torch.randn((tokens, H), device=dev).to(torch.bfloat16)
    b = torch.randn((H, inter), device=dev).to(torch.bfloat16)
    c = torch.empty((tokens, inter), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def run_sends():
        for f in sends:
            f()

    def run_mm():
        with torch.cuda.stream(side):
            torch.matmul(a, b, out=c)

    def timed_loop(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fork = torch.cuda.Event()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fork.record(main)
            side.wait_event(fork)
            fn()
            main.wait_stream(side)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3

    for fn in (run_sends, run_mm):
        fn()
    torch.cuda.synchronize()
    t_send = timed_loop(run_sends)
    t_mm = timed_loop(run_mm)
    t_both = timed_loop(lambda: (run_mm(), run_sends()))
    flops = 2.0 * tokens * H * inter
    return {"sends_us": round(t_send, 1), "matmul_us": round(t_mm, 1),
            "matmul": f"[{tokens}, {H}] x [{H}, {inter}] bf16, {flops / (t_mm * 1e-6) / 1e12:.0f} "
                      f"TFLOP/s alone",
            "together_us": round(t_both, 1),
            "hidden_us": round(t_send + t_mm - t_both, 1)}


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the routing path here runs on a single MI355X "
              "(destination ranks are row ranges of one receive buffer); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from combine_moe_route_03_amd import _lib as moe
    from combine_moe_route_03_amd.workloads import WORKLOADS, make_inputs
    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        r = copy_ceiling(torch, 1.0, 5)
        print(json.dumps({"calibration_copy": r}), flush=True)
        return

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: T={w.T} H={w.H} E={w.E} k={w.k} N={w.N} "
          f"payload={w.payload} out={w.out_dtype}; {args.sets} buffer sets", file=sys.stderr,
          flush=True)
    inp = make_inputs(w)
    sets = [make_set(w, inp, dev, moe, torch) for _ in range(max(1, args.sets))]

    headline = HEADLINE
    separate = ("route", "dispatch", "combine")
    split = ("route", "layout", "pack", "combine")
    settled_s = settle_clocks(torch, args.settle_seconds)
    n_settle = settle_steps(torch, sets, headline, args.settle_step_seconds)
    for i in range(args.warmup):
        for ph in headline:
            sets[i % len(sets)][ph]()
    torch.cuda.synchronize()
    K = args.steps
    wall0 = time.perf_counter()
    ms_per_step, _, _ = timed(torch, sets, headline, K, False)   # the headline: no inner events
    wall = time.perf_counter() - wall0
    ms_evented, phase_us, steps_ev = timed(torch, sets, headline, K, True)   # per-call times
    ms_sep, sep_us, _ = timed(torch, sets, separate, K, True)    # route, dispatch as two calls
    ms_split, split_us, _ = timed(torch, sets, split, K, True)   # packing kernel on its own
    ms_warm, _, _ = timed(torch, sets[:1], headline, K, False)   # one buffer set: warm caches

    alg = algorithmic_bytes(w)
    alg_total = sum(alg.values())
    value = alg_total / (ms_per_step * 1e-3) / 1e9
    # The dominant kernel of the step is combine: the step's other long kernel, the window-ordered
    # pack inside moe_route_dispatch, finds x already read ahead by the layout launches and runs
    # shorter (83-84 us against 86-88 us at prefill in the cold kernel trace). Combine is timed over
    # K back-to-back launches of itself (two events around the loop), which is what a kernel trace
    # averages. The token-order pack of moe_dispatch_pack, which is not part of the step and reads
    # x as it packs, is timed the same way for context.
    kernel_us = {ph: timed(torch, sets, (ph,), K, False)[0] * 1e3 for ph in ("pack", "combine")}
    dominant = "combine"
    pattern = r"k_combine<.*>"
    prof_name, traffic = hbm_traffic(pattern)
    kernel_name = prof_name or {"pack": "k_pack_rows" if w.payload != "fp8_e4m3"
                                else "k_pack_rows_fp8", "combine": "k_combine"}[dominant]
    achieved = alg[dominant] / (kernel_us[dominant] * 1e-6) / 1e9
    ceiling = copy_ceiling(torch)
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step; with per-call events "
          f"{ms_evented * 1e3:.1f} us/step: " +
          ", ".join(f"{ph} {v:.1f} us" for ph, v in phase_us.items()) +
          f" | separate calls {ms_sep * 1e3:.1f} us/step: " +
          ", ".join(f"{ph} {v:.1f} us" for ph, v in sep_us.items()) +
          f" | split path {ms_split * 1e3:.1f} us/step: " +
          ", ".join(f"{ph} {v:.1f} us" for ph, v in split_us.items()) +
          f"; copy ceiling {ceiling['GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    others = ep = None
    if args.other_workloads:
        del sets
        torch.cuda.empty_cache()
        print("[bench] other workloads", file=sys.stderr, flush=True)
        others = other_workloads(torch, moe, dev,
                                 ("tiny", "decode", "decode_fp8", "skewed", "prefill_fp8"),
                                 100, max(1, args.sets), args.settle_seconds,
                                 args.settle_step_seconds)
        print("[bench] " + "; ".join(f"{n} {r['us_per_step']} us" for n, r in others.items()),
              file=sys.stderr, flush=True)
        ep = ep_emulation(torch, moe, dev, 20)
        torch.cuda.empty_cache()
        print(f"[bench] expert-parallel emulation: step {ep['step_us']} us, "
              f"per call {ep['per_call_us']}; sends beside a matmul {ep['send_overlap']}",
              file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        print(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds, alg_total)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.T} tokens, hidden {w.H} {w.x_dtype}, {w.E} experts "
                               f"top-{w.k}, {w.N} ranks, {w.payload} payload, {w.out_dtype} out",
                   "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k, "ranks": w.N,
                   "payload": w.payload, "parallelism": "single GPU",
                   "buffer_sets": max(1, args.sets)},
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "us_route_dispatch_plus_combine": round(phase_us["route_dispatch"] +
                                                phase_us["combine"], 2),
        "hbm_frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "phases_us": {ph: round(v, 2) for ph, v in phase_us.items()},
        "evented_ms_per_step": round(ms_evented, 5),
        "evented_median_us_per_step": round(sorted(steps_ev)[len(steps_ev) // 2] * 1e3, 2),
        "warm_us_per_step": round(ms_warm * 1e3, 2),
        "separate_calls": {"ms_per_step": round(ms_sep, 5),
                           "phases_us": {ph: round(v, 2) for ph, v in sep_us.items()}},
        "split_path": {"ms_per_step": round(ms_split, 5),
                       "phases_us": {ph: round(v, 2) for ph, v in split_us.items()}},
        "algorithmic_bytes": alg,
        "roofline": {"kernel": kernel_name, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg[dominant],
                     "avg_launch_us": round(kernel_us[dominant], 2)},
        "kernel_alone_us": {"combine": round(kernel_us["combine"], 2),
                            "token_order_pack": round(kernel_us["pack"], 2)},
        "copy_ceiling_GBps": round(ceiling["GBps"], 1),
        "other_workloads": others,
        "ep_emulation": ep,
        "wall_s_timed_loop": round(wall, 4),
        "clock_settle_s": round(settled_s, 3),
        "settle_steps": n_settle,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
