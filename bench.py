"""Benchmark of the Echo int4 all-reduce on one MI355X.

Workload: a 1 GiB bfloat16 message per rank (536,870,912 elements, viewed as
[131072, 4096]), P = 8 emulated ranks whose partials are N(0,1) with 0.01 %
outliers x100, the same 8 partials for every call, group 32, compensation on.
A step is one whole all-reduce (stage-1 quantize of all ranks, owner
sum/correct/requantize, decode), inputs resident in HBM.  Sequence: reset,
W warm-up calls, reset, K timed back-to-back calls.

Prints one JSON line.  value = bf16-equivalent GB/s = P * 2 * N / t_step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Echo reduce GB/s (bf16-equiv payload) + % HBM peak, 1 GB msg, P=8 emulated"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published
# sources of the three kernels whose HBM traffic the counter runs measure
KERNEL_SOURCES = ["error_compensated_bit_echo_amd/csrc/echo_kernels.hip",
                  "error_compensated_bit_echo_amd/csrc/echo_owner.h",
                  "error_compensated_bit_echo_amd/csrc/echo_internal.h",
                  "error_compensated_bit_echo_amd/csrc/echo_div7.h",
                  "error_compensated_bit_echo_amd/csrc/echo_quant.h",
                  "error_compensated_bit_echo_amd/csrc/echo_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
COPY_FLOATS = 1 << 29  # 2 GiB of fp32 for the copy kernel
KERNEL_KEYS = {"stage1": "echo_quant_pack_k", "owner": "echo_owner_k", "decode": "echo_unpack_k"}


def algorithmic_bytes(P: int, N: int, b_in: int, compensate: bool, group: int = 32,
                      sender_feedback: bool = False, state_bf16: bool = False,
                      out_bf16: bool = False, own_exact: bool = False) -> dict:
    """Bytes each stage must move per call (reads + writes of HBM)."""
    pl = 0.5 + 4.0 / group                     # payload bytes per element: codes + scales
    sent = (P - 1) * N if own_exact else P * N  # rank elements that pass stage 1
    k1 = sent * (b_in + pl)                    # read partials; write codes + scales
    if sender_feedback:                        # read and write those elements' stage-1 errors
        k1 += sent * (4.0 if state_bf16 else 8.0)  # (bfloat16 with the bf16 state)
    if own_exact:                              # P - 1 payload segments and the owner's own partial
        k2 = N * (pl * (P - 1) + b_in + pl)
    else:                                      # read P payload segments; write broadcast payload
        k2 = N * (pl * P + pl)
    if compensate:
        k2 += (8.0 if state_bf16 else 16.0) * N  # read and write m_fast, m_slow
    k3 = N * (pl + (2.0 if out_bf16 else 4.0))  # read broadcast payload; write the output
    return {"stage1": k1, "owner": k2, "decode": k3}


def workload_tag(comp: bool, group: int = 32, sender_feedback: bool = False,
                 state_bf16: bool = False, out_bf16: bool = False, own_exact: bool = False) -> str:
    tag = f"1GiB-P8-bf16-{'comp' if comp else 'nocomp'}"
    if group != 32:
        tag += f"-g{group}"
    return tag + ("-sfb" if sender_feedback else "") + ("-sb16" if state_bf16 else "") + \
        ("-obf16" if out_bf16 else "") + ("-own" if own_exact else "")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when the kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def ingest_counters(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs of this
    benchmark (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is
    scaled by the factor that makes it read the known bytes of the copy kernel
    (COPY_FLOATS fp32 read and written): on gfx950 FETCH_SIZE reads half the
    true bytes and WRITE_SIZE reads them exactly."""
    import csv
    import statistics

    def per_kernel(path):
        vals = {k: [] for k in KERNEL_KEYS}
        copy = []
        with open(path) as f:
            for r in csv.DictReader(f):
                name, v = r["Kernel_Name"], float(r["Counter_Value"])
                for k, key in KERNEL_KEYS.items():
                    if key in name:
                        vals[k].append(v)
                if "MulFunctor<float>" in name:
                    copy.append(v)
        # the copy kernel's dispatches are the big MulFunctor ones (the synthetic
        # input generator also multiplies a few outliers)
        copy = [v for v in copy if v >= 0.5 * max(copy)] if copy else []
        if not copy:
            raise SystemExit(f"{path}: no copy-kernel dispatch found")
        return {k: statistics.median(v) for k, v in vals.items() if v}, statistics.median(copy)

    fk, fcopy = per_kernel(fetch_csv)
    wk, wcopy = per_kernel(write_csv)
    known = COPY_FLOATS * 4
    f_scale, w_scale = known / (fcopy * 1024), known / (wcopy * 1024)
    rec = {
        "kernel_source_sha": kernel_source_hash(),
        "workload": workload,
        "command": command,
        "copy_kernel": {"bytes_read": known, "bytes_written": known, "fetch_kib": fcopy,
                        "write_kib": wcopy, "fetch_scale": round(f_scale, 5),
                        "write_scale": round(w_scale, 5)},
        "kernels": {},
    }
    for k in KERNEL_KEYS:
        if k in fk and k in wk:
            rd, wr = fk[k] * 1024 * f_scale, wk[k] * 1024 * w_scale
            rec["kernels"][k] = {"fetch_kib": fk[k], "write_kib": wk[k], "read_bytes": int(rd),
                                 "write_bytes": int(wr), "bytes_per_launch": int(rd + wr)}
    return rec


# ---------------------------------------------------------------------------
# the other workloads: latency, effective bandwidth and accuracy reports
# ---------------------------------------------------------------------------
# the reports of --config; the first four are the synthetic workloads of the same name
REPORTS = ("tiny", "prefill", "decode", "training", "tp", "groups", "variants", "gemm")
CACHE_BYTES = 256 * 2**20  # MI355X Infinity Cache


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


GRAPH_CALLS = 32  # back-to-back calls captured in one graph for the latency figure


def _graph_us(E, torch, parts, out, st, direction, reps):
    """GPU time per call of GRAPH_CALLS back-to-back echo_reduce calls captured
    in one graph (launch overhead of the host language out of the way), over
    ``reps`` replays."""
    E.echo_reduce(parts, out, st, direction)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(GRAPH_CALLS):
            E.echo_reduce(parts, out, st, direction)
    torch.cuda.synchronize()
    g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 / GRAPH_CALLS for a, b in ev], g


def _stage_graph_us(E, torch, parts, out, st, reps) -> dict:
    """Median GPU time per launch of each stage alone (stage 1, owner, decode),
    GRAPH_CALLS back-to-back launches captured in one graph, over ``reps``
    replays (forward direction)."""
    stages = {"stage1": lambda: E.echo_stage1(parts, st, E.ECHO_FWD),
              "owner": lambda: E.echo_owner(st, E.ECHO_FWD),
              "decode": lambda: E.echo_decode(out, st)}
    res = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_CALLS):
                fn()
        torch.cuda.synchronize()
        g.replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        res[name] = round(_pct([a.elapsed_time(b) * 1e3 / GRAPH_CALLS for a, b in ev], 0.5), 2)
    return res


def _wall_us(E, torch, parts, out, st, direction, reps):
    """Host-clock time per call of ``reps`` back-to-back eager calls."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        E.echo_reduce(parts, out, st, direction)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / reps


def stream_report(name, E, synth, torch, dev, group: int = 32) -> dict:
    """tiny / prefill / training: the configuration's calls on fresh partials,
    each call's output added to a residual stream h (fp32) next to the exact
    stream h* = sum of all partials (float64); compensation on and off."""
    import numpy as np

    c = synth.WORKLOADS[name]
    P, N, dtype = c["P"], synth.numel(name), c["dtype"]
    dirs = (0, 1) if name == "training" else (0,)
    b_in = 4 if dtype == "f32" else 2

    def parts_for(d, t):
        if dtype == "f32":
            raw, _ = synth.host_partials(name, d, t)
            return [torch.from_numpy(np.ascontiguousarray(raw[r])).to(dev) for r in range(P)]
        return synth.device_partials(name, d, t, device=dev)

    st = {m: E.echo_init_state(E.EchoConfig.make(P, N, dtype, compensate=(m == "on"), group=group),
                               device=dev)
          for m in ("on", "off")}
    out = torch.empty(N, dtype=torch.float32, device=dev)
    h = {(m, d): torch.zeros(N, dtype=torch.float32, device=dev) for m in st for d in dirs}
    hx = {d: torch.zeros(N, dtype=torch.float64, device=dev) for d in dirs}
    evs = []
    for t in range(c["calls"]):
        for d in dirs:
            parts = parts_for(d, t)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            E.echo_reduce(parts, out, st["on"], d)
            b.record()
            evs.append((a, b))
            h[("on", d)] += out
            E.echo_reduce(parts, out, st["off"], d)
            h[("off", d)] += out
            for p in parts:
                hx[d] += p.double()
    torch.cuda.synchronize()
    eager = [a.elapsed_time(b) * 1e3 for a, b in evs]
    err = {}
    for d in dirs:
        ref = hx[d]
        scale = ref.pow(2).mean().sqrt().item()
        for m in ("on", "off"):
            e = (h[(m, d)].double() - ref).pow(2).mean().sqrt().item()
            err[f"{'fwd' if d == 0 else 'bwd'}_{m}"] = {"rms_err": e, "rel_rms_err": e / scale}
    wall = _wall_us(E, torch, parts, out, st["on"], dirs[-1], 20)
    gst = E.echo_init_state(E.EchoConfig.make(P, N, dtype, group=group), device=dev)
    gout = torch.empty_like(out)
    graph, _ = _graph_us(E, torch, parts, gout, gst, dirs[-1], 20)
    pl = 0.5 + 4.0 / group
    alg = N * (P * (b_in + pl) + pl * (P + 2) + 4 + 16)
    ws_bytes = N * (P * b_in + (P + 1) * pl + 8 + 4)
    med = _pct(graph, 0.5)
    return {
        "config": name if group == 32 else f"{name}-g{group}", "group": group,
        "P": P, "numel_per_rank": N, "input_dtype": dtype,
        "payload_bytes_per_element": pl,
        "calls": c["calls"] * len(dirs), "alg_bytes_per_call": int(alg),
        # distinct bytes a call touches: partials, the P + 1 payloads, one direction's
        # two fp32 estimates, the fp32 output
        "working_set_bytes": int(ws_bytes),
        "cache_resident": bool(ws_bytes <= CACHE_BYTES),
        # calls of 96 MB to 1.2 GB (the library's cache-policy measure) run stage 1 and
        # the owner with plain caching, so the owner reads much of the stage-1 payload
        # from the last-level cache: their algorithmic GB/s is not an HBM rate
        "payload_through_cache": bool(96e6 <= N * (P * (b_in + 0.625) + 21.25) <= 1200e6),
        "us_per_call": {"eager_events_median": round(_pct(eager, 0.5), 2),
                        "eager_events_p90": round(_pct(eager, 0.9), 2),
                        "eager_wall_back_to_back": round(wall, 2),
                        "graph_32_calls_median": round(med, 2),
                        "graph_32_calls_p90": round(_pct(graph, 0.9), 2)},
        "GBps_alg_graph": round(alg / (med * 1e-6) / 1e9, 1),
        "residual_stream_error_after_all_calls": err,
    }


def decode_report(E, synth, torch, dev) -> dict:
    """The decode-shaped chain: 128 layers, P = 8, [64, 4096] bf16 partials from
    a pre-norm random map per layer; four chains from the same h_0 (Echo with
    compensation, without, with compensation and sender feedback, and an exact
    all-reduce in float64).  Per-call
    latency of echo_reduce: eager from Python (includes the binding's host
    time), eager from plain C through the C ABI, one captured call replayed per
    layer, and 32 back-to-back calls in one graph (the library's own per-call
    time)."""
    c = synth.DECODE_CHAIN
    P, rows, hd, L = 8, c["rows"], c["hidden"], c["layers"]
    N = rows * hd
    h0 = synth.decode_h0(dev)
    modes = ("on", "off", "sfb")
    h = {m: h0.clone() for m in modes}
    hx = h0.double()
    st = {m: E.echo_init_state(E.EchoConfig.make(P, N, "bf16", compensate=(m != "off"),
                                                 sender_feedback=(m == "sfb")), device=dev)
          for m in modes}
    out = torch.empty(N, dtype=torch.float32, device=dev)
    # graph path: fixed partial buffers, its own state fed the same partials as "on"
    pbuf = [torch.empty(N, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    gst = E.echo_init_state(E.EchoConfig.make(P, N, "bf16"), device=dev)
    gout = torch.empty_like(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.echo_reduce(pbuf, gout, gst, E.ECHO_FWD)
    torch.cuda.synchronize()
    E.echo_reset(gst, 3)
    ev_e, ev_g, rel = [], [], {}
    graph_equal = True
    for layer in range(1, L + 1):
        w = synth.decode_weight(layer, dev)
        for m in modes:
            parts = synth.decode_partials(h[m], w, P)
            if m == "on":
                for b, p in zip(pbuf, parts):
                    b.copy_(p)
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record()
                g.replay()
                a1.record()
                ev_g.append((a0, a1))
                b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                b0.record()
                E.echo_reduce(parts, out, st[m], E.ECHO_FWD)
                b1.record()
                ev_e.append((b0, b1))
                graph_equal &= bool(torch.equal(out, gout))
            else:
                E.echo_reduce(parts, out, st[m], E.ECHO_FWD)
            h[m] += out.view(rows, hd)
        px = synth.decode_partials(hx.float(), w, P)
        hx += sum(p.double() for p in px).view(rows, hd)
        if layer & (layer - 1) == 0 or layer == L:
            scale = hx.pow(2).mean().sqrt().item()
            rel[str(layer)] = {m: round((h[m].double() - hx).pow(2).mean().sqrt().item() / scale, 8)
                               for m in modes}
    torch.cuda.synchronize()
    eager = [a.elapsed_time(b) * 1e3 for a, b in ev_e]
    graph = [a.elapsed_time(b) * 1e3 for a, b in ev_g]
    g32, _ = _graph_us(E, torch, pbuf, gout, gst, E.ECHO_FWD, 20)
    stage_us = _stage_graph_us(E, torch, pbuf, gout, gst, 20)
    alg = N * (P * 3.25 + 21.25)
    return {
        "config": "decode", "P": P, "numel_per_rank": N, "input_dtype": "bf16", "layers": L,
        "alg_bytes_per_call": int(alg), "cache_resident": True,
        "us_per_call": {"eager_events_median": round(_pct(eager, 0.5), 2),
                        "eager_events_p90": round(_pct(eager, 0.9), 2),
                        "graph_1_call_median": round(_pct(graph, 0.5), 2),
                        "graph_1_call_p90": round(_pct(graph, 0.9), 2),
                        "graph_32_calls_median": round(_pct(g32, 0.5), 2),
                        "graph_32_calls_p90": round(_pct(g32, 0.9), 2)},
        "GBps_alg_graph_32_calls": round(alg / (_pct(g32, 0.5) * 1e-6) / 1e9, 1),
        # each stage alone, 32 back-to-back launches in one graph: their sum against the call's
        # per-call time says whether the three-kernel call spends time between its kernels
        "us_per_launch_graph_32_launches_of_one_stage": stage_us,
        "us_per_call_minus_sum_of_stages": round(_pct(g32, 0.5) - sum(stage_us.values()), 2),
        "graph_replay_equals_eager_every_layer": graph_equal,
        "rel_rms_err_vs_exact_allreduce_chain": rel,
        "c_abi_eager": c_abi_latency(P, N),
    }


def c_abi_latency(P: int, N: int, calls: int = 2000) -> dict:
    """Per-call latency of eager echo_reduce calls made from plain C through the
    C ABI (tests/c_client/echo_c_latency, built with the library): device time of
    back-to-back calls, the host's time to issue one call, and one call followed
    by a stream synchronize.  Run as a child process on the same GPU."""
    import subprocess

    from error_compensated_bit_echo_amd import build as b
    if not os.path.exists(b.C_LATENCY):
        raise RuntimeError(f"{b.C_LATENCY} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    r = subprocess.run([b.C_LATENCY, str(P), str(N), str(calls)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        raise RuntimeError(f"echo_c_latency failed ({r.returncode}): {r.stderr.strip()}")
    res = json.loads(r.stdout.strip().splitlines()[-1])
    return {"us_per_call": {k: res[k] for k in ("device_us", "enqueue_us", "roundtrip_us")}, "calls": calls,
            "note": "plain C, default stream, the same partials every call"}


def tp_report(torch, dev) -> dict:
    """Echo inside a tensor-parallel MLP stack (8 layers, P = 4, 2048 tokens,
    hidden 4096, ffn 16384): one training step (forward + backward, 8 Echo calls
    per direction) with Echo, Echo without compensation and exact all-reduces
    (fp32 products), and with Echo and the row-parallel products in bfloat16 on
    libecho's kernel, written out or with stage 1 fused into them; errors of the
    loss and the gradients against the exact fp32 step, and step times (median
    of three steps after a warm-up step)."""
    from error_compensated_bit_echo_amd import tp

    T, H, F, P, L = 2048, 4096, 16384, 4, 8
    model = tp.TPMLPStack(L, H, F, P, seed=21, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(22)
    x0 = torch.randn(T, H, generator=g, device=dev)
    target = torch.randn(T, H, generator=g, device=dev)
    res, ms = {}, {}

    def timed(m, group):
        """One warm-up step, then the median of three timed steps."""
        tp.train_step(m, group, x0, target)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            out = tp.train_step(m, group, x0, target)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return out, sorted(times)[1]

    for mode in ("exact", "echo", "echo_off"):
        res[mode], ms[mode] = timed(model, tp.EchoGroup(P, T * H, mode=mode, device=dev))
    # variants of the all-reduce (fp32 products)
    variants = {"echo_sender_feedback": {"sender_feedback": True},
                "echo_own_exact": {"own_exact": True},
                "echo_sender_feedback_own_exact_bf16_state": {"sender_feedback": True, "own_exact": True,
                                                              "state_bf16": True}}
    for name, kw in variants.items():
        res[name], ms[name] = timed(model, tp.EchoGroup(P, T * H, mode="echo", device=dev, **kw))

    # the row-parallel product in bfloat16 on libecho's kernel, written out then
    # reduced, or with stage 1 in its epilogue (bit-identical results)
    for prod in ("bf16", "bf16_fused"):
        m2 = tp.TPMLPStack(L, H, F, P, seed=21, device=dev, product=prod)
        res["echo_" + prod], ms["echo_" + prod] = timed(m2, tp.EchoGroup(P, T * H, mode="echo", device=dev))
        if prod == "bf16_fused":  # the fused product with sender feedback and bf16 state
            name = "echo_bf16_fused_sender_feedback_bf16_state"
            res[name], ms[name] = timed(m2, tp.EchoGroup(P, T * H, mode="echo", device=dev, sender_feedback=True,
                                                         state_bf16=True))
        del m2

    def rel(x, y):
        return float((x - y).float().norm() / y.float().norm())

    errs = {}
    for mode in ("echo", "echo_off", *variants, "echo_bf16", "echo_bf16_fused",
                 "echo_bf16_fused_sender_feedback_bf16_state"):
        loss, dx, dw = res[mode]
        errs[mode] = {"loss_rel_err": abs(float(loss - res["exact"][0])) / float(res["exact"][0]),
                      "dx0_rel_err": rel(dx, res["exact"][1]),
                      "dW_rel_err_mean": sum(rel(p, q) for p, q in zip(dw, res["exact"][2])) / len(dw),
                      "dW_rel_err_max": max(rel(p, q) for p, q in zip(dw, res["exact"][2]))}
    return {"config": "tp", "P": P, "layers": L, "tokens": T, "hidden": H, "ffn": F,
            "echo_calls_per_step": {"fwd": L, "bwd": L},
            "step_ms": {k: round(v, 3) for k, v in ms.items()},
            "errors_vs_exact_allreduce": errs}


def sender_report(E, synth, torch, dev) -> dict:
    """The variants on the prefill workload (P = 4, bf16 [2048, 4096], 72 calls,
    fresh partials per call): error of the residual stream h_T = sum of all
    outputs against the exact stream, by call count T, for compensation on/off,
    sender feedback on/off, fp32 or bf16 state, fp32 or bf16 output and the
    owner adding its own partial exactly or not; per-call latency of each."""
    c = synth.WORKLOADS["prefill"]
    P, N, calls = c["P"], synth.numel("prefill"), c["calls"]
    # (compensate, sender feedback, bf16 state, bf16 output, own partial exact)
    combos = [(True, False, False, False, False), (False, False, False, False, False),
              (True, True, False, False, False), (False, True, False, False, False),
              (True, False, True, False, False), (True, True, True, False, False),
              (True, False, False, True, False), (False, False, False, True, False),
              (True, False, False, False, True), (True, True, False, False, True)]

    def name(k):
        return (f"comp_{'on' if k[0] else 'off'}_sfb_{'on' if k[1] else 'off'}"
                f"_state_{'bf16' if k[2] else 'fp32'}_out_{'bf16' if k[3] else 'fp32'}"
                + ("_own_exact" if k[4] else ""))

    def make(k):
        return E.echo_init_state(E.EchoConfig.make(P, N, "bf16", compensate=k[0], sender_feedback=k[1],
                                                   state_bf16=k[2], out_bf16=k[3], own_exact=k[4]),
                                 device=dev)

    def out_for(k):
        return torch.empty(N, dtype=torch.bfloat16 if k[3] else torch.float32, device=dev)

    modes = {k: make(k) for k in combos}
    outs = {k: out_for(k) for k in combos}
    h = {k: torch.zeros(N, dtype=torch.float64, device=dev) for k in modes}
    hx = torch.zeros(N, dtype=torch.float64, device=dev)
    err = {name(k): {} for k in modes}
    for t in range(calls):
        parts = synth.device_partials("prefill", 0, t, device=dev)
        for k, st in modes.items():
            E.echo_reduce(parts, outs[k], st, E.ECHO_FWD)
            h[k] += outs[k].double()
        for p in parts:
            hx += p.double()
        T = t + 1
        if T & (T - 1) == 0 or T == calls:
            for k in modes:
                err[name(k)][str(T)] = (h[k] - hx).pow(2).mean().sqrt().item()
    lat = {}
    for k in combos:
        g, _ = _graph_us(E, torch, parts, out_for(k), make(k), E.ECHO_FWD, 20)
        lat[name(k)] = round(_pct(g, 0.5), 2)
    return {"config": "variants", "P": P, "numel_per_rank": N, "calls": calls,
            "rms_err_of_accumulated_output_vs_exact_by_calls": err,
            "us_per_call_graph_32_calls": lat}


def gemm_report(E, torch, dev, weights: str = "both") -> dict:
    """Stage 1 fused into the producing product (bf16 MFMA, fp32 accumulation):
    per shape, the fused kernel against the same product written out followed
    by the stage-1 kernel, and against torch's library product (hipBLASLt)
    followed by the stage-1 kernel.  TFLOP/s against the MI355X dense bf16 peak.

    The weights are timed cold: consecutive calls rotate over enough weight sets
    (about 900 MiB, and as many transposed copies for the library) that no call
    finds its weights in the 256 MB Infinity Cache, as in a model whose layers
    each bring their own weights.  The activations stay the same.  The same
    timings with one weight set (cached after the first call) are given beside.
    torch's product gets the weights as they are given, [H, K] (transposed in the
    call): hipBLASLt was faster that way than on pre-transposed [K, H] copies
    (51.5 against 56.8 us at the prefill-like shape, 20.2 against 25.6 us at the
    decode-like one, per rank).
    `weights` ("cold", "cached" or "both") picks which of the two are timed, so
    that a profiler's kernel trace holds one kind only."""
    res = []
    # prefill-like (256 x 256 tiles), decode-like at 128 and 256 tokens (128 x 128 and 256 x 128
    # tiles), and a two-rank decode-like product (64 x 64 tiles)
    for P, M, K, H in ((4, 2048, 3072, 4096), (8, 128, 3072, 4096), (8, 256, 3072, 4096), (2, 128, 3072, 4096)):
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        set_bytes = P * H * K * 2
        nsets = max(2, -(-900 * 2 ** 20 // set_bytes))
        A = [torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16) for _ in range(P)]
        Ws = [[(torch.randn(H, K, generator=g, device=dev) / K ** 0.5).to(torch.bfloat16) for _ in range(P)]
              for _ in range(nsets)]
        out = [torch.empty(M, H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
        st = E.echo_init_state(E.EchoConfig.make(P, M * H, "bf16"), device=dev)
        flat = [o.view(-1) for o in out]

        def fused(i):
            E.echo_gemm_stage1(A, Ws[i], st)

        def ours_unfused(i):
            E.echo_gemm_bf16(A, Ws[i], out)
            E.echo_stage1(flat, st)

        def library_unfused(i):
            # the library's faster layout here: W_r as given ([H, K]), transposed in the call
            for r in range(P):
                torch.matmul(A[r], Ws[i][r].t(), out=out[r])
            E.echo_stage1(flat, st)

        def product_only(i):
            E.echo_gemm_bf16(A, Ws[i], out)

        # sustained load first (clocks ramp up over the first tens of milliseconds),
        # then five interleaved batches of 20 calls per variant; the median batch counts
        fns = (("fused", fused), ("ours_then_stage1", ours_unfused),
               ("library_then_stage1", library_unfused), ("ours_product_only", product_only))
        for i in range(100):
            product_only(i % nsets)
            library_unfused(i % nsets)
        torch.cuda.synchronize()
        reps = 20
        t = {}
        for mode in ("cold", "cached") if weights == "both" else (weights,):
            batches = {name: [] for name, _ in fns}
            for _ in range(5):
                for name, fn in fns:
                    fn(0)  # the cached timing's first call brings set 0 in
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for i in range(reps):
                        fn((i + 1) % nsets if mode == "cold" else 0)
                    b.record()
                    torch.cuda.synchronize()
                    batches[name].append(a.elapsed_time(b) * 1e3 / reps)
            t[mode] = {name: sorted(v)[len(v) // 2] for name, v in batches.items()}
        # what the timed fused kernel wrote must be stage 1 of the written-out product
        ref = E.echo_init_state(E.EchoConfig.make(P, M * H, "bf16"), device=dev)
        E.echo_gemm_stage1(A, Ws[0], st)
        E.echo_gemm_bf16(A, Ws[0], out)
        E.echo_stage1(flat, ref)
        vf, vr = E.echo_debug_views(st), E.echo_debug_views(ref)
        torch.cuda.synchronize()
        same = torch.equal(vf["codes1"], vr["codes1"]) and torch.equal(vf["scales1"], vr["scales1"])
        if not same:
            raise RuntimeError(f"fused payload differs from stage 1 of the written-out product at "
                               f"P={P} M={M} K={K} H={H}")
        flop = 2.0 * P * M * K * H
        res.append({"P": P, "M": M, "K": K, "H": H, "payload_equals_stage1_of_written_out": same,
                    "weights": f"cold: {nsets} sets of {set_bytes / 2 ** 20:.0f} MiB in rotation",
                    **({"us": {k: round(v, 2) for k, v in t["cold"].items()},
                        "TFLOPs": {k: round(flop / (v * 1e-6) / 1e12, 1) for k, v in t["cold"].items()},
                        "weight_GBps": {k: round(set_bytes / (v * 1e-6) / 1e9, 1) for k, v in t["cold"].items()}}
                       if "cold" in t else {}),
                    **({"us_weights_cached": {k: round(v, 2) for k, v in t["cached"].items()}}
                       if "cached" in t else {}),
                    "bf16_peak_TFLOPs": 2500.0,
                    **({"fused_frac_of_bf16_peak": round(flop / (t["cold"]["fused"] * 1e-6) / 1e12 / 2500.0, 3)}
                       if "cold" in t else {}),
                    "partial_bytes_not_written_or_read": 2 * 2 * P * M * H})
    return {"config": "gemm", "shapes": res, "decode_layer": decode_layer_report(E, torch, dev)}


def decode_layer_report(E, torch, dev) -> dict:
    """The decode-shaped layer's row-parallel product and its reduction: P = 8
    ranks, 64 tokens, K = 512 per rank (a 4096-wide layer split 8 ways), H = 4096.
    Our variants run as 32 calls captured in one graph, each call on its own
    weight set (1 GiB of weights in all, so every call reads its weights from
    HBM), timed over ten replays (median, us per call): fused_product = the
    product with stage 1 in its epilogue; fused_layer = that, the owner step and
    the decode (the layer's whole reduction); unfused_layer = the product written
    out, then echo_reduce; product = the product alone.  torch's product (one
    library call per rank) is not captured; it is timed, with echo_reduce, as
    eager calls from Python, beside our fused layer timed the same way.  The
    fused layer's output must equal the unfused layer's, which is checked."""
    P, M, K, H = 8, 64, 512, 4096
    sets = GRAPH_CALLS
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    A = [torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16) for _ in range(P)]
    Ws = [[(torch.randn(H, K, generator=g, device=dev) / K ** 0.5).to(torch.bfloat16) for _ in range(P)]
          for _ in range(sets)]
    st = E.echo_init_state(E.EchoConfig.make(P, M * H, "bf16"), device=dev)
    out = torch.empty(M * H, dtype=torch.float32, device=dev)
    parts = [torch.empty(M, H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    flat = [q.view(-1) for q in parts]

    def fused_product(W):
        E.echo_gemm_stage1(A, W, st)

    def fused_layer(W):
        E.echo_gemm_stage1(A, W, st)
        E.echo_owner(st, E.ECHO_FWD)
        E.echo_decode(out, st)

    def unfused_layer(W):
        E.echo_gemm_bf16(A, W, parts)
        E.echo_reduce(flat, out, st, E.ECHO_FWD)

    def product(W):
        E.echo_gemm_bf16(A, W, parts)

    def library_layer(W):
        for r in range(P):
            torch.matmul(A[r], W[r].t(), out=parts[r])
        E.echo_reduce(flat, out, st, E.ECHO_FWD)

    # the fused layer's output equals the unfused layer's (fresh state each)
    E.echo_reset(st, 3)
    fused_layer(Ws[0])
    ref = out.clone()
    E.echo_reset(st, 3)
    unfused_layer(Ws[0])
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref))
    if not same:
        raise RuntimeError("the fused decode layer's output differs from the unfused layer's")

    def median_us(run, calls, reps=10):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / calls)
        return round(sorted(ts)[len(ts) // 2], 2)

    graph_us = {}
    for name, fn in (("fused_product", fused_product), ("fused_layer", fused_layer),
                     ("unfused_layer", unfused_layer), ("product", product)):
        fn(Ws[0])
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(sets):
                fn(Ws[i])
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        graph_us[name] = median_us(gr.replay, sets)

    def eager(fn, ws):
        def run():
            for i in range(sets):
                fn(ws[i])
        run()
        torch.cuda.synchronize()
        return median_us(run, sets)

    eager_us = {"fused_layer": eager(fused_layer, Ws), "library_then_echo_reduce": eager(library_layer, Ws)}
    return {"P": P, "M": M, "K": K, "H": H, "weights": f"cold: {sets} sets of {P * H * K * 2 / 2 ** 20:.0f} MiB",
            "fused_layer_equals_unfused_layer": same, "us_per_call_graph_32": graph_us,
            "weight_GBps_fused_product": round(P * H * K * 2 / (graph_us["fused_product"] * 1e-6) / 1e9, 1),
            "us_per_call_eager": eager_us}


def trace_gaps(trace_csv: str, kernels_per_call: int = 3, calls_per_replay: int = GRAPH_CALLS) -> dict:
    """Per-call kernel time against the gaps between kernels, from a rocprofv3
    kernel trace of this benchmark: the library's dispatches are split into runs
    that follow one another with no host gap (over 20 us), and the runs made of
    whole graph replays (calls_per_replay calls of kernels_per_call kernels) are
    summarised per call: the span from the first kernel's start to the last one's
    end, the summed kernel durations, and the rest, the time between kernels."""
    import csv
    import statistics

    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if any(k in name for k in ("echo_quant_pack_k", "echo_owner_k", "echo_unpack")):
                kind = "stage1" if "quant_pack" in name else ("owner" if "owner" in name else "decode")
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind))
    rows.sort()
    runs, cur = [], []
    for r in rows:
        if cur and r[0] - cur[-1][1] > 20_000:  # ns
            runs.append(cur)
            cur = []
        cur.append(r)
    if cur:
        runs.append(cur)
    per_replay = kernels_per_call * calls_per_replay
    span, busy, dur, gap_after = [], [], {}, {}
    for run in runs:
        if len(run) < per_replay or len(run) % per_replay:
            continue
        calls = len(run) // kernels_per_call
        span.append((run[-1][1] - run[0][0]) / calls / 1e3)
        busy.append(sum(e - s for s, e, _ in run) / calls / 1e3)
        for i, (s, e, k) in enumerate(run):
            dur.setdefault(k, []).append((e - s) / 1e3)
            if i + 1 < len(run):
                gap_after.setdefault(k, []).append((run[i + 1][0] - e) / 1e3)
    if not span:
        raise SystemExit(f"{trace_csv}: no run of whole {calls_per_replay}-call graph replays found")
    med = statistics.median
    return {"runs": len(span), "calls_per_run": [len(r) // kernels_per_call for r in runs
                                                  if len(r) >= per_replay and len(r) % per_replay == 0][:4],
            "us_per_call_span_median": round(med(span), 3),
            "us_per_call_kernels_median": round(med(busy), 3),
            "us_per_call_between_kernels_median": round(med(span) - med(busy), 3),
            "kernel_us_median": {k: round(med(v), 3) for k, v in dur.items()},
            "gap_us_after_kernel_median": {k: round(med(v), 3) for k, v in gap_after.items()}}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def gpu_first_call_window(E, torch, parts, st, out, n: int) -> dict:
    """Reset the state, run one call and copy back what it left in the first n
    elements: both payloads, the output and the forward estimates (fresh state,
    so the oracle can replay exactly this call on the same window)."""
    E.echo_reset(st, 3)
    E.echo_reduce(parts, out, st, E.ECHO_FWD)
    v = E.echo_debug_views(st, E.ECHO_FWD)
    torch.cuda.synchronize()
    G = st.cfg.group
    return {"codes1": v["codes1"][:, :n // 2].cpu().numpy(), "scales1": v["scales1"][:, :n // G].cpu().numpy(),
            "codes2": v["codes2"][:n // 2].cpu().numpy(), "scales2": v["scales2"][:n // G].cpu().numpy(),
            "out": out[:n].float().cpu().numpy(), "m_fast": v["m_fast"][:n].float().cpu().numpy(),
            "m_slow": v["m_slow"][:n].float().cpu().numpy()}


def _parity_check(g: dict, o: dict, st, compensate: bool) -> dict:
    """The GPU's first call on the sample window against the oracle's: codes and
    scales of both stages bit-exact; out and the estimates within 1e-5 of the
    group's broadcast scale (also counted where not bit-identical)."""
    import numpy as np
    exact = all(np.array_equal(g[k].view(np.uint8), np.ascontiguousarray(o[k]).view(np.uint8))
                for k in ("codes1", "scales1", "codes2", "scales2"))
    s2 = np.repeat(o["scales2"].astype(np.float64), g["out"].size // max(o["scales2"].size, 1))
    pairs = [("out", o["out"])]
    if compensate:
        pairs += [("m_fast", st.m_fast[0]), ("m_slow", st.m_slow[0])]
    worst, differ = 0.0, 0
    for k, want in pairs:
        d = np.abs(g[k].astype(np.float64) - want.astype(np.float64))
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(s2 > 0, d / s2, np.where(d > 0, np.inf, 0.0))
        worst = max(worst, float(rel.max()) if rel.size else 0.0)
        differ += int(np.count_nonzero(g[k] != want))
    return {"elements_per_rank": int(g["out"].size), "codes_and_scales_bit_exact": bool(exact),
            "max_err_over_group_scale": worst, "floats_not_bit_identical": differ,
            "pass": bool(exact and worst <= 1e-5)}


def cpu_baseline(parts, n_sample: int, gpu_window=None, **variant) -> dict:
    """The CPU oracle, as it stands, timed on one call over a bounded sample:
    the first ``n_sample`` elements of each of the benchmark's own partials
    (``variant``: the oracle's switches of the benchmarked configuration).
    Then the same oracle run by a pool of threads, one call each over
    independent group-aligned windows of twice that sample (numpy releases the
    interpreter lock inside its array loops; windows are exact because groups
    and compensator elements are independent).  ``gpu_window``: what the
    GPU's first call from a fresh state left in the same sample window, checked
    against the timed oracle call."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from oracle import echo_oracle as eo

    P = len(parts)
    vals = np.stack([p[:n_sample].float().cpu().numpy() for p in parts])
    st = eo.OracleState(n_sample)
    t0 = time.perf_counter()
    o = eo.echo_call(vals, st, eo.FWD, **variant)
    dt = time.perf_counter() - t0
    del vals
    parity = None
    if gpu_window is not None:
        parity = _parity_check(gpu_window, o, st, variant.get("compensate", True))
    del o

    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    nthr = max(1, min(16, ncpu))
    win = (2 * n_sample) // nthr // 128 * 128
    wins = [np.stack([p[i * win:(i + 1) * win].float().cpu().numpy() for p in parts]) for i in range(nthr)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(lambda w: eo.echo_call(w, eo.OracleState(win), eo.FWD, **variant), wins))
    dt_par = time.perf_counter() - t0
    del wins
    what = ', '.join(f'{k}={v}' for k, v in variant.items()) or 'compensation on'
    return {
        "value": round(P * 2 * n_sample / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"one call, P={P} x the first {n_sample} elements of each rank's partial "
                  f"({n_sample / 536870912:.4g} of the 1 GiB message), {what}, fresh state; {dt:.2f} s; numpy "
                  f"elementwise ops on one core ({_cpu_model()}, os.cpu_count()={os.cpu_count()}, "
                  f"affinity {ncpu})",
        "threads": {
            "value": round(P * 2 * win * nthr / dt_par / 1e9, 4),
            "unit": "GB/s",
            "cores": nthr,
            "sample": f"{nthr} threads, one oracle call each on a window of {win} elements per rank "
                      f"(the first {win * nthr} elements), {what}; {dt_par:.2f} s",
        },
        "parity_check": parity,
    }


def make_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-comp", action="store_true", help="plain two-rounding int4 all-reduce")
    ap.add_argument("--group", type=int, default=32, choices=(32, 64, 128),
                    help="elements per scale (32; 64 and 128 are variants)")
    ap.add_argument("--sender-feedback", action="store_true",
                    help="variant: every rank feeds its stage-1 rounding error into its next call")
    ap.add_argument("--bf16-state", action="store_true",
                    help="variant: the carried state (both estimates and, with sender feedback, the "
                         "ranks' stage-1 errors) stored in bfloat16")
    ap.add_argument("--out-bf16", action="store_true",
                    help="variant: bfloat16 output, the owner's error measured against it")
    ap.add_argument("--own-exact", action="store_true",
                    help="variant: each owner adds its own partial exactly (not quantized)")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26,
                    help="elements per rank in the CPU oracle's timed sample")
    ap.add_argument("--skip-cpu", action="store_true", help="leave out the CPU oracle leg")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_counters.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of this benchmark, then exit")
    ap.add_argument("--counter-command", default="", help="command recorded with --ingest-counters")
    ap.add_argument("--trace-gaps", metavar="KERNEL_TRACE_CSV",
                    help="split the per-call time of the graph replays in a rocprofv3 kernel trace of this "
                         "benchmark into kernel time and time between kernels, then exit")
    ap.add_argument("--gemm-weights", choices=("cold", "cached", "both"), default="both",
                    help="with --config gemm: time the products with cold weights (rotating over sets "
                         "larger than the Infinity Cache), cached weights (one set), or both")
    ap.add_argument("--config", choices=sorted(REPORTS) + ["all"],
                    help="instead of the 1 GiB headline, report latency, bandwidth and accuracy of "
                         "another workload (one JSON line each)")
    return ap


def main():
    args = make_parser().parse_args()

    if args.ingest_counters:
        rec = ingest_counters(*args.ingest_counters,
                              workload=workload_tag(not args.no_comp, args.group, args.sender_feedback,
                                                    args.bf16_state, args.out_bf16, args.own_exact),
                              command=args.counter_command)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return

    if args.trace_gaps:
        print(json.dumps(trace_gaps(args.trace_gaps)))
        return

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); the P ranks "
              "are emulated as P partial buffers in one GPU's HBM.", file=sys.stderr)
        sys.exit(2)

    import torch
    import error_compensated_bit_echo_amd as E
    from error_compensated_bit_echo_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config:
        names = ["tiny", "prefill", "decode", "training", "tp", "groups", "variants", "gemm"] \
            if args.config == "all" \
            else [args.config]
        for name in names:
            print(f"# config {name}", file=sys.stderr, flush=True)
            if name == "groups":
                # the group-size variants on the prefill workload: bytes against accuracy
                for G in (32, 64, 128):
                    print(json.dumps(stream_report("prefill", E, synth, torch, dev, group=G)), flush=True)
                    torch.cuda.empty_cache()
                continue
            if name == "decode":
                rep = decode_report(E, synth, torch, dev)
            elif name == "gemm":
                rep = gemm_report(E, torch, dev, args.gemm_weights)
            elif name == "variants":
                rep = sender_report(E, synth, torch, dev)
            elif name == "tp":
                rep = tp_report(torch, dev)
            else:
                rep = stream_report(name, E, synth, torch, dev)
            print(json.dumps(rep), flush=True)
            torch.cuda.empty_cache()
        return
    msg = "headline_1GiB"
    c = synth.WORKLOADS[msg]
    P, N = c["P"], synth.numel(msg)
    comp = not args.no_comp
    print(f"# generating {P} x {N} bf16 partials on the device", file=sys.stderr, flush=True)
    parts = synth.device_partials(msg, 0, 0, device=dev)
    G = args.group
    SFB, SB16, OBF, OWN = args.sender_feedback, args.bf16_state, args.out_bf16, args.own_exact
    cfg = E.EchoConfig.make(P, N, "bf16", compensate=comp, group=G, sender_feedback=SFB,
                            state_bf16=SB16, out_bf16=OBF, own_exact=OWN)
    st = E.echo_init_state(cfg, device=dev)
    out = torch.empty(N, dtype=torch.bfloat16 if OBF else torch.float32, device=dev)
    torch.cuda.synchronize()

    # warm-up, then a fresh state for the timed calls
    for _ in range(args.warmup):
        E.echo_reduce(parts, out, st, E.ECHO_FWD)
    E.echo_reset(st, 3)
    torch.cuda.synchronize()
    print(f"# warm-up done ({args.warmup} calls)", file=sys.stderr, flush=True)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        e = ev[k]
        e[0].record()
        E.echo_stage1(parts, st)
        e[1].record()
        E.echo_owner(st, E.ECHO_FWD, partials=parts if OWN else None)
        e[2].record()
        E.echo_decode(out, st)
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    kern_ms = {
        "stage1": sum(e[0].elapsed_time(e[1]) for e in ev) / K,
        "owner": sum(e[1].elapsed_time(e[2]) for e in ev) / K,
        "decode": sum(e[2].elapsed_time(e[3]) for e in ev) / K,
    }
    call_ms = sorted(e[0].elapsed_time(e[3]) for e in ev)  # HIP events around each whole call
    gpu_ms_step = sum(call_ms) / K
    print(f"# timed {K} calls: {ms_step:.3f} ms/step wall, {gpu_ms_step:.3f} ms/step events",
          file=sys.stderr, flush=True)

    alg = algorithmic_bytes(P, N, 2, comp, G, SFB, SB16, OBF, OWN)
    total_alg = sum(alg.values())
    kernels = {}
    for k, ms in kern_ms.items():
        kernels[k] = {"ms": round(ms, 4), "alg_bytes": int(alg[k]),
                      "GBps": round(alg[k] / (ms * 1e-3) / 1e9, 1),
                      "frac": round(alg[k] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    dom = max(kern_ms, key=kern_ms.get)
    achieved = alg[dom] / (kern_ms[dom] * 1e-3) / 1e9
    workload = workload_tag(comp, G, SFB, SB16, OBF, OWN)
    traffic = measured_traffic(dom, workload)

    # a plain streaming copy kernel of 2 GiB (torch's elementwise x*1, read 2 GiB,
    # write 2 GiB): achievable-bandwidth context, and the known-size kernel whose
    # rocprofv3 FETCH_SIZE / WRITE_SIZE calibrate the counters (see --ingest-counters)
    src = torch.ones(COPY_FLOATS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    wire = E.echo_wire_bytes(st)
    value = P * 2 * N / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "1 GiB bf16 message per rank (536,870,912 elements), P=8 emulated ranks, "
                        f"group {G}, absmax/7 fp32 scales, compensation " + ("on" if comp else "off") +
                        (", sender feedback" if SFB else "") + (", bf16 state" if SB16 else "") +
                        (", bf16 output" if OBF else "") + (", owners add their own partials exactly" if OWN else "") +
                        ", same partials every call, reset -> warm-up -> reset -> timed calls",
            "P": P, "numel_per_rank": N, "input_dtype": "bf16", "wire": "int4 codes + fp32 group scales",
            "output_dtype": "bf16" if OBF else "f32", "group": G,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "hbm_frac_whole_step": round(total_alg / (gpu_ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "hbm_GBps_whole_step": round(total_alg / (gpu_ms_step * 1e-3) / 1e9, 1),
        "call_ms_events": {"median": round(statistics.median(call_ms), 4), "min": round(call_ms[0], 4),
                           "max": round(call_ms[-1], 4)},
        "alg_bytes_per_step": int(total_alg),
        "algbw_GBps": round(2 * N / (ms_step * 1e-3) / 1e9, 2),
        "kernels": kernels,
        "copy_GBps_context": round(copy_gbps, 1),  # torch elementwise x*1, 2 GiB in + 2 GiB out
        "wire_bytes_per_rank": wire,
    }
    if not args.skip_cpu:
        print(f"# CPU oracle sample: P={P} x {args.cpu_sample}", file=sys.stderr, flush=True)
        variant = {k: v for k, v in (("compensate", comp), ("group", G), ("sender_feedback", SFB),
                                     ("state_bf16", SB16), ("out_bf16", OBF), ("own_exact", OWN))
                   if v != {"compensate": True, "group": 32}.get(k, False)}
        # the owners' own shares need the whole message's owner split, which a window lacks
        gw = None if OWN else gpu_first_call_window(E, torch, parts, st, out, args.cpu_sample)
        line["cpu_baseline"] = cpu_baseline(parts, args.cpu_sample, gpu_window=gw, **variant)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
