"""Benchmark: DeepSeekMoE layer forward (route + dispatch + SwiGLU experts +
combine + load statistics) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-sample S] [--no-extra]

Default workload: the V3-shaped prefill layer (T=8192 tokens, hidden 7168,
256 routed SwiGLU experts of width 2048 in 8 groups, keep 4 groups, top-8,
sigmoid scores with selection bias, 1 shared expert), bf16 activations and
expert weights, fp32 router.  Inputs are seeded synthetic tensors generated
directly in HBM; the timed region is K calls of moe_layer_forward with
everything already resident.

Prints one JSON line.  `value` = tokens/s of the whole layer.  `roofline`
describes the dominant kernel (the SwiGLU gate/up grouped GEMM), timed with
HIP events recorded on the launch stream around that stage in every timed
step.  `layer` gives the whole layer's MFMA fraction and the median, min and
max step time from the same events.  For the V3 prefill workload the line
also carries `decode` (T = 128) and `skew` (T = 16384, capacity 640)
objects: the same layer and weights timed in the same process.  `clocks`
is the shader clock per long launch read with GRBM_GUI_ACTIVE in the
committed profile of the workload (null when the library's device code is
not the profiled one), `environment` names the
GPU, ROCm, torch and host CPU, and `wave_placement` checks the SIMD pairing
the prefill GEMM schedule relies on.  `cpu_baseline` is the single-threaded
C oracle on a bounded sample of tokens of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


class HipEvents:
    """hipEvent_t handles from the HIP runtime (recorded by the library on
    the stream that runs the kernels)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic_work(wl, kept_rows: int) -> dict:
    """FLOP and minimum bytes of each stage, counting only what the method
    must do (kept assignments; each tensor touched once)."""
    es = 2 if wl.act_dtype == 1 else 4
    ws = 2 if wl.w_dtype == 1 else 4
    rs = 2 if wl.router_dtype == 1 else 4
    Ish = wl.n_shared * wl.I_shared
    T, H, N, I = wl.T, wl.H, wl.N, wl.I
    gate_up_flop = 2.0 * kept_rows * H * 2 * I + 2.0 * T * H * 2 * Ish
    down_flop = 2.0 * kept_rows * I * H + 2.0 * T * Ish * H
    router_flop = 2.0 * T * H * N
    return {
        "router_flop": router_flop,
        "gate_up_flop": gate_up_flop,
        "down_flop": down_flop,
        "ffn_flop": gate_up_flop + down_flop,
        "layer_flop": router_flop + gate_up_flop + down_flop,
        "x_bytes": T * H * es,
        "router_w_bytes": N * H * rs,
        "expert_w_bytes_all": N * 3 * I * H * ws + 3 * Ish * H * ws,
    }


LIB_PATH = os.path.join(ROOT, "routing_expert_ffn_sigmoid_amd", "libmoe.so")
GATE_UP_KERNEL = "ffn_pp_kernel"


def code_object_digest(kernel: str, lib_path: str = LIB_PATH):
    """sha256 (16 hex digits) of the gfx950 code object in libmoe.so that
    holds `kernel`: the device code a counter record was taken on.  The
    library's .hip_fatbin section holds one clang offload bundle per
    translation unit; each bundle lists its entries (offset, size, target
    triple)."""
    import struct
    with open(lib_path, "rb") as f:
        data = f.read()
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def section(i):
        name, _t, _f, _a, off, size = struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)
        return name, off, size

    stroff = section(shstrndx)[1]
    fatbin = None
    for i in range(shnum):
        name, off, size = section(i)
        if data[stroff + name:data.index(b"\0", stroff + name)] == b".hip_fatbin":
            fatbin = data[off:off + size]
    if fatbin is None:
        return None
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    p = fatbin.find(magic)
    while p >= 0:
        n = struct.unpack_from("<Q", fatbin, p + len(magic))[0]
        q = p + len(magic) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, q)
            triple = fatbin[q + 24:q + 24 + tlen]
            q += 24 + tlen
            co = fatbin[p + off:p + off + size]
            if triple.endswith(b"gfx950") and kernel.encode() in co:
                return hashlib.sha256(co).hexdigest()[:16]
        p = fatbin.find(magic, p + 1)
    return None


def load_record(workload: str):
    """The committed rocprofv3 record of the workload (gate/up HBM bytes per
    launch, shader clock per launch), if it was taken on the device code
    this library holds (same code object digest); else None."""
    path = os.path.join(ROOT, "profiles", f"ffn_gate_up_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    cur = code_object_digest(GATE_UP_KERNEL)
    if cur is None or rec.get("code_object_digest") != cur:
        return None
    return rec


def profiled_clocks(rec):
    """Shader clock of the workload's long launches, from its record."""
    if not rec or not rec.get("sclk_mhz"):
        return None
    return {"source": f"GRBM_GUI_ACTIVE per launch, profiles/ffn_gate_up_traffic_{rec['workload']}.json",
            "mhz": rec["sclk_mhz"]}


def cpu_baseline(wl, inp, sample: int) -> dict:
    """The C oracle (one thread) on `sample` tokens of the workload: router
    logits, routing, dispatch and the layer output of each sampled token.
    An untimed first pass finds the experts the oracle's own routing picks,
    so their weights are on the host before the timed pass."""
    import numpy as np
    import torch

    import oracle
    from routing_expert_ffn_sigmoid_amd import workloads

    def typed(t):
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.float().numpy()

    rng = np.random.default_rng(1234)
    toks = sorted(rng.choice(wl.T, size=min(sample, wl.T), replace=False).tolist())
    x = typed(inp["x"][toks])
    wg = typed(inp["w_router"])
    bias = inp["bias"].cpu().numpy() if inp["bias"] is not None else None
    fn = oracle.SIGMOID if wl.score_fn == 1 else oracle.SOFTMAX
    gcap = workloads.group_capacity_for(wl) if wl.group_capacity else 0

    def route_dispatch():
        logits = oracle.router_logits(x, wg).astype(np.float32)
        r = oracle.route(logits, bias, wl.k, wl.n_groups, wl.topk_groups, wl.group_topn, fn,
                         wl.norm_topk, wl.route_scale)
        if gcap > 0:
            d = oracle.dispatch_grouped(r["topk_idx"], r["topk_score"], wl.N, wl.n_groups, gcap)
        else:
            d = oracle.dispatch(r["topk_idx"], r["topk_score"], wl.N, wl.capacity)
        return r, d

    r0, _ = route_dispatch()
    experts = sorted(set(int(e) for e in r0["topk_idx"].ravel()))
    w13 = {e: typed(inp["w13"][e]) for e in experts}
    w2 = {e: typed(inp["w2"][e]) for e in experts}
    ws13 = typed(inp["ws13"]) if inp.get("ws13") is not None else None
    ws2 = typed(inp["ws2"]) if inp.get("ws2") is not None else None

    t0 = time.perf_counter()
    r, d = route_dispatch()
    done = 0
    for i in range(len(toks)):
        sel = [int(e) if d["inv_row"][i, j] >= 0 else None for j, e in enumerate(r["topk_idx"][i])]
        if any(e is not None and e not in w13 for e in sel):
            continue  # cannot happen: the timed routing repeats the first pass
        oracle.token_output(x[i], [w13[e] if e is not None else None for e in sel],
                            [w2[e] if e is not None else None for e in sel], r["topk_gate"][i],
                            ws13, ws2, wl.n_shared, wl.I_shared, wl.I)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(toks)} tokens of {wl.name} ({done} computed, "
                      f"{len(toks) - done} skipped): router logits, routing, dispatch and the "
                      f"layer output of each, single-threaded C, {dt:.1f} s"}


COPY_BYTES = 1 << 30


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE readings calibrate the same counters for the
    library's kernels (bytes the counters report per byte really moved)."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": COPY_BYTES}))


def _csv_rows(path_glob):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(path_glob, recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_profile(d: str, workload: str, commands: dict, steps: int):
    """Turn the raw rocprofv3 output under d (trace/, fetch/, write/,
    copy_fetch/, copy_write/) into profiles/<kernel>_<workload>.txt and the
    gate/up traffic record profiles/ffn_gate_up_traffic_<workload>.json."""
    stats = _csv_rows(os.path.join(d, "trace", "**", "*kernel_stats.csv"))
    trace = _csv_rows(os.path.join(d, "trace", "**", "*kernel_trace.csv"))
    lines = [f"# rocprofv3 summary: DeepSeekMoE layer forward, workload {workload}", "",
             f"library code object (gfx950) holding the gate/up kernel: "
             f"{code_object_digest(GATE_UP_KERNEL)}"]
    for key in ("trace", "fetch", "write", "copy_fetch", "copy_write", "clock", "tcp"):
        if key in commands:
            lines.append(f"{key}: {commands[key]}")
    lines += ["", "## kernel trace (--kernel-trace --stats), library kernels, all calls",
              f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for r in stats:
        name = r["Name"]
        if "moe::" not in name:
            continue
        short = name.replace("void ", "").split("(")[0]
        lines.append(f"{short:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.1f} "
                     f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f}")
    # the timed steps only: the last `steps` dispatches of each kernel
    per = {}
    for r in trace:
        name = r["Kernel_Name"]
        if "moe::" not in name:
            continue
        short = name.replace("void ", "").split("(")[0]
        per.setdefault(short, []).append(
            (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    # the bench line printed by the traced run itself (its HIP-event stage
    # times, taken on the same dispatches as the trace)
    line = None
    for f in sorted(__import__("glob").glob(os.path.join(d, "trace", "*.out"))):
        with open(f) as fh:
            for ln in fh:
                if ln.startswith('{"metric"'):
                    line = json.loads(ln)
    avg = {}
    lines += ["", f"## the last {steps} calls of each kernel (the timed steps)",
              f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s}"]
    for k in sorted(per, key=lambda n: -sum(t for _, t in per[n])):
        v = [t for _, t in sorted(per[k])][-steps:]
        vs = sorted(v)
        avg[k] = sum(v) / len(v)
        lines.append(f"{k:60s} {len(v):6d} {avg[k]:10.1f} {vs[len(vs) // 2]:10.1f} {vs[0]:10.1f}")
    if line is not None:
        ev = line["layer"]["stage_ms"]
        lines += ["", "## the traced run's own bench line (HIP events on the launch stream, same steps)",
                  f"ms_per_step {line['ms_per_step']}; stage averages (ms): " +
                  ", ".join(f"{k} {v}" for k, v in ev.items())]
        gu = [k for k in avg if "ffn" in k and "<" in k and "true" in k[k.find("<"):]]
        if gu:
            k = max(gu, key=lambda n: avg[n])
            lines.append(f"gate/up: trace {avg[k] / 1e3:.4f} ms vs events {ev['ffn_gate_up']:.4f} ms "
                         f"({100 * (ev['ffn_gate_up'] / (avg[k] / 1e3) - 1):+.2f} %)")

    def per_kernel(sub, counter):
        acc = {}
        for r in _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"].replace("void ", "").split("(")[0]
            acc.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel("fetch", "FETCH_SIZE")
    write = per_kernel("write", "WRITE_SIZE")
    cf = per_kernel("copy_fetch", "FETCH_SIZE")
    cw = per_kernel("copy_write", "WRITE_SIZE")
    copy_f = max(cf.values()) if cf else None
    copy_w = max(cw.values()) if cw else None
    f_scale = COPY_BYTES / (copy_f * 1024) if copy_f else None
    w_scale = COPY_BYTES / (copy_w * 1024) if copy_w else None
    lines += ["", "## HBM traffic per dispatch (FETCH_SIZE / WRITE_SIZE, KiB as read, then "
              "scaled by a 1 GiB plain copy's readings)",
              f"copy calibration: FETCH_SIZE {copy_f} KiB, WRITE_SIZE {copy_w} KiB for "
              f"{COPY_BYTES} B each way -> fetch scale {f_scale}, write scale {w_scale}",
              f"{'kernel':60s} {'fetch_KiB':>14s} {'write_KiB':>12s} {'bytes(scaled)':>16s}"]
    traffic = {}
    for k in sorted(set(fetch) | set(write)):
        if "moe::" not in k:
            continue
        fb = fetch.get(k, 0.0) * 1024 * (f_scale or 1.0)
        wb = write.get(k, 0.0) * 1024 * (w_scale or 1.0)
        traffic[k] = fb + wb
        lines.append(f"{k:60s} {fetch.get(k, 0.0):14.1f} {write.get(k, 0.0):12.1f} {fb + wb:16.4g}")
    # shader clock during each launch: GRBM_GUI_ACTIVE (GPU-busy cycles of
    # the graphics clock) over the dispatch's own duration in the same run
    clk, clk_mhz = {}, {}
    for r in _csv_rows(os.path.join(d, "clock", "**", "*counter_collection.csv")):
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE" or "moe::" not in r["Kernel_Name"]:
            continue
        k = r["Kernel_Name"].replace("void ", "").split("(")[0]
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if ns > 0:
            clk.setdefault(k, []).append((float(r["Counter_Value"]), ns))
    if clk:
        # the counter is summed over the GPU's XCDs (one graphics engine each)
        nxcc = 1
        for r in _csv_rows(os.path.join(d, "clock", "**", "*agent_info.csv")):
            if r.get("Agent_Type") == "GPU" and int(r.get("Num_Xcc", 0) or 0) > 0:
                nxcc = int(r["Num_Xcc"])
        lines += ["", "## shader clock per launch (GRBM_GUI_ACTIVE summed over the "
                  f"{nxcc} XCDs / {nxcc} / launch duration, same run; launches of a few tens of "
                  "microseconds read high: the counter also runs outside the kernel's timestamps)",
                  f"{'kernel':60s} {'launches':>8s} {'MHz':>8s}"]
        for k in sorted(clk, key=lambda n: -sum(ns for _, ns in clk[n])):
            cyc = sum(c for c, _ in clk[k])
            ns = sum(n for _, n in clk[k])
            clk_mhz[k] = round(1e3 * cyc / ns / nxcc)
            lines.append(f"{k:60s} {len(clk[k]):8d} {clk_mhz[k]:8d}")
    # vector L1 -> L2 requests of the large kernels (per-CU counters summed
    # over the CUs), with GRBM_GUI_ACTIVE of the same run for the cycles
    tcp = {}
    for r in _csv_rows(os.path.join(d, "tcp", "**", "*counter_collection.csv")):
        if "moe::" not in r["Kernel_Name"]:
            continue
        k = r["Kernel_Name"].replace("void ", "").split("(")[0]
        tcp.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if tcp:
        ncu, nxcc = 0, 1
        for r in _csv_rows(os.path.join(d, "tcp", "**", "*agent_info.csv")):
            if r.get("Agent_Type") == "GPU":
                ncu = int(r.get("Cu_Count", 0) or 0)
                nxcc = max(1, int(r.get("Num_Xcc", 1) or 1))
        lines += ["", f"## vector L1 -> L2 reads per launch ({ncu} CUs; per-CU counters summed)",
                  f"{'kernel':60s} {'reads':>12s} {'avg latency':>12s} {'pending-stall':>14s}"]
        for k in sorted(tcp, key=lambda n: -max(tcp[n].get("TCP_TCC_READ_REQ_sum", [0]))):
            c = {n: sum(v) / len(v) for n, v in tcp[k].items()}
            req = c.get("TCP_TCC_READ_REQ_sum", 0.0)
            lat = c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / req if req else 0.0
            cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / nxcc  # graphics-clock cycles of the launch
            stall = c.get("TCP_PENDING_STALL_CYCLES_sum", 0.0) / (ncu * cyc) if ncu and cyc else 0.0
            if req < 1e6:
                continue
            lines.append(f"{k:60s} {req:12.4g} {lat:10.0f} cy {100 * stall:12.1f} %")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    txt = os.path.join(ROOT, "profiles", f"layer_kernels_{workload}.txt")
    with open(txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    # gate/up launches: the ping-pong gate/up kernel, or a SwiGLU
    # instantiation (template argument `true`) of the other FFN kernels
    gate_up = [k for k in traffic if "gate_up" in k
               or ("ffn" in k and "<" in k and "true" in k[k.find("<"):])]
    if gate_up:
        k = max(gate_up, key=lambda n: avg.get(n, 0.0))
        rec = {"kernel": k, "workload": workload, "bytes_per_launch": traffic[k],
               "fetch_kib": fetch.get(k), "write_kib": write.get(k),
               "fetch_scale": f_scale, "write_scale": w_scale,
               "avg_launch_us": avg.get(k), "code_object_digest": code_object_digest(GATE_UP_KERNEL),
               "sclk_mhz": {n: v for n, v in clk_mhz.items()
                            if avg.get(n, 0.0) >= 100.0},  # launches of 0.1 ms and longer
               "commands": commands}
        with open(os.path.join(ROOT, "profiles", f"ffn_gate_up_traffic_{workload}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    print("\n".join(lines))


def environment(torch) -> dict:
    env = {"gpu": torch.cuda.get_device_name(0)}
    try:
        env["max_sclk_mhz"] = torch.cuda.get_device_properties(0).clock_rate // 1000
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    env["torch"] = torch.__version__
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    env["host_cpu"] = cpu
    try:
        env["host_threads"] = len(os.sched_getaffinity(0))
    except AttributeError:
        env["host_threads"] = os.cpu_count()
    return env


def wave_placement(moe, torch) -> dict:
    """Whether waves w and w + 4 of a large-tile workgroup share a SIMD on
    this GPU (the ping-pong GEMM schedule is fastest when they do)."""
    n = 256
    simd = torch.full((n, 8), -1, dtype=torch.int32, device="cuda")
    moe.moe_probe_wave_simd(n, simd)
    torch.cuda.synchronize()
    s = simd.cpu().tolist()
    ok = sum(1 for g in s if all(g[w] == g[w + 4] for w in range(4)) and len(set(g[:4])) == 4)
    return {"workgroups": n, "w_and_w_plus_4_share_simd": ok, "example": s[0]}


def time_layer(moe, torch, wl, inp, weights, steps: int, warmup: int) -> dict:
    """Warm up, then run `steps` calls of moe_layer_forward bracketed by
    synchronisations; per-stage and per-step times from HIP events recorded
    by the library on the launch stream."""
    cfg = moe.make_cfg(wl)
    ws = moe.alloc_workspace(cfg, device="cuda")
    aux = moe.alloc_aux(cfg, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16 if wl.act_dtype == 1 else torch.float32,
                      device="cuda")
    stream = torch.cuda.current_stream()

    def step(events=None):
        moe.moe_layer_forward(cfg, weights, inp["x"], inp["bias"], out, aux, ws,
                              stage_events=events, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    hev = HipEvents()
    ns = moe.N_STAGES + 1
    evs = hev.create(steps * ns)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i * ns:(i + 1) * ns])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = [0.0] * moe.N_STAGES
    step_ms = []
    for i in range(steps):
        base = i * ns
        for s_ in range(moe.N_STAGES):
            stage_ms[s_] += hev.elapsed_ms(evs[base + s_], evs[base + s_ + 1]) / steps
        step_ms.append(hev.elapsed_ms(evs[base], evs[base + ns - 1]))
    hev.destroy(evs)
    step_ms.sort()
    res = {
        "ms_per_step": elapsed * 1e3 / steps,
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                    "max": round(step_ms[-1], 4)},
        "stage_ms": dict(zip(moe.STAGES, stage_ms)),
        "kept": int(aux["offsets"][-1].item()),
        "touched": int((aux["counts"] > 0).sum().item()),
        "n_dropped": [int(v) for v in aux["n_dropped"].cpu().tolist()],
        "aux": aux,
    }
    del ws, out
    return res


def touched_weight_bytes(wl, touched: int) -> int:
    wsz = 2 if wl.w_dtype == 1 else 4
    rsz = 2 if wl.router_dtype == 1 else 4
    return (touched * 3 * wl.I * wl.H * wsz + 3 * wl.n_shared * wl.I_shared * wl.H * wsz
            + wl.N * wl.H * rsz)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the decode and skew sub-measurements of the V3 prefill run")
    ap.add_argument("--cpu-sample", type=int, default=64)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarize rocprofv3 output under DIR into profiles/ and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.summarize_profile:
        cmd = "rocprofv3 {opt} -d <dir> -o run --output-format csv -- python3 bench.py {args}"
        run = f"--workload {args.workload} --steps {args.steps} --warmup {args.warmup} " \
              f"--no-cpu-baseline --no-extra"
        pmc = f"--workload {args.workload} --steps 2 --warmup 1 --no-cpu-baseline --no-extra"
        commands = {"trace": cmd.format(opt="--kernel-trace --stats", args=run),
                    "fetch": cmd.format(opt="--pmc FETCH_SIZE", args=pmc),
                    "write": cmd.format(opt="--pmc WRITE_SIZE", args=pmc),
                    "copy_fetch": cmd.format(opt="--pmc FETCH_SIZE", args="--calibrate-copy"),
                    "copy_write": cmd.format(opt="--pmc WRITE_SIZE", args="--calibrate-copy"),
                    "clock": cmd.format(opt="--pmc GRBM_GUI_ACTIVE", args=pmc),
                    "tcp": cmd.format(opt="--pmc TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum "
                                          "TCP_PENDING_STALL_CYCLES_sum GRBM_GUI_ACTIVE", args=pmc)}
        summarize_profile(args.summarize_profile, args.workload, commands, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs the layer on a single MI355X "
              f"(requested --gpus {args.gpus}); multi-GPU sharding is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import routing_expert_ffn_sigmoid_amd as moe
    from routing_expert_ffn_sigmoid_amd import synth, workloads

    wl = workloads.get(args.workload)
    dev = "cuda"
    print(f"[bench] workload {wl.name}: generating inputs in HBM", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl, device=dev)
    # expert weights in the layout the library reads (a one-time load step,
    # outside the timed region); the row-major originals stay for the
    # oracle's CPU baseline
    weights = moe.prepare_weights(moe.make_cfg(wl),
                                  {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    m = time_layer(moe, torch, wl, inp, weights, args.steps, args.warmup)
    ms_per_step = m["ms_per_step"]
    print(f"[bench] {ms_per_step:.3f} ms per step", file=sys.stderr, flush=True)
    kept, touched, st = m["kept"], m["touched"], m["stage_ms"]
    work = algorithmic_work(wl, kept)
    tok_s = wl.T / (ms_per_step / 1e3)

    gate_up_ms = st["ffn_gate_up"]
    achieved_tflops = work["gate_up_flop"] / (gate_up_ms / 1e3) / 1e12
    rec = load_record(args.workload)
    traffic = rec.get("bytes_per_launch") if rec else None
    # algorithmic bytes of the gate/up launch: the touched experts' gate/up
    # weights, the shared expert's, x once, h written once
    es = 2 if wl.act_dtype == 1 else 4
    wsz = 2 if wl.w_dtype == 1 else 4
    Ish = wl.n_shared * wl.I_shared
    gate_up_bytes = (touched * 2 * wl.I * wl.H * wsz + 2 * Ish * wl.H * wsz + wl.T * wl.H * es
                     + (kept * wl.I + wl.T * Ish) * es)
    achieved_gbs = gate_up_bytes / (gate_up_ms / 1e3) / 1e9
    mfma_roof = {"bound": "mfma", "achieved": round(achieved_tflops, 2),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(achieved_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    hbm_roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    # primary roof: HBM when the launch is clearly memory-bound (flop per
    # algorithmic byte under half the ridge point 2500 TFLOP/s / 8 TB/s),
    # MFMA otherwise; the other roof is reported beside it
    intensity = work["gate_up_flop"] / gate_up_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    primary, secondary = (hbm_roof, mfma_roof) if intensity < 0.5 * ridge else (mfma_roof, hbm_roof)
    roofline = dict(primary)
    roofline.update({"traffic": traffic,
                     "kernel": "ffn gate/up grouped GEMM (SwiGLU, routed + shared)",
                     "per_launch_flop": work["gate_up_flop"], "per_launch_bytes": gate_up_bytes,
                     "flop_per_byte": round(intensity, 1), "avg_launch_ms": round(gate_up_ms, 4),
                     "code_object": code_object_digest(GATE_UP_KERNEL),
                     "beside": secondary})
    layer_tflops = work["layer_flop"] / (ms_per_step / 1e3) / 1e12
    # the whole layer against the same MFMA peak (all of the step's flop over
    # the step time), kept inside the roofline object next to the kernel's
    roofline["layer"] = {"bound": "mfma", "achieved": round(layer_tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(layer_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "flop": work["layer_flop"], "ms": round(ms_per_step, 4)}
    tb = touched_weight_bytes(wl, touched)

    res = {
        "metric": "MoE-layer tokens/s (route+dispatch+FFN+combine); % MFMA or HBM peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.act_dtype == 1 else "f32",
        "data": "synthetic (seeded Gaussian inputs and weights in HBM)",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "routed_experts": wl.N,
                   "top_k": wl.k, "groups": f"{wl.n_groups} keep {wl.topk_groups}",
                   "expert_intermediate": wl.I, "shared": f"{wl.n_shared}x{wl.I_shared}",
                   "capacity": wl.capacity, "parallelism": "single GPU"},
        "roofline": roofline,
        "layer": {"roof": "mfma", "mfma_frac": round(layer_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                  "tflops": round(layer_tflops, 2), "layer_flop": work["layer_flop"],
                  "step_ms": m["step_ms"], "kept_rows": kept, "touched_experts": touched,
                  "hbm_frac_touched_weights": round(tb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "stage_ms": {k: round(v, 4) for k, v in st.items()}},
        "clocks": profiled_clocks(rec),
    }
    if wl.name == workloads.V3_PREFILL.name and not args.no_extra:
        # the decode and skew configurations of the same layer, same weights,
        # same process
        extra = {}
        for name, key, sub in (("decode", "v3_decode", workloads.V3_DECODE),
                               ("skew", "v3_skew", workloads.V3_SKEW)):
            si = dict(inp)
            si["x"] = synth.normal((sub.T, sub.H), sub.x_std, torch.bfloat16, dev, sub.seed,
                                   f"x_T{sub.T}")
            if sub.bias_kind == "zipf":
                si["bias"] = synth.zipf_bias(sub.N, sub.bias_param, dev, sub.seed)
            print(f"[bench] {name}: {sub.name}", file=sys.stderr, flush=True)
            r = time_layer(moe, torch, sub, si, weights, args.steps, args.warmup)
            tbs = touched_weight_bytes(sub, r["touched"])
            wk = algorithmic_work(sub, r["kept"])
            e = {"workload": sub.name, "ms_per_step": round(r["ms_per_step"], 4),
                 "step_ms": r["step_ms"], "tokens_per_s": round(sub.T / (r["ms_per_step"] / 1e3), 1),
                 "kept_rows": r["kept"], "touched_experts": r["touched"],
                 "touched_weight_bytes": tbs,
                 "hbm_frac_touched_weights": round(tbs / (r["step_ms"]["median"] / 1e3) / 1e9
                                                   / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(wk["layer_flop"] / (r["step_ms"]["median"] / 1e3) / 1e12
                                    / MFMA_BF16_PEAK_TFLOPS, 4),
                 "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
                 "clocks": profiled_clocks(load_record(key))}
            if sub.capacity:
                e["dropped_assignments"], e["tokens_all_dropped"] = r["n_dropped"]
                e["capacity"] = sub.capacity
            extra[name] = e
            del si, r
            torch.cuda.empty_cache()
        res.update(extra)
    res["wave_placement"] = wave_placement(moe, torch)
    res["environment"] = environment(torch)
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline: oracle on {args.cpu_sample} tokens", file=sys.stderr,
              flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
