"""Benchmark: DeepSeekMoE layer forward (route + dispatch + SwiGLU experts +
combine + load statistics) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-sample S]

Default workload: the V3-shaped prefill layer (T=8192 tokens, hidden 7168,
256 routed SwiGLU experts of width 2048 in 8 groups, keep 4 groups, top-8,
sigmoid scores with selection bias, 1 shared expert), bf16 activations and
expert weights, fp32 router.  Inputs are seeded synthetic tensors generated
directly in HBM; the timed region is K calls of moe_layer_forward with
everything already resident.

Prints one JSON line.  `value` = tokens/s of the whole layer.  `roofline`
describes the dominant kernel (the SwiGLU gate/up grouped GEMM), timed with
HIP events recorded on the launch stream around that stage in every timed
step.  `cpu_baseline` is the single-threaded C oracle on a bounded sample of
tokens of the same workload.
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


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_src: str, workload: str):
    """Measured HBM bytes per launch of the gate/up kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"ffn_gate_up_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest([kernel_src]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, inp, logits_gpu, sample: int) -> dict:
    """The C oracle (one thread) on `sample` tokens of the workload: router
    logits, routing, dispatch and the layer output of each sampled token."""
    import numpy as np
    import torch

    import oracle

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
    # the weights the sampled tokens need, copied to host before timing
    lg = logits_gpu[toks].cpu().numpy()
    r0 = oracle.route(lg, bias, wl.k, wl.n_groups, wl.topk_groups, wl.group_topn, fn,
                      wl.norm_topk, wl.route_scale)
    experts = sorted(set(int(e) for e in r0["topk_idx"].ravel()))
    w13 = {e: typed(inp["w13"][e]) for e in experts}
    w2 = {e: typed(inp["w2"][e]) for e in experts}
    ws13 = typed(inp["ws13"]) if inp.get("ws13") is not None else None
    ws2 = typed(inp["ws2"]) if inp.get("ws2") is not None else None

    t0 = time.perf_counter()
    logits = oracle.router_logits(x, wg).astype(np.float32)
    r = oracle.route(logits, bias, wl.k, wl.n_groups, wl.topk_groups, wl.group_topn, fn,
                     wl.norm_topk, wl.route_scale)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], wl.N, wl.capacity)
    for i in range(len(toks)):
        sel = [int(e) for e in r["topk_idx"][i]]
        a13 = [w13.get(e) if d["inv_row"][i, j] >= 0 else None for j, e in enumerate(sel)]
        a2 = [w2.get(e) if d["inv_row"][i, j] >= 0 else None for j, e in enumerate(sel)]
        if any(a is None and d["inv_row"][i, j] >= 0 for j, a in enumerate(a13)):
            continue  # fp32 rounding of the oracle's own logits chose an uncopied expert
        oracle.token_output(x[i], a13, a2, r["topk_gate"][i], ws13, ws2, wl.n_shared,
                            wl.I_shared, wl.I)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(toks)} tokens of {wl.name}: router logits, routing, dispatch and "
                      f"the layer output of each, single-threaded C, {dt:.1f} s"}


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


def summarize_profile(d: str, workload: str, commands: dict):
    """Turn the raw rocprofv3 output under d (trace/, fetch/, write/,
    copy_fetch/, copy_write/) into profiles/<kernel>_<workload>.txt and the
    gate/up traffic record profiles/ffn_gate_up_traffic_<workload>.json."""
    stats = _csv_rows(os.path.join(d, "trace", "**", "*kernel_stats.csv"))
    lines = [f"# rocprofv3 summary: DeepSeekMoE layer forward, workload {workload}", ""]
    for key in ("trace", "fetch", "write", "copy_fetch", "copy_write"):
        if key in commands:
            lines.append(f"{key}: {commands[key]}")
    lines += ["", "## kernel trace (--kernel-trace --stats), library kernels",
              f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    avg = {}
    for r in stats:
        name = r["Name"]
        if "moe::" not in name:
            continue
        short = name.replace("void ", "").split("(")[0]
        avg[short] = float(r["AverageNs"]) / 1e3
        lines.append(f"{short:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.1f} "
                     f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f}")

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
        src = os.path.join(ROOT, "routing_expert_ffn_sigmoid_amd", "csrc", "grouped_ffn.hip")
        rec = {"kernel": k, "workload": workload, "bytes_per_launch": traffic[k],
               "fetch_kib": fetch.get(k), "write_kib": write.get(k),
               "fetch_scale": f_scale, "write_scale": w_scale,
               "avg_launch_us": avg.get(k), "source_digest": source_digest([src]),
               "commands": commands}
        with open(os.path.join(ROOT, "profiles", f"ffn_gate_up_traffic_{workload}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        run = f"--workload {args.workload} --steps 5 --warmup 2 --no-cpu-baseline"
        pmc = f"--workload {args.workload} --steps 2 --warmup 1 --no-cpu-baseline"
        commands = {"trace": cmd.format(opt="--kernel-trace --stats", args=run),
                    "fetch": cmd.format(opt="--pmc FETCH_SIZE", args=pmc),
                    "write": cmd.format(opt="--pmc WRITE_SIZE", args=pmc),
                    "copy_fetch": cmd.format(opt="--pmc FETCH_SIZE", args="--calibrate-copy"),
                    "copy_write": cmd.format(opt="--pmc WRITE_SIZE", args="--calibrate-copy")}
        summarize_profile(args.summarize_profile, args.workload, commands)
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
    cfg = moe.make_cfg(wl)
    ws = moe.alloc_workspace(cfg, device=dev)
    aux = moe.alloc_aux(cfg, device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16 if wl.act_dtype == 1 else torch.float32,
                      device=dev)
    stream = torch.cuda.current_stream()
    # expert weights in the layout the library reads (a one-time load step,
    # outside the timed region)
    # (the row-major originals stay for the oracle's CPU baseline)
    weights = moe.prepare_weights(cfg, {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    torch.cuda.synchronize()

    def step(events=None):
        moe.moe_layer_forward(cfg, weights, inp["x"], inp["bias"], out, aux, ws,
                              stage_events=events, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hev = HipEvents()
    ns = moe.N_STAGES + 1
    evs = hev.create(args.steps * ns)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i * ns:(i + 1) * ns])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = [0.0] * moe.N_STAGES
    for i in range(args.steps):
        base = i * ns
        for s in range(moe.N_STAGES):
            stage_ms[s] += hev.elapsed_ms(evs[base + s], evs[base + s + 1]) / args.steps
    hev.destroy(evs)
    print(f"[bench] timed {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    ms_per_step = elapsed * 1e3 / args.steps
    kept = int(aux["offsets"][-1].item())
    touched = int((aux["counts"] > 0).sum().item())
    work = algorithmic_work(wl, kept)
    tok_s = wl.T / (ms_per_step / 1e3)
    st = dict(zip(moe.STAGES, stage_ms))

    gate_up_ms = st["ffn_gate_up"]
    achieved_tflops = work["gate_up_flop"] / (gate_up_ms / 1e3) / 1e12
    kernel_src = os.path.join(ROOT, "routing_expert_ffn_sigmoid_amd", "csrc", "grouped_ffn.hip")
    traffic = load_traffic(kernel_src, args.workload)
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
                     "beside": secondary})
    layer_tflops = work["layer_flop"] / (ms_per_step / 1e3) / 1e12
    touched_bytes = touched * 3 * wl.I * wl.H * 2 + 3 * wl.n_shared * wl.I_shared * wl.H * 2

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
        "layer": {"mfma_frac": round(layer_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                  "tflops": round(layer_tflops, 2), "kept_rows": kept,
                  "touched_experts": touched,
                  "touched_weight_gbs": round(touched_bytes / (ms_per_step / 1e3) / 1e9, 1),
                  "hbm_frac_touched_weights": round(touched_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "stage_ms": {k: round(v, 4) for k, v in st.items()}},
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline: oracle on {args.cpu_sample} tokens", file=sys.stderr,
              flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, inp, aux["logits"], args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
