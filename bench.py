"""Benchmark of the dequantise-fused GEMV path on one MI355X.

A step is one pass of the 27B-class dense layer at N = 1 (one decode token):
  QKV projection   [7168][5120]        G32 asymmetric int4
  gate/up + SwiGLU [2 x 17408][5120]   G32 asymmetric int5 (fused SwiGLU)
  down + residual  [5120][17408]       G32 asymmetric int5 (fused residual)
Weights and activations are seeded synthetic data of those shapes (no
checkpoint exists here). Layers are rotated over distinct device copies so
that the working set (several GB) far exceeds the 256 MB Infinity Cache and
every step reads its weights from HBM.

value = algorithmic bytes per step / time per step (GB/s): packed weights and
scales + x (bf16) + outputs (fp32) + residual read.

Also reported on the same JSON line:
  roofline      the dominant kernel (gate/up + SwiGLU, int5) against 8 TB/s:
                its average launch duration from HIP events on the launch
                stream around batches of back-to-back launches (median batch)
  nvfp4_layer   the same layer in NVFP4 at N = 1, 2, 4, 8, 16, 32
  per_format    qgemv on [17408][5120] for each format at N = 1, 2, 4, 8, 16,
                and qgemv_mx (MXFP4 / MXFP8
                weights, MXFP8 activations) at N = 1, 2, 4, 8, 16, 32, alone
                and after qgemv_act_quant
  moe           qgemv_moe on the 128-expert, top-8 workload at N = 1 and 8
  probe         the plain streaming-read kernel on the same rotation
  cpu_baseline  the CPU oracle on a bounded sample of the layer
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
LAYER = [("qkv", 7168, 5120, "int4"), ("gate_up", 2 * 17408, 5120, "int5"), ("down", 5120, 17408, "int5")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(qg, fmt, M, K):
    a, b = qg.packed_bytes(fmt, M, K)
    return a + b


# the committed rocprofv3 summary of --profile-set (kernel trace and counters)
PROFILE_SUMMARY = "qgemv_kernels_trace_and_counters.txt"

# the sources the dense kernels (k_gemv) are compiled from
DENSE_SOURCES = ["gemv.hip", "kloop.hpp", "device.hpp", "layout.hpp", "mx.hpp"]


def kernel_source_hash() -> str:
    """sha256 over the dense kernels' sources (and the ABI header)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_quantized_weight_amd", "csrc")
    for f in DENSE_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "qgemv.h"), "rb") as fh:
        h.update(b"qgemv.h" + fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(name: str, src_hash: str):
    """HBM bytes per launch of profiling case `name` from the committed
    rocprofv3 summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the same
    counter reads for a 1 GiB device copy), or None when the summary is
    missing or was taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", PROFILE_SUMMARY)
    try:
        with open(p) as f:
            lines = [ln.strip() for ln in f]
    except OSError:
        return None
    if f"src_hash: {src_hash}" not in lines:
        return None
    key = f"traffic {name}:"
    for ln in lines:
        if ln.startswith(key):
            return int(ln[len(key):].split()[0])
    return None


def mx_only(qg, torch, synthetic, dev, steps):
    """MXFP8 / MXFP4 qgemv_mx on [17408][5120] at N = 1 after qgemv_act_quant,
    rotated over >= 1.2 GB of weight copies; HIP events on the launch stream."""
    M, K, N = 17408, 5120, 1
    W = synthetic.weights(synthetic.rng_for(0, 3, M), M, K)
    x = torch.from_numpy(synthetic.activations(synthetic.rng_for(0, 3, 4), N, K)).to(dev)
    xq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((N, M), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = {"workload": "qgemv_mx [17408][5120], N=1, MXFP8 activations", "steps": steps}
    for fmt in ("mxfp8", "mxfp4"):
        wq, ws = qg.pack(fmt, W)
        nb = wq.size + ws.size
        copies = max(2, int(np.ceil(1.2e9 / nb)))
        d = [(torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)) for _ in range(copies)]
        for i in range(10):
            qg.act_quant(x, xq, xs, N, K)
            qg.qgemv_mx(fmt, *d[i % copies], xq, xs, y, M, K, N)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            qg.act_quant(x, xq, xs, N, K)
            qg.qgemv_mx(fmt, *d[i % copies], xq, xs, y, M, K, N)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        byt = nb + N * K + N * K // 32 + N * M * 4
        out[fmt] = {"us_per_pair": round(us, 2), "weight_bytes": nb, "algorithmic_bytes": byt}
        del d
        torch.cuda.empty_cache()
    return out


# Cases of --profile-set, in run order: (name, kind, format, M, K, N). Each
# runs `steps` launches (steps) after 3 warm-up steps; a 16-byte probe
# launch before each case marks it in the kernel trace.
PROFILE_CASES = [("layer_int_n1", "layer", "int", 0, 0, 1), ("gu_int5_n1", "gu", "int5", 2 * 17408, 5120, 1),
                 ("gu_int5_n8", "gu", "int5", 2 * 17408, 5120, 8)] + \
    [(f"perfmt_{f}_n{n}", "perfmt", f, 17408, 5120, n) for f in ("int4", "int5", "int8", "nvfp4") for n in (1, 8)] + \
    [("layer_nvfp4_n8", "layer", "nvfp4", 0, 0, 8), ("moe_n1", "moe", "int4", 0, 0, 1), ("moe_n8", "moe", "int4", 0, 0, 8),
     ("moe_fused_n1", "moe_fused", "int4", 0, 0, 1), ("moe_fused_n8", "moe_fused", "int4", 0, 0, 8)]


def profile_set(qg, torch, synthetic, dev, steps, calib_mib):
    """Run every PROFILE_CASES case for rocprofv3 (kernel trace, counters).
    Prints one JSON line: per case the launches per step and the
    algorithmic bytes per step, for --summarize-profile."""
    stream = torch.cuda.current_stream()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    mark = torch.zeros(16, dtype=torch.uint8, device=dev)
    wsp = qg.split_workspace(dev)
    out = {"steps": steps, "src_hash": kernel_source_hash(), "cases": {}}
    if calib_mib > 0:
        qg.qgemv_probe_read(mark, 16, sink)
        src = torch.ones(calib_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        out["calib_copy_bytes"] = calib_mib << 20
    for name, kind, fmt, M, K, N in PROFILE_CASES:
        rng = synthetic.rng_for(0, 12, len(name))
        if kind in ("perfmt", "gu"):
            wq, ws = qg.pack(fmt, synthetic.weights(rng, M, K))
            nb = wq.size + ws.size
            copies = max(2, int(np.ceil(1.1e9 / nb)))
            d = [(torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)) for _ in range(copies)]
            x = torch.from_numpy(synthetic.activations(rng, N, K, 0.01 if kind == "perfmt" else 0.0)).to(dev)
            Mo = M // 2 if kind == "gu" else M
            y = torch.empty((N, Mo), dtype=torch.float32, device=dev)
            per = 1
            byt = nb + N * K * 2 + N * Mo * 4

            if kind == "gu":
                def step(i):
                    qg.qgemv_swiglu_ex(fmt, *d[i % copies], x, y, Mo, K, N, workspace=wsp)
            else:
                def step(i):
                    qg.qgemv_ex(fmt, *d[i % copies], x, y, M, K, N, workspace=wsp)
        elif kind == "layer":
            fm = {"qkv": "int4", "gate_up": "int5", "down": "int5"} if fmt == "int" else \
                {"qkv": fmt, "gate_up": fmt, "down": fmt}
            host = {nm: qg.pack(fm[nm], synthetic.weights(rng, Mm, Kk)) for nm, Mm, Kk, _ in LAYER}
            nb = sum(a.size + b.size for a, b in host.values())
            copies = max(2, int(np.ceil(1.1e9 / nb)))
            d = [{k: (torch.from_numpy(v[0]).to(dev), torch.from_numpy(v[1]).to(dev)) for k, v in host.items()}
                 for _ in range(copies)]
            x = torch.from_numpy(synthetic.activations(rng, N, 5120)).to(dev)
            xd = torch.from_numpy(synthetic.activations(rng, N, 17408)).to(dev)
            qkv = torch.empty((N, 7168), dtype=torch.float32, device=dev)
            h = torch.empty((N, 17408), dtype=torch.float32, device=dev)
            r = torch.from_numpy(synthetic.residual(rng, N, 5120)).to(dev)
            y = torch.empty((N, 5120), dtype=torch.float32, device=dev)
            per = 3
            byt = nb + N * (5120 * 2 + 7168 * 4 + 5120 * 2 + 17408 * 4 + 17408 * 2 + 5120 * 8)

            def step(i):
                L = d[i % copies]
                qg.qgemv_ex(fm["qkv"], *L["qkv"], x, qkv, 7168, 5120, N, workspace=wsp)
                qg.qgemv_swiglu_ex(fm["gate_up"], *L["gate_up"], x, h, 17408, 5120, N, workspace=wsp)
                qg.qgemv_ex(fm["down"], *L["down"], xd, y, 5120, 17408, N, residual=r, workspace=wsp)
        else:
            E, H, I, k = 128, 2048, 768, 8
            bufs, per_expert = moe_buffers(qg, synthetic, torch, dev, E, H, I, copies=8)
            copies = len(bufs)
            sets = [synthetic.router_logits(rng, N, E) for _ in range(16)]
            uniq = [len({int(e) for e in np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k].reshape(-1)})
                    for lg in sets]
            xb = torch.from_numpy(synthetic.activations(rng, N, H)).to(dev)
            rr = torch.from_numpy(synthetic.residual(rng, N, H)).to(dev)
            y = torch.empty((N, H), dtype=torch.float32, device=dev)
            byt = float(np.mean(uniq)) * per_expert + N * H * 2 + N * H * 8 + N * k * 8
            if kind == "moe":
                idsg = []
                for lg in sets:
                    ids = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)
                    g = np.exp(np.take_along_axis(lg.astype(np.float64), ids, 1))
                    idsg.append((torch.from_numpy(ids).to(dev), torch.from_numpy((g / g.sum(1, keepdims=True)).astype(np.float32)).to(dev)))
                nbytes = qg.moe_workspace_bytes(E, H, I, N, k)
                mw = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
                per = 3

                def step(i):
                    qg.qgemv_moe("int4", *bufs[i % copies], E, H, I, xb, *idsg[i % 16], k, y, N, mw, nbytes, residual=rr)
            else:
                lt = [torch.from_numpy(lg).to(dev) for lg in sets]
                nbytes = qg.moe_fused_workspace_bytes(E, H, I, N, k)
                mw = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
                per = 1 if N * k <= 8 else 4

                def step(i):
                    qg.qgemv_moe_fused("int4", *bufs[i % copies], E, H, I, xb, lt[i % 16], k, y, N, mw, nbytes,
                                       residual=rr)
        for i in range(3):
            step(i)
        torch.cuda.synchronize()
        qg.qgemv_probe_read(mark, 16, sink)        # marker: the case's launches follow
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            step(3 + i)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        out["cases"][name] = {"launches_per_step": per, "algorithmic_bytes_per_step": int(byt),
                              "us_per_step_events": round(us, 2)}
        log(name, out["cases"][name])
        del step
        torch.cuda.empty_cache()
    qg.check_split_workspace(wsp)
    print(json.dumps(out), flush=True)


def moe_buffers(qg, synthetic, torch, dev, E, H, I, copies):
    """Expert-stacked int4 buffers of E experts ([2I][H] gate/up, [H][I]
    down), packed once on the host, `copies` device copies."""
    sq, ss = qg.expert_stride("int4", 2 * I, H)
    dq, ds = qg.expert_stride("int4", H, I)
    bufs = [np.zeros(E * sq, np.uint8), np.zeros(E * ss, np.uint8), np.zeros(E * dq, np.uint8), np.zeros(E * ds, np.uint8)]
    rng = synthetic.rng_for(0, 5)
    for e in range(E):
        q, s = qg.pack("int4", synthetic.weights(rng, 2 * I, H))
        bufs[0][e * sq: e * sq + q.size] = q
        bufs[1][e * ss: e * ss + s.size] = s
        q, s = qg.pack("int4", synthetic.weights(rng, H, I))
        bufs[2][e * dq: e * dq + q.size] = q
        bufs[3][e * ds: e * ds + s.size] = s
    return [[torch.from_numpy(b).to(dev) for b in bufs] for _ in range(copies)], sq + ss + dq + ds


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _manifest(log_path):
    with open(log_path) as f:
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"cases"' in ln:
                return json.loads(ln)
    raise SystemExit(f"no --profile-set manifest line in {log_path}")


def _case_groups(rows, man, name_key, order_key):
    """Split dispatch rows (dicts with a kernel name) into the manifest's
    cases: after each case's marker (a k_probe launch) come its timed steps,
    the first steps x launches_per_step library dispatches; before the first
    case, the calibration copies (when the run had them)."""
    rows = sorted(rows, key=lambda r: int(r[order_key]))
    groups, cur, pre = [], None, []
    for r in rows:
        if "k_probe" in r[name_key]:
            cur = []
            groups.append(cur)
        elif cur is None:
            pre.append(r)
        else:
            cur.append(r)
    calib = []
    if "calib_copy_bytes" in man and groups:
        calib = [r for r in groups[0] if "copy" in r[name_key].lower()]
        groups = groups[1:]
    out = {}
    for (name, meta), g in zip(man["cases"].items(), groups):
        n = man["steps"] * meta["launches_per_step"]
        out[name] = [r for r in g if "qg::" in r[name_key]][:n]
    return out, calib


def summarize_profile(out_path, command_lines, trace, counter_runs):
    """Text summary of --profile-set runs under rocprofv3: per case and
    kernel, launches and average duration (kernel trace) and, per launch, the
    counters of each --pmc run (FETCH_SIZE / WRITE_SIZE also as bytes,
    scaled by what they read for the 1 GiB calibration copy).
    trace, counter_runs: (directory, log with the run's manifest line)."""
    import glob
    tdir, tlog = trace
    man = _manifest(tlog)
    tr = glob.glob(os.path.join(tdir, "**", "*kernel_trace.csv"), recursive=True)
    tcases, _ = _case_groups(_csv_rows(tr[0]), man, "Kernel_Name", "Start_Timestamp")
    counters, scale = [], {}
    for cdir, clog in counter_runs:
        cman = _manifest(clog)
        cc = glob.glob(os.path.join(cdir, "**", "*counter_collection.csv"), recursive=True)
        by_disp = {}
        for r in _csv_rows(cc[0]):
            c = by_disp.setdefault(r["Dispatch_Id"], {"Kernel_Name": r["Kernel_Name"], "Dispatch_Id": r["Dispatch_Id"]})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        cases, calib = _case_groups(list(by_disp.values()), cman, "Kernel_Name", "Dispatch_Id")
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [c[cn] for c in calib if cn in c]
            if vals:
                scale[cn] = cman["calib_copy_bytes"] / (float(np.median(vals)) * 1024)
        counters.append(cases)
    src_hash = man.get("src_hash", "unrecorded")
    lines = [f"# rocprofv3 summary of bench.py --profile-set (kernel sources: src_hash {src_hash})", "",
             "commands (from /tmp with TMPDIR=/tmp; R = the repository root):"]
    lines += [f"  {c}" for c in command_lines] + [""]
    if scale:
        lines.append("calibration: for a 1 GiB device copy FETCH_SIZE reads {:.4f} and WRITE_SIZE {:.4f} of the "
                     "bytes moved; the byte figures below are scaled by the inverse".format(
                         1 / scale.get("FETCH_SIZE", float("nan")), 1 / scale.get("WRITE_SIZE", float("nan"))))
        lines.append("")
    lines.append(f"{'case':16s} {'kernel':52s} {'calls':>6s} {'avg us':>8s}   counters per launch (means)")
    for name, meta in man["cases"].items():
        per_kernel = {}
        for r in tcases.get(name, []):
            per_kernel.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        step_us = 0.0
        for kn, durs in per_kernel.items():
            short = kn.replace("void ", "").split("(")[0].replace("qg::", "")[:52]
            cs = []
            for cases in counters:
                sel = [c for c in cases.get(name, []) if c["Kernel_Name"] == kn]
                if not sel:
                    continue
                for k in sorted(k for k in sel[0] if k not in ("Kernel_Name", "Dispatch_Id")):
                    v = float(np.mean([c[k] for c in sel]))
                    if k in scale:
                        cs.append(f"{k}={v:.0f}KiB={v * 1024 * scale[k] / 1e6:.2f}MB")
                    else:
                        cs.append(f"{k}={v:.4g}")
            avg = float(np.mean(durs))
            step_us += avg * len(durs) / man["steps"]
            lines.append(f"{name:16s} {short:52s} {len(durs):6d} {avg:8.2f}   " + " ".join(cs))
        if per_kernel:
            gbs = meta["algorithmic_bytes_per_step"] / (step_us * 1e-6) / 1e9
            lines.append(f"{name:16s} {'= step: sum of the kernel averages':52s} {'':6s} {step_us:8.2f}   "
                         f"{meta['algorithmic_bytes_per_step']} algorithmic B -> {gbs:.0f} GB/s "
                         f"({gbs / PEAK_GBS:.3f} of 8 TB/s); HIP events in the same run {meta['us_per_step_events']} us")
    # machine-readable traffic per launch of the single-kernel cases (bench.py
    # reads these for its roofline entries; they hold only for this src_hash)
    if {"FETCH_SIZE", "WRITE_SIZE"} <= set(scale):
        lines += ["", "machine-readable (HBM bytes per launch, scaled FETCH_SIZE + WRITE_SIZE):", f"src_hash: {src_hash}"]
        for name, meta in man["cases"].items():
            if meta["launches_per_step"] != 1:
                continue
            tot = 0.0
            for cases in counters:
                sel = cases.get(name, [])
                for cn in ("FETCH_SIZE", "WRITE_SIZE"):
                    vals = [c[cn] for c in sel if cn in c]
                    if vals:
                        tot += float(np.mean(vals)) * 1024 * scale[cn]
            lines.append(f"traffic {name}: {int(round(tot))}  (algorithmic {meta['algorithmic_bytes_per_step']})")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=16, help="distinct layer copies rotated on the device")
    ap.add_argument("--no-extra", action="store_true", help="skip per-format, MoE, probe and CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB three times "
                         "(the known-size reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--profile-set", action="store_true",
                    help="run the profiling cases (per-format [17408][5120] at N = 1 and 8, the dense layer, "
                         "the NVFP4 layer at N = 8, MoE) under rocprofv3 and print their manifest")
    ap.add_argument("--summarize-profile", nargs="+", metavar="ARG",
                    help="OUT_TXT COMMANDS_TXT TRACE_DIR:LOG [COUNTER_DIR:LOG ...]: write the text summary of "
                         "--profile-set runs (each directory with the log holding that run's manifest line; "
                         "COMMANDS_TXT: the profiler command lines, one per line)")
    ap.add_argument("--mx-only", action="store_true",
                    help="only the MX GEMV on [17408][5120] at N = 1 (MXFP8 and MXFP4, after the activation "
                         "quantiser): a short run for profiling those kernels")
    args = ap.parse_args()
    if args.summarize_profile:
        a = args.summarize_profile
        with open(a[1]) as f:
            cmds = [ln.rstrip("\n") for ln in f if ln.strip()]
        pairs = [tuple(x.split(":", 1)) for x in a[2:]]
        summarize_profile(a[0], cmds, pairs[0], pairs[1:])
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_weight_amd as qg
    import synthetic

    qg.load()
    dev = torch.device("cuda:0")
    if args.mx_only:
        print(json.dumps(mx_only(qg, torch, synthetic, dev, args.steps)), flush=True)
        return
    if args.profile_set:
        profile_set(qg, torch, synthetic, dev, args.steps, args.calib_copy_mib)
        return
    stream = torch.cuda.current_stream()
    N = 1
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: 3 x {args.calib_copy_mib} MiB")

    # ---- weights: a few unique layers packed on the host, replicated on device
    uniq = 2
    t0 = time.time()
    host_layers = []
    for u in range(uniq):
        mats = {}
        for name, M, K, fmt in LAYER:
            rng = synthetic.rng_for(0, 2, u, M)
            W = synthetic.weights(rng, M, K)
            mats[name] = qg.pack(fmt, W)
            del W
        host_layers.append(mats)
    log(f"packed {uniq} unique layers in {time.time() - t0:.1f}s")
    layers = []
    for li in range(args.layers):
        src = host_layers[li % uniq]
        layers.append({k: (torch.from_numpy(v[0]).to(dev), torch.from_numpy(v[1]).to(dev)) for k, v in src.items()})
    del host_layers
    rng = synthetic.rng_for(0, 2, 99)
    x = torch.from_numpy(synthetic.activations(rng, N, 5120)).to(dev)
    h = torch.empty((N, 17408), dtype=torch.float32, device=dev)
    qkv = torch.empty((N, 7168), dtype=torch.float32, device=dev)
    res = torch.from_numpy(synthetic.residual(rng, N, 5120)).to(dev)
    y = torch.empty((N, 5120), dtype=torch.float32, device=dev)
    xd = torch.from_numpy(synthetic.activations(rng, N, 17408)).to(dev)  # bf16 input of the down projection

    layer_w = sum(weight_bytes(qg, f, M, K) for _, M, K, f in LAYER)
    act = (N * 5120 * 2 + N * 7168 * 4) + (N * 5120 * 2 + N * 17408 * 4) + (N * 17408 * 2 + N * 5120 * 4 * 2)
    step_bytes = layer_w + act
    gu_bytes = weight_bytes(qg, "int5", 2 * 17408, 5120) + N * 5120 * 2 + N * 17408 * 4
    log(f"layer weights {layer_w / 1e6:.1f} MB, rotation {args.layers} layers = {args.layers * layer_w / 1e9:.2f} GB")

    # split-remainder workspace: the launches balance their last row blocks
    wsp = qg.split_workspace(dev)

    def step(i):
        L = layers[i % args.layers]
        qg.qgemv_ex("int4", *L["qkv"], x, qkv, 7168, 5120, N, workspace=wsp)
        qg.qgemv_swiglu_ex("int5", *L["gate_up"], x, h, 17408, 5120, N, workspace=wsp)
        qg.qgemv_ex("int5", *L["down"], xd, y, 5120, 17408, N, residual=res, workspace=wsp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us -> {value:.0f} GB/s")

    # Per-kernel average launch duration: batches of back-to-back launches of
    # one kernel over the rotated layers, events on the launch stream; the
    # median over batches.
    def time_alone(fn, reps, batches=5):
        for i in range(min(reps, 8)):
            fn(i)
        torch.cuda.synchronize()
        out = []
        for bi in range(batches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                fn(bi * reps + i)
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return float(np.median(out)), float(min(out)), float(max(out))

    kern = {}
    kern["qkv_int4"] = (time_alone(lambda i: qg.qgemv_ex("int4", *layers[i % args.layers]["qkv"], x, qkv, 7168, 5120, N,
                                                         workspace=wsp), 300),
                        weight_bytes(qg, "int4", 7168, 5120) + N * 5120 * 2 + N * 7168 * 4)
    kern["gate_up_swiglu_int5"] = (time_alone(lambda i: qg.qgemv_swiglu_ex("int5", *layers[i % args.layers]["gate_up"], x, h,
                                                                            17408, 5120, N, workspace=wsp), 150), gu_bytes)
    kern["down_residual_int5"] = (time_alone(lambda i: qg.qgemv_ex("int5", *layers[i % args.layers]["down"], xd, y, 5120,
                                                                   17408, N, residual=res, workspace=wsp), 200),
                                  weight_bytes(qg, "int5", 5120, 17408) + N * 17408 * 2 + N * 5120 * 8)
    kernels = {k: {"us": round(t[0] * 1e3, 2), "us_min": round(t[1] * 1e3, 2), "us_max": round(t[2] * 1e3, 2),
                   "GB/s": round(b / (t[0] * 1e-3) / 1e9, 1)} for k, (t, b) in kern.items()}
    log("kernels alone:", kernels)
    gu_ms = kern["gate_up_swiglu_int5"][0][0]
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9

    # the same gate/up + SwiGLU kernel at N = 8 (eight decode lanes)
    x8 = torch.from_numpy(synthetic.activations(synthetic.rng_for(0, 2, 98), 8, 5120)).to(dev)
    h8 = torch.empty((8, 17408), dtype=torch.float32, device=dev)
    gu8_bytes = weight_bytes(qg, "int5", 2 * 17408, 5120) + 8 * 5120 * 2 + 8 * 17408 * 4
    gu8_ms = time_alone(lambda i: qg.qgemv_swiglu_ex("int5", *layers[i % args.layers]["gate_up"], x8, h8, 17408, 5120, 8,
                                                     workspace=wsp), 150)[0]
    gu8_gbs = gu8_bytes / (gu8_ms * 1e-3) / 1e9

    # the MLP block chained on the device, each launch consuming the previous
    # one's output (NInfer article, section 2: norm, matmul, SwiGLU and
    # residual fused per format): RMSNorm(r) -> gate/up + SwiGLU -> bf16 h ->
    # down(h) + r, int5, N = 1, rotated layers
    gamma = torch.from_numpy((1 + 0.1 * synthetic.rng_for(0, 7).standard_normal(5120)).astype(np.float32)).to(dev)
    r1 = torch.from_numpy(synthetic.residual(synthetic.rng_for(0, 7, 1), 1, 5120)).to(dev)
    hb = torch.zeros((1, 17408), dtype=torch.int16, device=dev)
    ym = torch.empty((1, 5120), dtype=torch.float32, device=dev)

    def mlp(i):
        L = layers[i % len(layers)]
        qg.qgemv_swiglu_ex("int5", *L["gate_up"], None, None, 17408, 5120, 1, norm_src=r1, norm_gamma=gamma,
                           norm_eps=1e-6, out_bf16=hb, workspace=wsp)
        qg.qgemv_ex("int5", *L["down"], hb, ym, 5120, 17408, 1, residual=r1, workspace=wsp)
    mlp_bytes = (weight_bytes(qg, "int5", 2 * 17408, 5120) + weight_bytes(qg, "int5", 5120, 17408)
                 + 5120 * 4 * 2 + 5120 * 4 + 17408 * 2 * 2 + 5120 * 8)
    mlp_ms = time_alone(mlp, 100)[0]

    src_hash = kernel_source_hash()
    qg.check_split_workspace(wsp)
    roofline = {"bound": "hbm", "kernel": "k_gemv<int5, swiglu> (gate/up + SwiGLU, split remainder), N=1",
                "achieved": round(gu_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / PEAK_GBS, 4),
                "traffic": pmc_traffic("gu_int5_n1", src_hash),
                "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_ms * 1e3, 2)}
    roofline_n8 = {"bound": "hbm", "kernel": "k_gemv<int5, swiglu> (gate/up + SwiGLU, split remainder), N=8",
                   "achieved": round(gu8_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                   "frac": round(gu8_gbs / PEAK_GBS, 4), "traffic": pmc_traffic("gu_int5_n8", src_hash),
                   "algorithmic_bytes_per_launch": gu8_bytes, "avg_launch_us": round(gu8_ms * 1e3, 2)}
    mlp_chain = {"workload": "27B-class MLP block, N=1, dependent launches: RMSNorm + gate/up 2x17408x5120 int5 + "
                             "SwiGLU -> bf16 h -> down 5120x17408 int5 + residual",
                 "us_per_block": round(mlp_ms * 1e3, 2), "GB/s": round(mlp_bytes / (mlp_ms * 1e-3) / 1e9, 1),
                 "frac": round(mlp_bytes / (mlp_ms * 1e-3) / 1e9 / PEAK_GBS, 4), "algorithmic_bytes": mlp_bytes}
    log("roofline N=8", roofline_n8, "mlp_chain", mlp_chain)

    extra = {}
    if not args.no_extra:
        extra = extras(qg, torch, dev, stream, layers, args, wsp)
        del layers
        torch.cuda.empty_cache()
        extra["cpu_baseline"] = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "achieved HBM GB/s (% of MI355X peak) for qgemv at N=1 and N=8, per format",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "27B-class dense layer, N=1: QKV 7168x5120 int4 + gate/up 2x17408x5120 int5 "
                               "with SwiGLU + down 5120x17408 int5 with residual",
                   "step": "three launches in stream order whose inputs do not depend on each other (QKV and "
                           "gate/up read x, down reads a separate bf16 input); mlp_chain is the dependent chain",
                   "layers_rotated": args.layers, "rotation_GB": round(args.layers * layer_w / 1e9, 2),
                   "algorithmic_bytes_per_step": step_bytes, "frac_of_peak": round(value / PEAK_GBS, 4),
                   "tok_per_s_64_layers": round(1.0 / (64 * ms_step * 1e-3), 1),
                   "arithmetic": "bf16 MFMA operands (exact codes), fp32 accumulate"},
        "roofline": roofline,
        "roofline_n8": roofline_n8,
        "mlp_chain": mlp_chain,
        "kernels": kernels,
        "src_hash": src_hash,
    }
    out.update({k: v for k, v in extra.items() if k != "cpu_baseline"})
    out["cpu_baseline"] = extra.get("cpu_baseline")
    print(json.dumps(out), flush=True)


def extras(qg, torch, dev, stream, layers, args, wsp):
    import synthetic
    res = {}

    def timeit(fn, reps, batches=3):
        # warm launches, then the median of `batches` event-timed batches
        for i in range(16):
            fn(i)
        torch.cuda.synchronize()
        out = []
        for bi in range(batches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                fn(bi * reps + i)
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return float(np.median(out))

    # probe: plain streaming read of each 134 MB gate/up weight buffer
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    pb = [L["gate_up"][0] for L in layers]
    ms = timeit(lambda i: qg.qgemv_probe_read(pb[i % len(pb)], pb[0].numel() // 16 * 16, sink), 64)
    res["probe"] = {"bytes": pb[0].numel(), "us": round(ms * 1e3, 2), "GB/s": round(pb[0].numel() / (ms * 1e-3) / 1e9, 1)}
    log("probe", res["probe"])

    # the same layer in NVFP4 at N = 1, 2, 4, 8 (1-8 decode lanes) and 16, 32
    # (verify windows of 8 lanes), 8 rotated layer copies
    nv = {}
    nv_host = {}
    for name, M_, K_, _ in LAYER:
        rng_l = synthetic.rng_for(0, 3, 1, M_)
        nv_host[name] = qg.pack("nvfp4", synthetic.weights(rng_l, M_, K_))
    nv_layers = [{k: (torch.from_numpy(v[0]).to(dev), torch.from_numpy(v[1]).to(dev)) for k, v in nv_host.items()}
                 for _ in range(8)]
    nv_w = sum(v[0].size + v[1].size for v in nv_host.values())
    del nv_host
    for n in (1, 2, 4, 8, 16, 32):
        rng_x = synthetic.rng_for(0, 3, 2, n)
        xn = torch.from_numpy(synthetic.activations(rng_x, n, 5120)).to(dev)
        xdn = torch.from_numpy(synthetic.activations(rng_x, n, 17408)).to(dev)
        qn = torch.empty((n, 7168), dtype=torch.float32, device=dev)
        hn = torch.empty((n, 17408), dtype=torch.float32, device=dev)
        rn = torch.from_numpy(synthetic.residual(rng_x, n, 5120)).to(dev)
        yn = torch.empty((n, 5120), dtype=torch.float32, device=dev)

        def nv_step(i):
            L = nv_layers[i % len(nv_layers)]
            qg.qgemv_ex("nvfp4", *L["qkv"], xn, qn, 7168, 5120, n, workspace=wsp)
            qg.qgemv_swiglu_ex("nvfp4", *L["gate_up"], xn, hn, 17408, 5120, n, workspace=wsp)
            qg.qgemv_ex("nvfp4", *L["down"], xdn, yn, 5120, 17408, n, residual=rn, workspace=wsp)
        ms = timeit(nv_step, 40)
        b = nv_w + n * (5120 * 2 + 7168 * 4 + 5120 * 2 + 17408 * 4 + 17408 * 2 + 5120 * 8)
        nv[f"N{n}"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                       "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 4),
                       "tok_per_s_64_layers": round(n / (64 * ms * 1e-3), 1)}
    del nv_layers
    res["nvfp4_layer"] = {"workload": "27B-class dense layer in NVFP4 (QKV, gate/up + SwiGLU, down + residual), "
                                      "8 rotated copies", "weight_bytes": nv_w, **nv}
    log("nvfp4_layer", res["nvfp4_layer"])

    # the same layer in MXFP4 on the block-scaled MFMA, N = 1, 8, 16, 32: x
    # quantised to MXFP8 on the device (qgemv_act_quant) for QKV and gate/up;
    # gate/up + SwiGLU hands h on as MXFP8 (qgemv_mx_swiglu_quant), which the
    # down projection reads
    mx_host = {}
    for name, M_, K_, _ in LAYER:
        rng_l = synthetic.rng_for(0, 3, 2, M_)
        mx_host[name] = qg.pack("mxfp4", synthetic.weights(rng_l, M_, K_))
    mx_layers = [{k: (torch.from_numpy(v[0]).to(dev), torch.from_numpy(v[1]).to(dev)) for k, v in mx_host.items()}
                 for _ in range(8)]
    mx_w = sum(v[0].size + v[1].size for v in mx_host.values())
    del mx_host
    mxr = {}
    for n in (1, 8, 16, 32):
        rng_x = synthetic.rng_for(0, 3, 3, n)
        xn = torch.from_numpy(synthetic.activations(rng_x, n, 5120)).to(dev)
        xq = torch.empty((n, 5120), dtype=torch.uint8, device=dev)
        xs = torch.empty((n, 5120 // 32), dtype=torch.uint8, device=dev)
        dq = torch.empty((n, 17408), dtype=torch.uint8, device=dev)
        dsc = torch.empty((n, 17408 // 32), dtype=torch.uint8, device=dev)
        qn = torch.empty((n, 7168), dtype=torch.float32, device=dev)
        rn = torch.from_numpy(synthetic.residual(rng_x, n, 5120)).to(dev)
        yn = torch.empty((n, 5120), dtype=torch.float32, device=dev)

        def mx_step(i):
            L = mx_layers[i % len(mx_layers)]
            qg.act_quant(xn, xq, xs, n, 5120)
            qg.qgemv_mx("mxfp4", *L["qkv"], xq, xs, qn, 7168, 5120, n)
            qg.qgemv_mx_swiglu_quant("mxfp4", *L["gate_up"], xq, xs, dq, dsc, 17408, 5120, n)
            qg.qgemv_mx("mxfp4", *L["down"], dq, dsc, yn, 5120, 17408, n, residual=rn)
        ms = timeit(mx_step, 40)
        # weights; x (bf16) read; MXFP8 x and h written and read; q, residual, y
        b = mx_w + n * 5120 * 2 + n * (5120 + 17408) * (1 + 1 / 32) * 2 + n * (7168 * 4 + 5120 * 8)
        mxr[f"N{n}"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                        "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 4),
                        "tok_per_s_64_layers": round(n / (64 * ms * 1e-3), 1)}
    del mx_layers
    res["mxfp4_layer"] = {"workload": "27B-class dense layer in MXFP4 with MXFP8 activations (x quantiser, QKV, "
                                      "gate/up + SwiGLU + MXFP8 quantisation of h, down + residual on that h), "
                                      "8 rotated copies",
                          "weight_bytes": mx_w, **mxr}
    log("mxfp4_layer", res["mxfp4_layer"])

    # the chained MLP block (timed eagerly in the main line) captured for 16
    # rotated layers in one HIP graph and replayed
    gamma = torch.from_numpy((1 + 0.1 * synthetic.rng_for(0, 7).standard_normal(5120)).astype(np.float32)).to(dev)
    r1 = torch.from_numpy(synthetic.residual(synthetic.rng_for(0, 7, 1), 1, 5120)).to(dev)
    hb = torch.zeros((1, 17408), dtype=torch.int16, device=dev)
    ym = torch.empty((1, 5120), dtype=torch.float32, device=dev)

    def mlp(i):
        L = layers[i % len(layers)]
        qg.qgemv_swiglu_ex("int5", *L["gate_up"], None, None, 17408, 5120, 1, norm_src=r1, norm_gamma=gamma,
                           norm_eps=1e-6, out_bf16=hb, workspace=wsp)
        qg.qgemv_ex("int5", *L["down"], hb, ym, 5120, 17408, 1, residual=r1, workspace=wsp)
    mlp_bytes = (weight_bytes(qg, "int5", 2 * 17408, 5120) + weight_bytes(qg, "int5", 5120, 17408)
                 + 5120 * 4 * 2 + 5120 * 4 + 17408 * 2 * 2 + 5120 * 8)
    nl = len(layers)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(nl):
            mlp(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(nl):
            mlp(i)
    ms_g = timeit(lambda i: graph.replay(), 8) / nl
    res["mlp_chain_graph"] = {"workload": "the chained MLP block of mlp_chain, 16 rotated layers in one HIP graph",
                              "graph_us_per_layer": round(ms_g * 1e3, 2),
                              "graph_GB/s": round(mlp_bytes / (ms_g * 1e-3) / 1e9, 1), "graph_layers": nl}
    del graph

    # the single-GEMV workload: M = K = 1024, int4, N = 1, seed 0 (fits the
    # L2 and the Infinity Cache: a launch-latency figure, not a roofline row)
    rng1 = np.random.default_rng(0)
    W1 = synthetic.weights(rng1, 1024, 1024)
    x1 = torch.from_numpy(synthetic.activations(rng1, 1, 1024)).to(dev)
    q1, s1 = (torch.from_numpy(a).to(dev) for a in qg.pack("int4", W1))
    y1 = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    ms1 = timeit(lambda i: qg.qgemv("int4", q1, s1, x1, y1, 1024, 1024, 1), 200)
    b1 = q1.numel() + s1.numel() + 1024 * 2 + 1024 * 4
    res["config1_int4_1024"] = {"workload": "single GEMV M=K=1024 int4, N=1, seed 0 (cache-resident)",
                                "us": round(ms1 * 1e3, 2), "GB/s": round(b1 / (ms1 * 1e-3) / 1e9, 1),
                                "algorithmic_bytes": b1}
    log("mlp_chain_graph", res["mlp_chain_graph"], "config1", res["config1_int4_1024"])

    # per format on [17408][5120], N = 1, 2, 4, 8 (int formats: also 16; MX: 16, 32), rotated over >= 1 GB
    M, K = 17408, 5120
    rng = synthetic.rng_for(0, 3, M)
    W = synthetic.weights(rng, M, K)
    pf = {}
    for fmt in ("int4", "int5", "int8", "nvfp4", "mxfp4", "mxfp8"):
        wq, ws = qg.pack(fmt, W)
        nb = wq.size + ws.size
        copies = max(2, int(np.ceil(1.2e9 / nb)))
        d = [(torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)) for _ in range(copies)]
        pf[fmt] = {}
        # plain streaming read of the same code buffers: the ceiling at this size
        ms = timeit(lambda i: qg.qgemv_probe_read(d[i % copies][0], wq.size // 16 * 16, sink), 60)
        probe_gbs = (wq.size // 16 * 16) / (ms * 1e-3) / 1e9
        pf[fmt]["probe_GB/s"] = round(probe_gbs, 1)
        ns = (1, 2, 4, 8, 16, 32) if fmt.startswith("mx") else (1, 2, 4, 8, 16)
        for n in ns:
            xb = torch.from_numpy(synthetic.activations(rng, n, K, 0.01)).to(dev)
            yy = torch.empty((n, M), dtype=torch.float32, device=dev)
            if fmt.startswith("mx"):
                # MXFP8 activations (qgemv_act_quant), then the block-scaled MFMA GEMV
                xq = torch.empty((n, K), dtype=torch.uint8, device=dev)
                xs = torch.empty((n, K // 32), dtype=torch.uint8, device=dev)
                qg.act_quant(xb, xq, xs, n, K)
                ms = timeit(lambda i: qg.qgemv_mx(fmt, *d[i % copies], xq, xs, yy, M, K, n), 60)
                ms2 = timeit(lambda i: (qg.act_quant(xb, xq, xs, n, K),
                                        qg.qgemv_mx(fmt, *d[i % copies], xq, xs, yy, M, K, n)), 60)
                b = nb + n * K + n * (K // 32) + n * M * 4
                gbs = b / (ms * 1e-3) / 1e9
                pf[fmt][f"N{n}"] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4),
                                    "of_probe": round(gbs / probe_gbs, 4), "us_with_act_quant": round(ms2 * 1e3, 2)}
                continue
            ms = timeit(lambda i: qg.qgemv_ex(fmt, *d[i % copies], xb, yy, M, K, n, workspace=wsp), 60)
            ms0 = timeit(lambda i: qg.qgemv(fmt, *d[i % copies], xb, yy, M, K, n), 60)
            b = nb + n * K * 2 + n * M * 4
            gbs = b / (ms * 1e-3) / 1e9
            pf[fmt][f"N{n}"] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4),
                                "of_probe": round(gbs / probe_gbs, 4), "us_no_workspace": round(ms0 * 1e3, 2)}
        if fmt == "int4":
            # the same calls with the batch-invariant summation order
            inv = {}
            for n in (1, 8):
                xb = torch.from_numpy(synthetic.activations(rng, n, K, 0.01)).to(dev)
                yy = torch.empty((n, M), dtype=torch.float32, device=dev)
                ms = timeit(lambda i: qg.qgemv_ex(fmt, *d[i % copies], xb, yy, M, K, n, batch_invariant=True), 60)
                inv[f"N{n}"] = {"us": round(ms * 1e3, 2), "GB/s": round((nb + n * K * 2 + n * M * 4) / (ms * 1e-3) / 1e9, 1)}
            pf[fmt]["batch_invariant"] = inv
        del d
        log("per_format", fmt, pf[fmt])
    res["per_format"] = {"shape": [M, K], "formats": pf}
    del W

    # MoE: 128 experts, H 2048, I 768, top-8, int4, N = 1 and 8
    E, H, I, k = 128, 2048, 768, 8
    sq, ss = qg.expert_stride("int4", 2 * I, H)
    dq, ds = qg.expert_stride("int4", H, I)
    bufs = [np.zeros(E * sq, np.uint8), np.zeros(E * ss, np.uint8), np.zeros(E * dq, np.uint8), np.zeros(E * ds, np.uint8)]
    rng = synthetic.rng_for(0, 5)
    for e in range(E):
        q, s = qg.pack("int4", synthetic.weights(rng, 2 * I, H))
        bufs[0][e * sq: e * sq + q.size] = q
        bufs[1][e * ss: e * ss + s.size] = s
        q, s = qg.pack("int4", synthetic.weights(rng, H, I))
        bufs[2][e * dq: e * dq + q.size] = q
        bufs[3][e * ds: e * ds + s.size] = s
    copies = 32
    dbufs = [[torch.from_numpy(b).to(dev) for b in bufs] for _ in range(copies)]
    per_expert = (sq + ss + dq + ds)
    moe = {}
    for n in (1, 4, 8):
        logits = synthetic.router_logits(rng, n, E)
        ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)
        g = np.exp(np.take_along_axis(logits.astype(np.float64), ids, 1))
        gates = (g / g.sum(1, keepdims=True)).astype(np.float32)
        uniq = len(set(ids.reshape(-1).tolist()))
        xb = torch.from_numpy(synthetic.activations(rng, n, H)).to(dev)
        idt = torch.from_numpy(ids).to(dev)
        gt = torch.from_numpy(gates).to(dev)
        nbytes = qg.moe_workspace_bytes(E, H, I, n, k)
        wsp = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        yy = torch.empty((n, H), dtype=torch.float32, device=dev)
        ms = timeit(lambda i: qg.qgemv_moe("int4", *dbufs[i % copies], E, H, I, xb, idt, gt, k, yy, n, wsp, nbytes), 60)
        b = uniq * per_expert + n * H * 2 + n * H * 4 + n * k * 8
        moe[f"N{n}"] = {"active_experts": uniq, "us": round(ms * 1e3, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1)}
    res["moe"] = {"workload": "128 experts, H 2048, I 768, top-8, int4, 32 rotated copies", **moe}
    log("moe", res["moe"])

    # the same MoE routed on the device (qgemv_moe_fused), with 16 seeded
    # logit sets in rotation so the routing changes every call;
    # algorithmic bytes: the selected experts' weights + x + logits + r + y
    fused = {}
    for n in (1, 2, 4, 8):
        sets = [synthetic.router_logits(rng, n, E) for _ in range(16)]
        uniq = [len({int(e) for e in np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k].reshape(-1)})
                for lg in sets]
        lt = [torch.from_numpy(lg).to(dev) for lg in sets]
        xb = torch.from_numpy(synthetic.activations(rng, n, H)).to(dev)
        rr = torch.from_numpy(synthetic.residual(rng, n, H)).to(dev)
        nbytes = qg.moe_fused_workspace_bytes(E, H, I, n, k)
        wsp = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        yy = torch.empty((n, H), dtype=torch.float32, device=dev)
        ms = timeit(lambda i: qg.qgemv_moe_fused("int4", *dbufs[i % copies], E, H, I, xb, lt[i % 16], k, yy, n, wsp,
                                                 nbytes, residual=rr), 64)
        b = float(np.mean(uniq)) * per_expert + n * H * 2 + n * E * 4 + n * H * 8
        fused[f"N{n}"] = {"mean_active_experts": round(float(np.mean(uniq)), 2), "us": round(ms * 1e3, 2),
                          "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 4)}
        err = int(wsp[12:16].cpu().view(torch.int32).item())
        if err:
            raise RuntimeError("qgemv_moe_fused reported a timed-out dependency wait")
    res["moe_fused"] = {"workload": "128 experts, H 2048, I 768, top-8 routed on the device from fresh logits, int4 "
                                    "(qgemv_moe_fused: one launch at N = 1, router + 3 launches above), "
                                    "32 rotated copies", **fused}
    log("moe_fused", res["moe_fused"])
    return res


def cpu_baseline(seconds: float):
    """The oracle (dequantise to fp64 + numpy matmul on all host cores) on a
    sample of the layer: whole row tiles of each matrix, repeated for about
    `seconds`; reported as GB/s over the same algorithmic bytes."""
    from oracle import gemv as G
    from oracle import layout, quant
    from oracle.dequant import dequant
    import synthetic

    rng = synthetic.rng_for(0, 6)
    parts = []
    for name, M, K, fmt in LAYER:
        rows = 256
        W = synthetic.weights(rng, rows, K)
        wq, ws = layout.pack(quant.quantize(W, fmt))
        parts.append((fmt, rows, K, wq, ws, sum(layout.packed_bytes(fmt, rows, K)) + K * 2 + rows * 4))
    x = {K: G.x_from_bits(synthetic.activations(rng, 1, K)) for K in (5120, 17408)}
    done, nbytes, t0 = 0, 0, time.perf_counter()
    while True:
        for fmt, rows, K, wq, ws, b in parts:
            Wd = dequant(layout.unpack(fmt, rows, K, wq, ws))
            G.gemv(x[K], Wd)
            nbytes += b
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": blas or cores, "kind": "oracle",
            "host_cores_visible": cores,
            "sample": f"{done} passes over 256-row slices of the three layer matrices (unpack + dequantise to fp64 "
                      f"single-threaded, numpy matmul on {blas} BLAS threads, N=1), {el:.1f} s"}


if __name__ == "__main__":
    main()
