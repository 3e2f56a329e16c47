"""Benchmark of the error-compensated W4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]

Default workload (config c3): the 70B-shaped MLP down-projection
(d_in = 28672, d_out = 8192, int4 group-wise g = 128 asymmetric with fp16
scales and int4 zero-points, compensator rank 64).  One step is the mixed
phase of chunked-prefill serving: a 16-token decode batch and a 512-token
prefill chunk, both through the phase-aware dispatcher (spear_ec_linear), on
one stream.  Decode runs first, so it streams its weights from HBM; weights
rotate over several copies so no call finds them in the 256 MB last-level
cache from an earlier step.  Inputs are seeded synthetic tensors of the
workload's shapes and distributions, resident in HBM before timing starts.

Timing.  The K timed steps run back to back between two events
(ms_per_step).  Then each call of the step is timed on its own: the same
call launched K times back to back between two events on the launch stream,
rotating the weight copies (its mean duration: the kernel time plus the
launch gap, what a kernel trace of the same run averages), and once more with
an event pair around every launch (p10/p50/p90; these include the events' own
overhead of a few microseconds).  Each timed batch is queued behind a spin
kernel long enough for the host to enqueue the whole batch first, so the
host's launch overhead never leaves the GPU idle inside a timed interval.

Reported (one JSON line):
  value        decode effective bandwidth: algorithmic bytes of the decode
               call / its mean duration (GB/s); prefill TFLOP/s alongside.
  roofline     for the dominant call (prefill, matrix cores) and, under
               roofline_decode, for the decode call (HBM).
  cpu_baseline the single-threaded fp64 oracle on a row slice of the same
               layer (all tokens, a subset of output rows), scaled to GB/s.

Algorithmic bytes of a call = packed weights + scales + zeros + A + B + g + b
+ x + y, each once.  Algorithmic flops = 2TKN + 2Tr(K + N) + 4Tr.
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

METRIC = "decode: effective HBM GB/s (% peak); prefill: TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def layer_bytes(K, N, r, g, asym, T, serq=False):
    G = K // g
    w = N * K // 2 + N * G * 2 + (N * ((G + 7) // 8) * 4 if asym else 0)
    # SPEAR: A, B, g, b; SERQ: R only (its k salient channels come from x)
    comp = N * r * 2 if serq else r * K * 2 + N * r * 2 + 2 * r * 4
    return w + comp + T * K * 2 + T * N * 2


def weight_bytes(K, N, r, g, asym):
    G = K // g
    return N * K // 2 + N * G * 2 + (N * ((G + 7) // 8) * 4 if asym else 0) + r * K * 2 + N * r * 2


def layer_flops(K, N, r, T, serq=False):
    if serq:  # W4 product + the k-channel reconstruction
        return 2 * T * K * N + 2 * T * r * N
    return 2 * T * K * N + 2 * T * r * (K + N) + 4 * T * r


def _code_only(src):
    """C++ source with its comments removed and blank runs collapsed, so that
    a change to comments alone leaves the hash (and the measurements tied to
    it) in place."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the kernel sources' code (comments and layout excluded)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantization_error_compensation_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


WORKLOADS = {
    "c3": dict(steps=[("decode", 16), ("prefill", 512)],
               text="70B MLP down-projection d_in=28672 d_out=8192, int4 g=128 asymmetric "
                    "(fp16 scales, int4 zero-points), rank 64; mixed step = 16-token decode + "
                    "512-token prefill chunk through the dispatcher"),
    "c1": dict(steps=[("decode", 1), ("decode", 8), ("decode", 32)],
               text="7B attention projection d_in=d_out=4096, int4 g=128 asymmetric, rank 32; "
                    "decode batches of 1, 8 and 32 tokens"),
    "c2": dict(steps=[("prefill", 2048)],
               text="7B MLP up-projection d_in=4096 d_out=11008, int4 symmetric per-channel, "
                    "rank 64; 2048-token prefill"),
    "c4": dict(steps=[("decode", 1), ("decode", 16), ("prefill", 256), ("prefill", 4096)],
               text="d_in=d_out=8192 sweep point, int4 symmetric per-channel, rank 128; tokens "
                    "1, 16, 256, 4096"),
    "v1": dict(steps=[("decode", 9)],
               text="Quasar-shaped verify pass: d_in=d_out=8192, int4 symmetric per-tensor, no "
                    "compensator (rank 0); 9 tokens (8 drafted + 1)"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--rank", type=int, default=None, help="override the compensator rank")
    ap.add_argument("--mlp-gate", type=int, default=0, metavar="H",
                    help="use the bottleneck-MLP gate of width H (0: the elementwise gate)")
    ap.add_argument("--serq", type=int, default=0, metavar="K",
                    help="SERQ single-matrix reconstruction of K salient channels (the first K "
                         "after the permutation) instead of the SPEAR compensator")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--sweep", action="store_true",
                    help="rank sweep: run the config's calls at every rank of the nested "
                         "compensator draws (0, 16, 64, 128) and report t(r)/t(0) - 1 per call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: read the counter CSVs of two rocprofv3 --pmc runs of this "
                         "script (FETCH_SIZE, then WRITE_SIZE, both with --copy-calibration) and "
                         "write profiles/traffic_<config>.json")
    return ap.parse_args()


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        rank_sweep(args)
        return

    import torch

    import quantization_error_compensation_amd as q
    import synth

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import to_dev_bf16, to_dev_f32

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.load_library()

    spec = synth.CONFIGS[args.config]
    K, N, g, asym = spec.d_in, spec.d_out, spec.group_size, spec.asym
    r = spec.rank if args.rank is None else args.rank
    serq = args.serq > 0
    if serq:
        r = args.serq
    plan = WORKLOADS[args.config]["steps"]
    Tmax = max(T for _, T in plan)
    Ttot = sum(T for _, T in plan)

    t_setup = time.time()
    W = synth.weights(spec)
    X = synth.serq_activations(spec, Ttot) if serq else synth.activations(spec, Ttot)
    A, B, gv, bv = synth.compensator(spec, r)
    if serq:  # R in B's place; no A, g, b
        B = synth.serq_matrix(spec, r)
    mlp = synth.mlp_gate(spec, r, args.mlp_gate) if args.mlp_gate and r else None
    desc = q.make_desc(K, N, r, g, asym, spec.per_tensor)
    wq0, sc0, zs0 = q.alloc_packed(desc, dev)
    q.spear_ec_quantize_rtn(desc, to_dev_f32(W, dev), wq0, sc0, zs0)
    torch.cuda.synchronize()
    del W
    wbytes = weight_bytes(K, N, r, g, asym)
    copies = args.copies or max(2, int(np.ceil(1.0e9 / wbytes)))
    layers = []
    for c in range(copies):
        layers.append(dict(
            wq=wq0.clone(), sc=sc0.clone(), zs=zs0.clone() if zs0 is not None else None,
            A=to_dev_bf16(A, dev) if r else None, B=to_dev_bf16(B, dev) if r else None,
            g=to_dev_f32(gv, dev) if r else None, b=to_dev_f32(bv, dev) if r else None,
            mlp={k: to_dev_f32(v, dev) for k, v in mlp.items()} if mlp else None))
    xs, ys, off = [], [], 0
    for _, T in plan:
        xs.append(to_dev_bf16(X[off:off + T], dev))
        ys.append(torch.empty((T, N), dtype=torch.bfloat16, device=dev))
        off += T
    ws = q.alloc_workspace(desc, Tmax, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    stream = torch.cuda.current_stream()

    def call(j, i):
        """Call j of the step on weight copy i (mod copies)."""
        L = layers[i % copies]
        if serq:
            q.spear_ec_linear_serq(desc, xs[j], L["wq"], L["sc"], L["zs"], 0, L["B"], ys[j], ws,
                                   stream)
        elif L["mlp"] is not None:
            m = L["mlp"]
            q.spear_ec_linear_mlp_gate(desc, xs[j], L["wq"], L["sc"], L["zs"], L["A"], L["B"],
                                       m["w1"], m["b1"], m["w2"], m["b2"], spec.alpha, ys[j], ws,
                                       stream)
        else:
            q.spear_ec_linear(desc, xs[j], L["wq"], L["sc"], L["zs"], L["A"], L["B"], L["g"],
                              L["b"], spec.alpha, ys[j], ws, stream)

    def step(i):
        for j in range(len(plan)):
            call(j, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    n = len(plan)
    # host enqueue time per call, and the spin kernel's rate, to size the
    # spin that holds the GPU while a timed batch is enqueued
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    host_s = (time.perf_counter() - h0) / max(1, args.warmup * n)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1 << 22)
    c1.record(stream)
    torch.cuda.synchronize()
    spin_s_per_cycle = c0.elapsed_time(c1) / 1e3 / (1 << 22)

    def hold(launches):
        """Keep the stream busy while `launches` calls are enqueued."""
        need = 2.0 * launches * host_s + 1e-3
        torch.cuda._sleep(int(need / max(spin_s_per_cycle, 1e-12)))

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold(args.steps * n)
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps

    # each call alone: K launches back to back (mean), then K launches each
    # between its own events (distribution)
    per_call_ms, call_ms = [], []
    for j in range(n):
        for i in range(args.warmup):
            call(j, args.warmup + i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        hold(args.steps)
        e0.record(stream)
        for i in range(args.steps):
            call(j, i)
        e1.record(stream)
        torch.cuda.synchronize()
        per_call_ms.append(e0.elapsed_time(e1) / args.steps)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        hold(args.steps * 2)
        for i in range(args.steps):
            evs[i][0].record(stream)
            call(j, i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        call_ms.append(np.array([a.elapsed_time(b) for a, b in evs]))

    calls = []
    for j, (path, T) in enumerate(plan):
        by = layer_bytes(K, N, r, g, asym, T, serq)
        fl = layer_flops(K, N, r, T, serq)
        s = per_call_ms[j] / 1e3
        p10, p50, p90 = (float(v) for v in np.percentile(call_ms[j], [10, 50, 90]))
        calls.append(dict(path=path, tokens=T, ms=per_call_ms[j], p10_ms=p10, p50_ms=p50,
                          p90_ms=p90, bytes=by, flops=fl, gbs=by / s / 1e9, tflops=fl / s / 1e12))
        assert q.spear_ec_workspace_status(ws) == 0, "a decode wait gave up during the run"

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.uint8, device=dev)   # 256 MiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    dec = [c for c in calls if c["path"] == "decode"]
    pre = [c for c in calls if c["path"] == "prefill"]
    dominant = max(calls, key=lambda c: c["ms"])
    # the stored counter figures are for the default elementwise-gate layer
    traffic = {} if (serq or mlp) else load_traffic(args.config)

    def roof(c):
        if c["path"] == "decode":
            return {"bound": "hbm", "achieved": round(c["gbs"], 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(c["gbs"] / HBM_PEAK_GBS, 4),
                    "traffic": traffic.get(f"decode_T{c['tokens']}"),
                    "kernel": f"decode_kernel: the whole decode call ({c['tokens']} tokens) is this one launch",
                    "avg_us": round(c["ms"] * 1e3, 2),
                    "timing": "mean of back-to-back launches between two events on the launch stream"}
        return {"bound": "mfma", "achieved": round(c["tflops"], 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(c["tflops"] / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic.get(f"prefill_T{c['tokens']}"),
                "kernel": f"prefill call ({c['tokens']} tokens): " + PREFILL_KERNELS_TEXT,
                "avg_us": round(c["ms"] * 1e3, 2),
                "timing": "mean of back-to-back calls between two events on the launch stream"}

    head = dec[0] if dec else pre[0]
    value = head["gbs"] if dec else head["tflops"]
    unit = "GB/s" if dec else "TFLOP/s"
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: " + WORKLOADS[args.config]["text"],
                   "d_in": K, "d_out": N, "rank": r, "group_size": g,
                   "zero_points": asym, "per_tensor": spec.per_tensor,
                   "gate": (f"SERQ, {r} salient channels" if serq else
                            f"bottleneck MLP, hidden {args.mlp_gate}" if mlp else "elementwise"),
                   "tokens_per_step": [T for _, T in plan],
                   "weight_copies_rotated": copies, "parallelism": "single GPU"},
        "calls": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items()}
                  for c in calls],
        "roofline": roof(dominant),
    }
    if dec and pre:
        out["prefill"] = {"value": round(pre[0]["tflops"], 2), "unit": "TFLOP/s",
                          "frac_of_peak": round(pre[0]["tflops"] / BF16_PEAK_TFLOPS, 4)}
        out["roofline_decode"] = roof(dec[0])
    out["host_enqueue_us_per_call"] = round(host_s * 1e6, 1)
    out["kernel_source_hash"] = kernel_source_hash()
    out["setup_s"] = round(setup_s, 1)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, r, plan, X, A, B, gv, bv, unit, mlp, serq)
    print(json.dumps(out), flush=True)


def rank_sweep(args):
    """Each rank of the nested draws in a child process of its own (this
    process never touches the GPU); per call, the time relative to rank 0 and
    the compensator's bytes relative to the W4 layer's, 2r(K+N) / (KN/2 +
    scales + zeros)."""
    import subprocess

    import synth
    spec = synth.CONFIGS[args.config]
    K, N, g, asym = spec.d_in, spec.d_out, spec.group_size, spec.asym
    runs = {}
    for r in (0, 16, 64, 128):
        cmd = [sys.executable, os.path.abspath(__file__), "--config", args.config, "--rank", str(r),
               "--steps", str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline"]
        if args.copies:
            cmd += ["--copies", str(args.copies)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode:
            sys.stderr.write(res.stderr)
            sys.exit(res.returncode)
        runs[r] = json.loads(res.stdout.strip().splitlines()[-1])
        print(f"rank {r}: " + ", ".join(f"{c['path']} T={c['tokens']} {c['ms'] * 1e3:.2f} us"
                                        for c in runs[r]["calls"]), file=sys.stderr, flush=True)
    w4 = weight_bytes(K, N, 0, g, asym)
    table = []
    for r, run in runs.items():
        for c, c0 in zip(run["calls"], runs[0]["calls"]):
            table.append({"rank": r, "path": c["path"], "tokens": c["tokens"],
                          "us": round(c["ms"] * 1e3, 2), "p50_us": round(c["p50_ms"] * 1e3, 2),
                          "rel_to_rank0": round(c["ms"] / c0["ms"] - 1.0, 4),
                          "ec_bytes_over_w4": round(2 * r * (K + N) / w4, 4)})
    print(json.dumps({"metric": "rank sweep: call time relative to rank 0 (t(r)/t(0) - 1)",
                      "config": args.config, "steps": args.steps, "warmup": args.warmup,
                      "weight_copies_rotated": runs[0]["config"]["weight_copies_rotated"],
                      "kernel_source_hash": kernel_source_hash(), "sweep": table}), flush=True)


CALIB_BYTES = 1 << 28   # the --copy-calibration copy: 256 MiB read, 256 MiB written
PREFILL_KERNELS_TEXT = "projection_kernel + finish_kernel + prefill_kernel, timed together"

# Kernels of each call of the dispatcher (matched against the mangled names).
CALL_KERNELS = {"decode": ("decode_kernel",),
                "prefill": ("projection_kernel", "finish_kernel", "prefill_kernel")}


def read_counter_csv(d, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc run written
    with --output-format csv: [(kernel_name, grid_size, value), ...]."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0),
                                 float(r["Counter_Value"])))
    return rows


def write_traffic(args):
    """HBM bytes per call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the 256 MiB calibration
    copy, averaged over the dispatches of each kernel of the call."""
    spec_plan = WORKLOADS[args.config]["steps"]
    out = {"config": args.config, "kernel_source_hash": kernel_source_hash(),
           "calibration_bytes": CALIB_BYTES, "bytes_per_call": {}, "counters": {}}
    per_kernel = {}
    for d, counter in zip(args.traffic_from, ("FETCH_SIZE", "WRITE_SIZE")):
        rows = read_counter_csv(d, counter)
        copies = [v for k, g, v in rows if "copy" in k.lower() or "elementwise" in k.lower()]
        if not copies:
            raise SystemExit(f"{counter}: no copy kernel found for the calibration")
        factor = CALIB_BYTES / (max(copies) * 1024.0)
        out["counters"][counter] = {"calibration_kib": max(copies), "scale": factor}
        for path, names in CALL_KERNELS.items():
            for nm in names:
                vals = [v for k, g, v in rows if nm in k]
                if vals:
                    per_kernel.setdefault(nm, {})[counter] = float(np.mean(vals)) * 1024.0 * factor
    for path, T in spec_plan:
        tot = 0.0
        for nm in CALL_KERNELS[path]:
            if nm in per_kernel:
                tot += per_kernel[nm].get("FETCH_SIZE", 0.0) + per_kernel[nm].get("WRITE_SIZE", 0.0)
        out["bytes_per_call"][f"{path}_T{T}"] = round(tot)
    out["bytes_per_kernel"] = {k: {c: round(v) for c, v in d.items()} for k, d in per_kernel.items()}
    dst = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def load_traffic(config):
    """HBM traffic per call measured with rocprofv3 counters, if it was taken
    on the current kernel sources (profiles/traffic_<config>.json)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return {}
    return t.get("bytes_per_call", {})


def cpu_baseline(spec, r, plan, X, A, B, gv, bv, unit, mlp=None, serq=False):
    """The fp64 oracle on a bounded sample of the same layer: every token of
    the first call of the step, a slice of output rows.  Scaled to the unit
    of `value` by the algorithmic bytes (or flops) of that slice."""
    import oracle
    K, N, g, asym = spec.d_in, spec.d_out, spec.group_size, spec.asym
    path, T = plan[0]
    x = X[:T]
    # the slice: a few seconds of single-core work
    rows = max(16, min(N, int(6.0e9 / max(1, T * K))))
    import synth
    Wsl = synth.weights(spec, rows=rows)
    t0 = time.time()
    wq, sc, zs = oracle.quantize_rtn_per_tensor(Wsl) if spec.per_tensor else oracle.quantize_rtn(Wsl, g, asym)
    t1 = time.time()
    if serq:
        oracle.forward_serq(x, wq, sc, zs, 0, B[:rows], g)
    else:
        oracle.forward(x, wq, sc, zs, A if r else None, B[:rows] if r else None, gv, bv,
                       spec.alpha, g, mlp=mlp)
    t2 = time.time()
    secs = t2 - t1
    by = layer_bytes(K, rows, r, g, asym, T, serq)
    fl = layer_flops(K, rows, r, T, serq)
    val = by / secs / 1e9 if unit == "GB/s" else fl / secs / 1e12
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(val, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": model,
            "sample": f"{path} call, all {T} tokens x first {rows} of {N} output rows "
                      f"(compensator for all tokens); forward {secs:.1f} s, quantize {t1 - t0:.1f} s"}


if __name__ == "__main__":
    main()
