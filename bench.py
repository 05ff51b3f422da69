"""Benchmark of the routed MoE FFN layer (libmoe) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A step is one pass of the whole layer -- router logits + top-k, sort by
expert, grouped gate/up + SwiGLU, grouped down projection, (shared expert),
weighted combine -- over one resident batch of synthetic inputs.  Prints
one JSON line: layer tokens/s for the workload, the roofline position of
its dominant kernel (timed with HIP events on the launch stream), and the
CPU oracle timed on a bounded sample of the same workload.

The default workload is the Mixtral-shaped prefill layer (T=4096, d=4096,
f=14336, E=8, top-2, bf16).  The other workloads (c3_t1 ... c3_t64 decode,
c4, c5) can be selected with --workload; decode workloads evict the caches
between steps and are timed per step with events.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import moe_workloads as W  # noqa: E402

METRIC = "MoE layer tokens/s + % peak bf16 MFMA (prefill) / % peak HBM GB/s (decode)"

# MI355X published peaks (dense, no sparsity)
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0

KERNEL_SOURCES = {
    "gateup": ["gemm_bf16.hip", "grouped_gemm.h", "common.h"],
    "decode_gateup": ["decode.hip", "common.h"],
}


# ------------------------------------------------------------ accounting

def decode_tokens_per_s(bandwidth_bytes_per_s: float, active_params: float, bytes_per_param: float) -> float:
    """Bandwidth model of decode speed: every generated token reads every
    active parameter once, so tokens/s ~ bandwidth / (active params x bytes
    per param)."""
    return bandwidth_bytes_per_s / (active_params * bytes_per_param)


def layer_flops(wl) -> float:
    """Algorithmic FLOPs of one layer call: router + 3 expert GEMMs per
    routed pair (+ the shared expert on every token)."""
    return (2.0 * wl.T * wl.d * wl.E + 6.0 * wl.T * wl.k * wl.d * wl.f
            + 6.0 * wl.T * wl.d * wl.f_shared)


def layer_bytes(wl, active: int) -> float:
    """Algorithmic HBM bytes of one layer call: each active expert's weights
    once, the router weights, x read and y written once (+ shared expert)."""
    b = wl.elem_bytes
    return b * (3.0 * wl.d * wl.f * active + wl.d * wl.E + 2.0 * wl.T * wl.d + 3.0 * wl.d * wl.f_shared)


def gateup_flops(wl) -> float:
    """Grouped gate/up projection: 2 x (2f) x d FLOPs per routed row."""
    return 4.0 * wl.P * wl.d * wl.f


def gateup_bytes(wl, active: int) -> float:
    """Gate/up kernel: active experts' [2f, d] weights + routed rows in + H out."""
    b = wl.elem_bytes
    return b * (2.0 * wl.f * wl.d * active + wl.P * wl.d + wl.P * wl.f)


def tile_work(wl, counts) -> dict:
    """MFMA work the grouped tile kernels issue, as a multiple of the
    algorithmic work of each routed projection.  Rows are covered in 32-row
    fragments (a fragment holding no row of its expert is skipped), columns
    in whole output tiles (128 SwiGLU outputs for gate/up, 256 for down).
    Padding each expert to whole 256-row tiles is given for comparison."""
    c = np.asarray(counts, np.int64)
    c = c[c > 0]
    P = int(c.sum())
    if P == 0:
        return {"gateup": None, "down": None, "rows_at_256_row_tiles": None}
    r32 = int((-(-c // 32) * 32).sum())
    r256 = int((-(-c // 256) * 256).sum())
    return {"gateup": r32 / P * (-(-wl.f // 128) * 128) / wl.f,
            "down": r32 / P * (-(-wl.d // 256) * 256) / wl.d,
            "rows_at_256_row_tiles": r256 / P}


# ------------------------------------------------------------ setup

def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "mixture_experts_ffn_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from the rocprofv3 counter summary under
    profiles/, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def setup(wl, device):
    import torch
    from mixture_experts_ffn_04_amd import MoeLayer, MoeWeights

    def dev(a, shape=None):
        if wl.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        return t if shape is None else t.view(shape)

    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = W.gen_x(wl)
    wr, bias = W.gen_router(wl)
    gu = torch.empty(wl.E, 2 * wl.f, wl.d, dtype=tdt, device=device)
    dn = torch.empty(wl.E, wl.d, wl.f, dtype=tdt, device=device)
    host_experts = {}
    keep = wl.E * 3 * wl.d * wl.f * wl.elem_bytes <= (4 << 30)
    for e, g, w in W.iter_experts(wl):
        gu[e].copy_(dev(g))
        dn[e].copy_(dev(w))
        if keep:
            host_experts[e] = (g, w)
    sh = W.gen_shared(wl)
    weights = MoeWeights(dev(wr), None if bias is None else torch.from_numpy(bias).to(device), gu, dn,
                         None if sh is None else dev(sh[0]), None if sh is None else dev(sh[1]))
    layer = MoeLayer(weights, wl.k, wl.score)
    host = dict(x=x, wr=wr, bias=bias, experts=host_experts, shared=sh)
    return layer, dev(x), host


# ------------------------------------------------------------ CPU oracle

def cpu_baseline(wl, host, sample_tokens: int, target_s: float = 15.0):
    """Time the CPU oracle (router + eager expert loop, float64) on the first
    `sample_tokens` tokens of the workload; when that takes well under
    target_s seconds, time it again on enough tokens (at most T) to take
    about target_s.  Input generation is excluded; decoding the stored bf16
    values for the oracle is included."""
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    S = min(sample_tokens, wl.T)
    experts = host["experts"]

    def fetch(e):
        if e in experts:
            g, w = experts[e]
        else:
            g, w = W.gen_expert(wl, e)
        return W.values(g, wl.dtype), W.values(w, wl.dtype)

    def run(S):
        t0 = time.perf_counter()
        x = W.values(host["x"][:S], wl.dtype)
        L = O.router_logits(x, W.values(host["wr"], wl.dtype), host["bias"])
        ids, w = O.route(L, wl.k, wl.score)
        sh = host["shared"]
        shared = None if sh is None else (W.values(sh[0], wl.dtype), W.values(sh[1], wl.dtype))
        O.moe_layer_eager(x, ids, w, fetch, wl.E, shared)
        return time.perf_counter() - t0, ids

    dt, ids = run(S)
    if target_s and dt < 0.5 * target_s and S < wl.T:
        # a bounded sample of about target_s seconds of CPU work
        S = min(wl.T, max(S + 1, int(S * target_s / dt)))
        dt, ids = run(S)
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {S} of {wl.T} tokens of workload {wl.name}: float64 router + eager "
                      f"per-expert loop over the {len(np.unique(ids))} experts they select; "
                      f"{dt:.1f} s wall"}


# ------------------------------------------------------------ profiles

def copy_probe(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of known size (torch's copy kernel), to
    calibrate what the HBM byte counters read for a known amount of data."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def _smi_sample():
    """One amd-smi reading: socket power (W) and the gfx clocks (MHz) of the
    XCDs, or None where amd-smi is missing."""
    import csv
    import io
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--csv"], capture_output=True, text=True,
                             timeout=20).stdout
        row = list(csv.DictReader(io.StringIO(out.strip())))[0]
    except (OSError, subprocess.SubprocessError, IndexError, ValueError):
        return None
    clk = [float(row[k]) for k in row if k.startswith("gfx_") and k.endswith("_clk") and k[4:-4].isdigit()
           and row[k] not in ("N/A", "")]
    try:
        power = float(row.get("socket_power", "nan"))
    except ValueError:
        power = float("nan")
    return {"power_w": power, "gfx_clk_mhz": clk}


def clock_probe(workload: str, seconds: float, command: str, out: str):
    """Run the dominant kernel (gate/up) back to back for `seconds` while
    sampling the reported gfx clocks and socket power, then the same for
    torch.matmul (hipBLASLt) on the same work -- one product per expert with
    that expert's rows and weights -- and on one dense product of the same
    P x d x 2f size (a single weight matrix, so 1/E of the weight bytes), and
    write a markdown summary: the achieved TFLOP/s next to the clock."""
    import threading
    import torch
    wl = W.get(workload)
    layer, x, _ = setup(wl, torch.device("cuda:0"))
    layer.forward(x)
    torch.cuda.synchronize()
    L = layer
    flops = gateup_flops(wl)

    st = torch.cuda.current_stream()
    gate_stage = [a for n, fn, a in L.stages(x, st) if n == "gateup"][0]
    gate_fn = [fn for n, fn, a in L.stages(x, st) if n == "gateup"][0]

    def gate():
        gate_fn(*gate_stage)

    P = wl.T * wl.k
    a = torch.randn(P, wl.d, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(wl.d, 2 * wl.f, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(P, 2 * wl.f, dtype=torch.bfloat16, device="cuda")
    offs = L.offsets.cpu().numpy()
    wgu = L.w.w_gate_up
    groups = [(e, int(offs[e]), int(offs[e + 1])) for e in range(len(offs) - 1) if offs[e + 1] > offs[e]]

    def dense():
        torch.matmul(a, b)

    def per_expert():
        for e, lo, hi in groups:
            torch.matmul(a[lo:hi], wgu[e].t(), out=y[lo:hi])

    rows = []
    for name, fn in (("libmoe gate/up (grouped, fused SwiGLU)", gate),
                     ("torch.matmul (hipBLASLt), one product per expert", per_expert),
                     ("torch.matmul (hipBLASLt), one dense P x d x 2f product", dense)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        samples, stop = [], []

        def sampler():
            while not stop:
                r = _smi_sample()
                if r is not None:
                    samples.append(r)
                time.sleep(0.25)

        th = threading.Thread(target=sampler)
        th.start()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, t0 = 0, time.time()
        e0.record()
        while time.time() - t0 < seconds:
            for _ in range(10):
                fn()
            n += 10
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        stop.append(1)
        th.join()
        ms = e0.elapsed_time(e1) / n
        clk = [float(np.mean(s["gfx_clk_mhz"])) for s in samples[1:] if s["gfx_clk_mhz"]]
        pw = [s["power_w"] for s in samples[1:]]
        rows.append((name, ms, flops / (ms * 1e-3) / 1e12, float(np.median(clk)) if clk else float("nan"),
                     float(np.median(pw)) if pw else float("nan"), len(samples)))
    lines = [f"# Clock and power under load: gate/up on workload {workload}", "", "Command:", "", "```", command,
             "```", "",
             "| kernel | ms per launch | TFLOP/s | median gfx clock (MHz, mean over XCDs) | median socket power (W) | samples |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r[0]} | {r[1]:.3f} | {r[2]:.0f} | {r[3]:.0f} | {r[4]:.0f} | {r[5]} |")
    lines += ["", "Dense bf16 peak at the measured clock = 2.5 PFLOP/s x clock / 2400 MHz.  The per-expert products do "
              "the same work as the grouped kernel (without the fused SwiGLU and row gather); the dense product "
              "reads one weight matrix instead of E."]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_trace(d: str, title: str, command: str, out: str, log: str = None):
    """rocprofv3 --kernel-trace --stats CSV -> a short markdown table, with the
    median of each kernel's dispatch durations from the per-dispatch trace.
    With `log` (the profiled bench.py run's output), the bench's own figure
    for its roofline kernel from the same run is quoted as well."""
    rows = _read_csv(_find(d, "kernel_stats.csv"))
    durs = {}
    for r in _read_csv(_find(d, "kernel_trace.csv")):
        durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "Part `layer` is libmoe's kernels.  Part `harness` is the benchmark's own work outside the timed "
             "steps: weight uploads and read-backs (`copyBuffer`), buffer fills, and the cache-flush read "
             "between decode steps (`reduce_kernel`).  The averages include the warm-up calls and the "
             "untimed per-stage pass; the medians are over all dispatches.", ""]
    if log:
        rec = None
        for line in open(log, errors="replace"):
            if line.startswith("{") and '"roofline"' in line:
                rec = json.loads(line)
        if rec is not None:
            r = rec["roofline"]
            lines += [f"bench.py in the same run: `{r['kernel']}` {r['kernel_ms'] * 1e3:.1f} us per call "
                      f"(HIP events on the launch stream over the timed steps), {rec['ms_per_step']:.3f} ms per "
                      f"step, {rec['value']:.4g} {rec['unit']}.", ""]
    lines += ["| kernel | part | calls | avg us | median us | min us | max us | total % |",
              "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        part = "layer" if "moe::" in name else "harness"
        med = float(np.median(durs[name])) / 1e3 if name in durs else float("nan")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {part} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | {med:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def _pmc_by_kernel(d: str):
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _read_csv(_find(d, "counter_collection.csv")):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return acc


def summarize_traffic(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                      kernel_match: str, kernel: str, workload: str, copy_bytes: int, command: str,
                      out_md: str, out_json: str):
    """Two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    over the benchmark -> HBM bytes per launch of the matched kernel, each
    counter scaled by what it reads, in its own passes, for a plain copy of
    copy_bytes (bench.py --copy-probe)."""
    f = _pmc_by_kernel(fetch_dir)
    w = _pmc_by_kernel(write_dir)
    cf = _pmc_by_kernel(copy_fetch_dir)
    cw = _pmc_by_kernel(copy_write_dir)

    def per_dispatch(tab, match, counter):
        vals = [v for k, c in tab.items() if match in k for v in c.get(counter, [])]
        if not vals:
            raise ValueError(f"no {counter} for {match}")
        return float(np.median(vals)) * 1024.0

    copy_fetch = per_dispatch(cf, "copy", "FETCH_SIZE")
    copy_write = per_dispatch(cw, "copy", "WRITE_SIZE")
    sf, sw = copy_bytes / copy_fetch, copy_bytes / copy_write
    kf = per_dispatch(f, kernel_match, "FETCH_SIZE") * sf
    kw = per_dispatch(w, kernel_match, "WRITE_SIZE") * sw
    rec = {"source_hash": kernel_source_hash(kernel), "bytes_per_launch": kf + kw,
           "fetch_bytes": kf, "write_bytes": kw, "copy_scale_fetch": sf, "copy_scale_write": sw,
           "kernel_match": kernel_match}
    table = {}
    if os.path.exists(out_json):
        table = json.load(open(out_json))
    table[f"{kernel}:{workload}"] = rec
    with open(out_json, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    lines = [f"# HBM traffic: {kernel} on workload {workload}", "", "Commands:", "", "```", command, "```", "",
             f"- copy calibration: {copy_bytes} bytes copied; FETCH_SIZE read {copy_fetch:.4g} B "
             f"(scale {sf:.4f}), WRITE_SIZE read {copy_write:.4g} B (scale {sw:.4f})",
             f"- kernel `{kernel_match}`: fetch {kf/1e6:.2f} MB, write {kw/1e6:.2f} MB per launch "
             f"(scaled, median over dispatches)",
             f"- source hash of the kernel files when measured: {rec['source_hash']}"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out_md)


# ------------------------------------------------------------ main

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens for the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernels", action="store_true", help="also print per-stage times to stderr")
    ap.add_argument("--copy-probe", type=int, default=0, help="run a plain copy of this many bytes and exit")
    ap.add_argument("--clock-probe", nargs=4, metavar=("WORKLOAD", "SECONDS", "COMMAND", "OUT"),
                    help="gate/up and hipBLASLt back to back while sampling clocks and power; write OUT")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="DIR TITLE COMMAND OUT [LOG]: summarise a rocprofv3 kernel trace")
    ap.add_argument("--summarize-traffic", nargs=11,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "MATCH", "KERNEL",
                             "WORKLOAD", "COPY_BYTES", "COMMAND", "OUT_MD", "OUT_JSON"))
    args = ap.parse_args(argv)

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.summarize_traffic:
        a = list(args.summarize_traffic)
        a[7] = int(a[7])
        summarize_traffic(*a)
        return 0
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if args.clock_probe:
        w, sec, cmd, out = args.clock_probe
        clock_probe(w, float(sec), cmd, out)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and libmoe has no "
              "multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    wl = W.get(args.workload)
    decode = args.workload.startswith("c3")

    layer, x, host = setup(wl, device)
    st = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    active = int((counts > 0).sum())

    marks = {}
    if decode:
        # each step reads a cold cache: reading a 1 GiB buffer between steps
        # (outside the per-step events) evicts L2 and the 256 MB Infinity
        # Cache.  A read leaves clean lines, so the timed step pays no
        # write-back of the flush data.
        flush = torch.ones(1 << 28, dtype=torch.float32, device=device)
        sink = torch.empty((), dtype=torch.float32, device=device)
        step_ev = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            torch.sum(flush, dim=0, out=sink)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            layer.forward(x, marks=marks, stages=("gateup",))
            e1.record(st)
            step_ev.append((e0, e1))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = float(np.mean([a.elapsed_time(b) for a, b in step_ev]))
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer.forward(x, marks=marks, stages=("gateup",))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = wall * 1e3 / args.steps
    gateup_ms = float(np.mean([a.elapsed_time(b) for a, b in marks["gateup"]]))

    # per-stage breakdown (reported, not part of the timed steps)
    brk = {}
    for _ in range(3):
        if decode:
            torch.sum(flush, dim=0, out=sink)
        layer.forward(x, marks=brk)
    torch.cuda.synchronize()
    stage_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in brk.items()}
    stage_ms["gateup"] = gateup_ms
    tokens_per_s = wl.T / (ms * 1e-3)

    if decode:
        kname = "decode_gateup"
        alg = gateup_bytes(wl, active)
        achieved = alg / (stage_ms["gateup"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS}
    else:
        kname = "gateup"
        alg = gateup_flops(wl)
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = alg / (stage_ms["gateup"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof["kernel"] = kname
    roof["kernel_ms"] = stage_ms["gateup"]
    roof["traffic"] = load_traffic(kname, wl.name)

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "d_ff": wl.f, "experts": wl.E,
                   "top_k": wl.k, "score": wl.score, "zipf_s": wl.zipf_s, "shared_d_ff": wl.f_shared,
                   "active_experts": active, "parallelism": "single GPU",
                   "timing": "per-step events, caches flushed by a 1 GiB read between steps" if decode
                   else "wall clock over the timed steps"},
        "roofline": roof,
        "layer": {"tflops": layer_flops(wl) / (ms * 1e-3) / 1e12,
                  "mfma_frac": layer_flops(wl) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "gbps": layer_bytes(wl, active) / (ms * 1e-3) / 1e9,
                  "hbm_frac": layer_bytes(wl, active) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                  "stage_ms": stage_ms, "wall_s": wall,
                  "mfma_issued_over_algorithmic": None if decode else tile_work(wl, counts)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_sample)
    if args.kernels:
        print(json.dumps(stage_ms), file=sys.stderr)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
