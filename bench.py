"""Benchmark of the routed MoE FFN layer (libmoe) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

A step is one pass of the whole layer -- router logits + top-k, sort by
expert, grouped gate/up + SwiGLU, grouped down projection, (shared expert),
weighted combine -- over one resident batch of synthetic inputs.  Prints
one JSON line: layer tokens/s for the workload, the roofline position of
its dominant kernel (timed with HIP events on the launch stream), and the
CPU oracle timed on a bounded sample of the same workload.

The default workload is the largest layer that fits one GPU, the
DeepSeek-V3-shaped one (T=16384, d=7168, f=2048, E=256 routed experts,
top-8 sigmoid router with a Zipf(1.0) popularity bias, one shared expert of
f=2048, bf16).  The other workloads (c2 Mixtral-shaped, c3_t1 ... c3_t64
decode, c4 fine-grained) can be selected with --workload; decode workloads
evict the caches between steps and are timed per step with events.
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
    "down": ["gemm_bf16.hip", "grouped_gemm.h", "common.h"],
    "decode_gateup": ["decode.hip", "common.h"],
    "decode_down": ["decode.hip", "common.h"],
    "decode_mx_gateup": ["decode_mx.hip", "common.h", "select.h"],
    "decode_mx_down": ["decode_mx.hip", "common.h", "select.h"],
    "batched_gateup": ["batched.hip", "common.h", "select.h"],
    "batched_down": ["batched.hip", "common.h", "select.h"],
    "batched_mx_gateup": ["decode_mx.hip", "common.h", "select.h"],
    "batched_mx_down": ["decode_mx.hip", "common.h", "select.h"],
}


# ------------------------------------------------------------ accounting

def decode_tokens_per_s(bandwidth_bytes_per_s: float, active_params: float, bytes_per_param: float) -> float:
    """Bandwidth model of decode speed: every generated token reads every
    active parameter once, so tokens/s ~ bandwidth / (active params x bytes
    per param)."""
    return bandwidth_bytes_per_s / (active_params * bytes_per_param)


def layer_flops(wl, P=None, Ts=None) -> float:
    """Algorithmic FLOPs of one layer call: router + 3 expert GEMMs per
    routed pair (+ the shared expert on every token).  P: the routed pairs
    computed here (an expert-parallel share's), else all T*k; Ts: the
    tokens the shared expert runs on here, else all T."""
    P = wl.P if P is None else P
    Ts = wl.T if Ts is None else Ts
    return (2.0 * wl.T * wl.d * wl.E + 6.0 * P * wl.d * wl.f
            + 6.0 * Ts * wl.d * wl.f_shared)


def layer_bytes(wl, active: int) -> float:
    """Algorithmic HBM bytes of one layer call: each active expert's weights
    once, the router weights, x read and y written once (+ shared expert)."""
    b = wl.elem_bytes
    return (wl.expert_weight_bytes * 3.0 * wl.d * wl.f * active
            + b * (wl.d * wl.E + 2.0 * wl.T * wl.d + 3.0 * wl.d * wl.f_shared))


def gateup_flops(wl, P=None) -> float:
    """Grouped gate/up projection: 2 x (2f) x d FLOPs per routed row."""
    return 4.0 * (wl.P if P is None else P) * wl.d * wl.f


def gateup_bytes(wl, active: int, P=None) -> float:
    """Gate/up kernel: active experts' [2f, d] weights (as stored: MXFP4 at
    4.25 bits per weight) + routed rows in + H out."""
    b = wl.elem_bytes
    P = wl.P if P is None else P
    return wl.expert_weight_bytes * 2.0 * wl.f * wl.d * active + b * (P * wl.d + P * wl.f)


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


def down_bytes(wl, active: int, P=None) -> float:
    """Down kernel: active experts' [d, f] weights (as stored) + H rows in +
    Y_perm out."""
    b = wl.elem_bytes
    P = wl.P if P is None else P
    return wl.expert_weight_bytes * wl.d * wl.f * active + b * (P * wl.f + P * wl.d)


def kernel_rooflines(wl, active: int, kern_ms: dict, decode: bool, P=None, Ts=None) -> dict:
    """Roofline position of each projection kernel from its mean duration
    (HIP events on the launch stream over the timed steps).  Grouped
    workloads: algorithmic FLOPs (gate/up 4 d f, down 2 d f per routed row;
    the shared expert's per token) against dense bf16 MFMA peak.  Decode
    workloads: algorithmic bytes (active experts' weights once, rows in and
    out) against HBM peak."""
    out = {}
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    work = {
        "gateup": (gateup_flops(wl, P), gateup_bytes(wl, active, P)),
        "down": (2.0 * (wl.P if P is None else P) * wl.d * wl.f, down_bytes(wl, active, P)),
    }
    if wl.f_shared:
        fs, b = wl.f_shared, wl.elem_bytes
        Ts = wl.T if Ts is None else Ts             # the shared expert's tokens here
        work["shared_gateup"] = (4.0 * Ts * wl.d * fs, b * (2.0 * fs * wl.d + Ts * wl.d + Ts * fs))
        work["shared_down"] = (2.0 * Ts * wl.d * fs, b * (fs * wl.d + Ts * fs + Ts * wl.d))
    for name, (flops, nbytes) in work.items():
        if name not in kern_ms:
            continue
        s = kern_ms[name] * 1e-3
        if decode:
            a = nbytes / s / 1e9
            out[name] = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": a / PEAK_HBM_GBPS, "kernel_ms": kern_ms[name], "algorithmic_bytes": nbytes}
        else:
            a = flops / s / 1e12
            out[name] = {"bound": "mfma", "achieved": a, "peak": peak, "unit": "TFLOP/s", "frac": a / peak,
                         "kernel_ms": kern_ms[name], "algorithmic_flops": flops}
    return out


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


def setup(wl, device, keep_host: bool = True, mode: str = "auto", overlap_shared: bool = False, share: int = 1,
          split_shared: bool = False, share_index: int = 0, interleave: bool = False, balanced: bool = False):
    """Upload the workload's seeded inputs to the GPU and build the layer.
    With keep_host, the storage-format expert weights stay in host memory
    too (for the CPU oracle leg; the DeepSeek-shaped layer holds 22.5 GB).
    share > 1: one GPU's expert-parallel share of the layer, share_index
    I of them -- experts [I E/share, (I + 1) E/share), or with interleave
    the experts I, I + share, I + 2 share, ..., or with balanced the
    experts placement.balanced_shares gives share I from the routed load of
    a calibration batch (calibration_loads), and the shared expert on
    share 0 (with split_shared, on every share for its 1/share of the
    tokens) -- with every token routed."""
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
    if wl.experts == "mxfp4":
        gq, gs, dq, ds = W.gen_all_experts_mxfp4(wl)
        u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        weights = MoeWeights(dev(wr), None if bias is None else torch.from_numpy(bias).to(device), u8(gq), u8(dq),
                             w_gate_up_scales=u8(gs), w_down_scales=u8(ds))
        host_experts = {e: (gq[e], gs[e], dq[e], ds[e]) for e in range(wl.E)} if keep_host else {}
        host = dict(x=x, wr=wr, bias=bias, experts=host_experts, shared=None)
        return MoeLayer(weights, wl.k, wl.score, mode=mode), dev(x), host
    E_loc = wl.E // share
    e0 = share_index if interleave else share_index * E_loc
    stride = share if interleave else 1
    held = [e0 + j * stride for j in range(E_loc)]          # global ids in local order
    if balanced:
        from mixture_experts_ffn_04_amd.placement import balanced_shares
        held = balanced_shares(calibration_loads(wl, device, wr, bias, dev), share)[share_index]
    local = {e: j for j, e in enumerate(held)}
    gu = torch.empty(E_loc, 2 * wl.f, wl.d, dtype=tdt, device=device)
    dn = torch.empty(E_loc, wl.d, wl.f, dtype=tdt, device=device)
    host_experts = {}
    for e, g, w in W.iter_experts(wl, held):
        gu[local[e]].copy_(dev(g))
        dn[local[e]].copy_(dev(w))
        if keep_host:
            host_experts[e] = (g, w)
    sh = W.gen_shared(wl)
    if share > 1 and share_index > 0 and not split_shared:
        sh = None                                   # the shared expert lives on share 0
    weights = MoeWeights(dev(wr), None if bias is None else torch.from_numpy(bias).to(device), gu, dn,
                         None if sh is None else dev(sh[0]), None if sh is None else dev(sh[1]))
    where = {} if share == 1 else dict(expert_ids=held) if balanced else dict(experts=(e0, E_loc, stride))
    layer = MoeLayer(weights, wl.k, wl.score, mode=mode, overlap_shared=overlap_shared,
                     shared_part=(share_index, share) if split_shared and share > 1 else None, **where)
    host = dict(x=x, wr=wr, bias=bias, experts=host_experts, shared=sh)
    return layer, dev(x), host


def calibration_loads(wl, device, wr, bias, dev):
    """Routed rows per expert for a calibration batch: T tokens drawn like
    the workload's own but from another seed, routed by the library on the
    GPU (the load statistics an expert placement is made from; the timed
    batch is not used)."""
    import torch
    from mixture_experts_ffn_04_amd import binding
    xc = dev(W.gen_x(wl.replace(seed=wl.seed + 7919)))
    logits = torch.empty(wl.T, wl.E, device=device, dtype=torch.float32)
    ids = torch.empty(wl.T, wl.k, device=device, dtype=torch.int32)
    wts = torch.empty(wl.T, wl.k, device=device, dtype=torch.float32)
    binding.route(xc, dev(wr), None if bias is None else torch.from_numpy(bias).to(device), wl.k, wl.score,
                  logits, ids, wts)
    return torch.bincount(ids.view(-1).long(), minlength=wl.E).cpu().numpy()


# ------------------------------------------------------------ CPU oracle

def cpu_baseline(wl, host, sample_tokens: int, target_s: float = 15.0):
    """Time the CPU oracle (float64 router + eager expert loop) on the first
    `sample_tokens` tokens of the workload; when that takes well under
    target_s seconds, time it again on enough tokens (at most T) to take
    about target_s.

    Every input is generated before the clock starts (setup() keeps the
    storage-format weights in host memory).  The oracle takes float64
    values, so the bf16 -> float64 decode of each expert's weights, which
    the oracle's expert loop asks for one expert at a time, is timed on its
    own and subtracted: the figure is the oracle's arithmetic only."""
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    S = min(sample_tokens, wl.T)
    experts = host["experts"]
    if len(experts) != wl.E:
        raise RuntimeError("cpu_baseline needs the expert weights in host memory (setup(keep_host=True))")
    decode_s = [0.0]

    def fetch(e):
        t = time.perf_counter()
        if wl.experts == "mxfp4":
            gq, gs, dq, ds = experts[e]
            out = O.mxfp4_dequantize(gq, gs), O.mxfp4_dequantize(dq, ds)
        else:
            g, w = experts[e]
            out = W.values(g, wl.dtype), W.values(w, wl.dtype)
        decode_s[0] += time.perf_counter() - t
        return out

    x_all = host["x"]
    wr = W.values(host["wr"], wl.dtype)
    sh = host["shared"]
    shared = None if sh is None else (W.values(sh[0], wl.dtype), W.values(sh[1], wl.dtype))

    def run(S):
        x = W.values(x_all[:S], wl.dtype)
        decode_s[0] = 0.0
        t0 = time.perf_counter()
        L = O.router_logits(x, wr, host["bias"])
        ids, w = O.route(L, wl.k, wl.score)
        O.moe_layer_eager(x, ids, w, fetch, wl.E, shared)
        wall = time.perf_counter() - t0
        return wall - decode_s[0], wall, decode_s[0], ids

    dt, wall, dec, ids = run(S)
    if target_s and dt < 0.5 * target_s and S < wl.T:
        # a bounded sample of about target_s seconds of CPU work
        S = min(wl.T, max(S + 1, int(S * target_s / dt)))
        dt, wall, dec, ids = run(S)
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {S} of {wl.T} tokens of workload {wl.name}: float64 router + eager "
                      f"per-expert loop over the {len(np.unique(ids))} experts they select; "
                      f"{dt:.1f} s of oracle arithmetic ({wall:.1f} s wall, of which {dec:.1f} s decoding "
                      f"bf16 weights to float64, subtracted); inputs generated beforehand"}


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


def _grid(r) -> str:
    """Grid size of a dispatch (work-items) from a rocprofv3 trace row."""
    for key in ("Grid_Size_X", "Grid_Size", "Grid_Size_x"):
        if r.get(key) not in (None, ""):
            g = [r.get(key)] + [r.get(key[:-1] + c) for c in "YZ" if key.endswith("X") and r.get(key[:-1] + c)]
            return "x".join(x for x in g if x not in (None, "", "1")) or "1"
    return "?"


def summarize_trace(d: str, title: str, command: str, out: str, log: str = None):
    """rocprofv3 --kernel-trace CSV -> a short markdown table, one row per
    (kernel, grid size): the same tile kernel serves the routed projections
    and the shared expert (and both projections), which differ in grid size.
    With `log` (the profiled bench.py run's output), the bench's own figures
    for its projection kernels from the same run are quoted as well."""
    durs = {}
    for r in _read_csv(_find(d, "kernel_trace.csv")):
        key = (r["Kernel_Name"], _grid(r))
        durs.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = float(sum(sum(v) for v in durs.values())) or 1.0
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "Part `layer` is libmoe's kernels.  Part `harness` is the benchmark's own work outside the timed "
             "steps: weight uploads and read-backs (`copyBuffer`), buffer fills, and the cache-flush read "
             "between decode steps (`reduce_kernel`).  One row per kernel and grid size (work-items): the "
             "tile kernel runs the routed projections and the shared expert with different grids.  The "
             "averages include the warm-up calls and the untimed per-stage pass.", ""]
    if log:
        rec = None
        for line in open(log, errors="replace"):
            if line.startswith("{") and '"roofline"' in line:
                rec = json.loads(line)
        if rec is not None:
            r = rec["roofline"]
            lines += [f"bench.py in the same run: {rec['ms_per_step']:.3f} ms per step, "
                      f"{rec['value']:.4g} {rec['unit']}; per call (HIP events on the launch stream over the "
                      f"timed steps):"]
            for name, k in rec.get("layer", {}).get("kernels", {}).items():
                lines.append(f"- `{name}` {k['kernel_ms'] * 1e3:.1f} us, {k['achieved']:.4g} {k['unit']} "
                             f"({100 * k['frac']:.1f}% of {k['peak']:.0f})")
            lines.append("")
    lines += ["| kernel | grid | part | calls | avg us | median us | min us | max us | total % |",
              "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        part = "layer" if "moe::" in name else "harness"
        a = np.asarray(v, np.float64) / 1e3
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {grid} | {part} | {len(v)} | {a.mean():.2f} | {np.median(a):.2f} | "
                     f"{a.min():.2f} | {a.max():.2f} | {100.0 * sum(v) / total:.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def _pmc_by_kernel(d: str):
    """counter_collection.csv -> {"kernel name@grid": {counter: [values]}}."""
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _read_csv(_find(d, "counter_collection.csv")):
        acc[f"{r['Kernel_Name']}@{_grid(r)}"][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return acc


def summarize_pmc(d: str, title: str, command: str, out: str, n_simd: int = 1024, n_xcd: int = 8):
    """One rocprofv3 --pmc pass (with --kernel-trace for the durations) ->
    the median of every counter per (kernel, grid size), and where the
    counters are present:
      MFMA FLOPs issued = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (one MOP is 512
                          bf16 FLOPs)
      cycles            = GRBM_GUI_ACTIVE / 8 (the counter is summed over the
                          8 XCDs, each counting the kernel's active cycles)
      MFMA busy         = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)
                          (the busy counter is summed over all SIMDs; it reads
                          32 cycles per v_mfma_f32_32x32x16_bf16)
      clock             = cycles / the dispatch's duration"""
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _read_csv(_find(d, "counter_collection.csv")):
        acc[(r["Kernel_Name"], _grid(r))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    durs = collections.defaultdict(list)
    try:
        for r in _read_csv(_find(d, "kernel_trace.csv")):
            durs[(r["Kernel_Name"], _grid(r))].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    except FileNotFoundError:
        pass
    names = sorted({c for v in acc.values() for c in v})
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "Medians over the dispatches of each (kernel, grid size).  Derived: MFMA TFLOP issued = 512 x "
             f"SQ_INSTS_VALU_MFMA_MOPS_BF16; cycles = GRBM_GUI_ACTIVE / {n_xcd} (summed over the {n_xcd} XCDs); "
             f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {n_simd} SIMDs) (the busy counter is summed over "
             "the SIMDs and reads 32 cycles per 32x32x16 bf16 MFMA); clock = cycles / dispatch duration "
             "(kernel trace of the same run; the profiler serialises dispatches).", "",
             "| kernel | grid | dispatches | " + " | ".join(names) +
             " | MFMA TFLOP issued | cycles | MFMA busy | us | clock MHz |",
             "|---|---|---|" + "---|" * len(names) + "---|---|---|---|---|"]
    for (name, grid), cs in sorted(acc.items(), key=lambda kv: kv[0]):
        if "moe::" not in name:
            continue
        med = {c: float(np.median(v)) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        fl = med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES")
        gui = med.get("GRBM_GUI_ACTIVE")
        cyc = gui / n_xcd if gui else None
        us = float(np.median(durs[(name, grid)])) / 1e3 if durs.get((name, grid)) else None
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {grid} | {n} | " + " | ".join(f"{med[c]:.6g}" if c in med else "" for c in names)
                     + f" | {'' if fl is None else f'{512 * fl / 1e12:.4g}'}"
                     + f" | {'' if cyc is None else f'{cyc:.4g}'}"
                     + f" | {'' if busy is None or not cyc else f'{busy / (cyc * n_simd):.3f}'}"
                     + f" | {'' if us is None else f'{us:.1f}'}"
                     + f" | {'' if us is None or not cyc else f'{cyc / us:.0f}'} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


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
        # match: a substring of the kernel name, optionally "...@grid" to pick
        # one grid size (the routed and shared-expert launches of one kernel)
        name, _, grid = match.partition("@")
        vals = [v for k, c in tab.items() if name in k.rpartition("@")[0] and (not grid or k.rpartition("@")[2] == grid)
                for v in c.get(counter, [])]
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
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--mode", default="auto", choices=("auto", "grouped", "decode", "batched"),
                    help="layer strategy (auto: decode calls up to 256 routed rows, grouped above)")
    ap.add_argument("--overlap-shared", action="store_true",
                    help="run the shared expert on a second stream beside the router, the sort and the routed "
                         "experts (measured no faster on the DeepSeek-shaped layer; default: after them)")
    ap.add_argument("--ep-share", type=int, default=1, metavar="N",
                    help="time one GPU's expert-parallel share of N (experts [0, E/N) and the shared expert, "
                         "every token routed, local pairs only); prefill workloads")
    ap.add_argument("--ep-index", type=int, default=0, metavar="I",
                    help="with --ep-share N: time share I (experts [I E/N, (I + 1) E/N)) instead of share 0")
    ap.add_argument("--ep-interleave", action="store_true",
                    help="with --ep-share N: share I holds the experts I, I + N, I + 2N, ... instead of a block")
    ap.add_argument("--ep-balanced", action="store_true",
                    help="with --ep-share N: share I holds the experts that a load-balanced placement gives it "
                         "from the routed load of a calibration batch (T tokens of another seed)")
    ap.add_argument("--split-shared", action="store_true",
                    help="with --ep-share N: every share runs the shared expert on 1/N of the tokens (share I on "
                         "tokens [T I/N, T (I + 1)/N)) instead of share 0 on all of them")
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens for the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernels", action="store_true", help="also print per-stage times to stderr")
    ap.add_argument("--copy-probe", type=int, default=0, help="run a plain copy of this many bytes and exit")
    ap.add_argument("--clock-probe", nargs=4, metavar=("WORKLOAD", "SECONDS", "COMMAND", "OUT"),
                    help="gate/up and hipBLASLt back to back while sampling clocks and power; write OUT")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="DIR TITLE COMMAND OUT [LOG]: summarise a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("DIR", "TITLE", "COMMAND", "OUT"),
                    help="summarise one rocprofv3 --pmc pass per kernel and grid")
    ap.add_argument("--summarize-traffic", nargs=11,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "MATCH", "KERNEL",
                             "WORKLOAD", "COPY_BYTES", "COMMAND", "OUT_MD", "OUT_JSON"))
    args = ap.parse_args(argv)

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
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

    wl = W.get(args.workload)
    decode = args.workload.startswith("c3")   # weight streaming: timed per step after a cache flush
    if wl.experts == "mxfp4" and args.mode not in ("auto", "decode", "batched"):
        print("MXFP4 experts run on the decode or the batched calls", file=sys.stderr)
        return 2
    share = args.ep_share
    if share > 1:
        if decode or wl.experts == "mxfp4" or wl.E % share or args.mode not in ("auto", "grouped"):
            print("--ep-share: prefill workloads with E divisible by N, grouped calls", file=sys.stderr)
            return 2
        args.no_cpu = True          # the oracle leg needs every expert

    if (args.split_shared or args.ep_index or args.ep_interleave or args.ep_balanced) and share == 1:
        print("--split-shared, --ep-index, --ep-interleave and --ep-balanced go with --ep-share N (N > 1)",
              file=sys.stderr)
        return 2
    if args.ep_interleave and args.ep_balanced:
        print("--ep-interleave and --ep-balanced are two different placements: pass one", file=sys.stderr)
        return 2
    if not 0 <= args.ep_index < share:
        print("--ep-index I needs 0 <= I < N", file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    layer, x, host = setup(wl, device, keep_host=not args.no_cpu, mode=args.mode,
                           overlap_shared=args.overlap_shared, share=share, split_shared=args.split_shared,
                           share_index=args.ep_index, interleave=args.ep_interleave, balanced=args.ep_balanced)
    # the shared expert's tokens here
    ts0, ts1 = wl.T * args.ep_index // share, wl.T * (args.ep_index + 1) // share
    Ts = ts1 - ts0 if args.split_shared else (0 if args.ep_index else None)
    st = torch.cuda.current_stream()
    # the projection kernels are timed by events on the launch stream inside
    # the timed steps; an event pair costs a few microseconds, so the
    # microsecond-scale decode steps carry one only around the dominant
    # kernel, and only every other step: the step time is the mean over the
    # steps without it (the other kernels come from the untimed per-stage
    # pass)
    timed = ("gateup",) if decode else ("gateup", "down", "shared_gateup", "shared_down")

    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    if layer.use_batched(wl.T):
        # no sort: the experts the pairs chose
        counts = np.bincount(layer.ids.cpu().numpy().reshape(-1), minlength=wl.E)
    else:
        counts = layer.counts.cpu().numpy()
    active = int((counts > 0).sum())
    P_here = int(counts.sum()) if share > 1 else None     # an expert-parallel share's routed pairs

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
            if i % 2:
                layer.forward(x, marks=marks, stages=timed)      # the dominant kernel's events
            else:
                layer.forward(x)
            e1.record(st)
            step_ev.append((e0, e1))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = float(np.mean([a.elapsed_time(b) for i, (a, b) in enumerate(step_ev) if i % 2 == 0]))
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer.forward(x, marks=marks, stages=timed)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = wall * 1e3 / args.steps
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in v])) for n, v in marks.items()}

    # per-stage breakdown (reported, not part of the timed steps)
    brk = {}
    for _ in range(3):
        if decode:
            torch.sum(flush, dim=0, out=sink)
        layer.forward(x, marks=brk)
    torch.cuda.synchronize()
    stage_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in brk.items()}
    stage_ms.update(kern_ms)
    for name in ("gateup", "down", "shared_gateup", "shared_down"):
        if name in stage_ms and name not in kern_ms:
            kern_ms[name] = stage_ms[name]          # from the per-stage pass
    tokens_per_s = wl.T / (ms * 1e-3)

    kernels = kernel_rooflines(wl, active, kern_ms, decode, P_here, Ts)
    if layer.use_batched(wl.T):
        kname = "batched_mx_gateup" if wl.experts == "mxfp4" else "batched_gateup"
    elif decode:
        kname = "decode_mx_gateup" if wl.experts == "mxfp4" else "decode_gateup"
    else:
        kname = "gateup"
    roof = dict(kernels["gateup"])
    roof["kernel"] = kname
    roof["traffic"] = load_traffic(kname, wl.name) if share == 1 else None   # taken on the whole layer

    if args.ep_balanced:
        experts_desc = (f"{(layer.emap >= 0).nonzero().view(-1).tolist()} (placed by the "
                        f"routed load of a calibration batch)")
    elif args.ep_interleave:
        experts_desc = f"{args.ep_index}, {args.ep_index + share}, ... (every {share}th)"
    else:
        experts_desc = f"{args.ep_index * (wl.E // share)}..{(args.ep_index + 1) * (wl.E // share) - 1}"
    if not wl.f_shared or Ts == 0:
        shared_desc = ""
    elif args.split_shared:
        shared_desc = f" and the shared expert on tokens {ts0}..{ts1 - 1}"
    else:
        shared_desc = " and the shared expert"
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
        "dtype": "mxfp4 weights, bf16 activations" if wl.experts == "mxfp4" else wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "d_ff": wl.f, "experts": wl.E,
                   "top_k": wl.k, "score": wl.score, "zipf_s": wl.zipf_s, "shared_d_ff": wl.f_shared,
                   "active_experts": active, "strategy": args.mode,
                   "parallelism": "single GPU" if share == 1 else
                   f"one GPU's expert-parallel share ({args.ep_index} of {share}): experts {experts_desc}"
                   f"{shared_desc}, every token routed, {P_here} of {wl.P} "
                   f"routed pairs here (the sum over shares is not run)",
                   "shared_expert": None if not wl.f_shared else
                   ("second stream beside the routed experts" if args.overlap_shared else "after the routed experts"),
                   "timing": "per-step events, caches flushed by a 1 GiB read between steps; the dominant "
                             "kernel's events on every other step, the step time over the others" if decode
                   else "wall clock over the timed steps"},
        "roofline": roof,
        "layer": {"tflops": layer_flops(wl, P_here, Ts) / (ms * 1e-3) / 1e12,
                  "mfma_frac": layer_flops(wl, P_here, Ts) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "gbps": layer_bytes(wl, active) / (ms * 1e-3) / 1e9,
                  "hbm_frac": layer_bytes(wl, active) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                  "stage_ms": stage_ms, "wall_s": wall, "kernels": kernels,
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
