"""Benchmark of the PaTH attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM: the prefill forward (block UT solve and
preconditioning, right-to-left scan with online softmax), the alignment of
the prompt's keys into the decode cache, then `decode_steps` fused decode
steps (rewrite every cached key with the new transition, append, attend).
Default workload: long-context PaTH-FoX, batch 1, 32 heads, head dim 64,
prompt 32768 tokens, 256 decode steps, bf16.

Prints one JSON line.  Phase and kernel times come from HIP events recorded
on the stream the kernels run on (the library records the prefill phase
events itself).  The fp64 CPU oracle is timed on a bounded sample of query
rows of the same workload as the CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("PaTH prefill TFLOP/s + tokens/s (fraction of bf16 MFMA peak); decode GB/s")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak

WORKLOADS = {
    "tiny": dict(cfg="tiny"),
    "long": dict(cfg="long"),
    "lm": dict(cfg="lm"),
    "fox2048": dict(cfg="fox", L=2048),
    "fox4096": dict(cfg="fox", L=4096),
    "fox8192": dict(cfg="fox", L=8192),
    "flipflop": dict(cfg="flipflop"),
}


def scan_flops(N, H, L, d, B=64):
    """GEMM flops the scan kernel executes: per query block b, the diagonal
    tile's P.V (its logits come from preconditioning), then for c < b the
    Q.K^T and P.V tiles, and (for c >= 1) one d x d transition of Qwork."""
    nb = (L + B - 1) // B
    per_slice = (nb * 2 * B * B * d
                 + nb * (nb - 1) // 2 * 4 * B * B * d
                 + max(nb - 1, 0) * max(nb - 2, 0) // 2 * 2 * B * d * d)
    return N * H * per_slice


def precond_flops(N, H, L, d, B=64):
    """GEMM flops of the per-block preconditioning (products of B x d and B x B
    operands: W W^T, Q W^T, W K^T, Q K^T, P = lower(QW^T) U, P W, U M, R^T W,
    U^T W, W^T Y, P M) and the B^3/3 triangular solve."""
    nb = (L + B - 1) // B
    per_block = 12 * B * B * d + 4 * B ** 3 + 2 * B * d * d
    return N * H * nb * per_block


def bwd_flops(N, H, L, d, B=64):
    """Matrix-core flops the backward kernels execute, for B = d: per block
    pair c < b, seven B x B x d products (key pass: the logits, dP, dV, dK;
    query pass: the transposed logits, dP^T, and the dQ-chain update
    Kr^T dS^T); per pair with c >= 1, three B x d x d ones (dE, the gradient
    chain's E^T product, the carried queries' transition); per block, 33
    products of B x B x d size (30 in the backward of the preconditioning with
    its recomputed forward products, three for the diagonal tile); plus the
    recomputed preconditioning, counted as in the forward.  rocprofv3's
    SQ_INSTS_VALU_MFMA_MOPS_BF16 matches this to 0.01 % once the
    preconditioning's split-operand products are counted twice."""
    nb = (L + B - 1) // B
    pairs = nb * (nb - 1) // 2
    tpairs = max(nb - 1, 0) * max(nb - 2, 0) // 2
    per_slice = pairs * 7 * 2 * B * B * d + tpairs * 3 * 2 * B * d * d + nb * 33 * 2 * B * B * d
    return N * H * per_slice + precond_flops(N, H, L, d, B)


def fa_eq_flops(N, H, L, d):
    return 2.0 * N * H * L * L * d


TRACKED_SOURCES = {
    "scan": "dependent_position_encoding_amd/csrc/fwd_bf16.hip",
    "precond": "dependent_position_encoding_amd/csrc/fwd_bf16.hip",
    "causal_baseline": "dependent_position_encoding_amd/csrc/fwd_bf16.hip",
    "decode": "dependent_position_encoding_amd/csrc/decode.hip",
}


def kernel_keys(workload):
    """Kernel name and launch size (work-items, as rocprofv3 reports
    Grid_Size) of each tracked kernel at a workload's shape."""
    import workloads
    spec = WORKLOADS[workload]
    wl = workloads.CONFIGS[spec["cfg"]]
    N, H, L, d = wl.N, wl.H, spec.get("L", wl.L), wl.d
    nb = (L + 63) // 64
    pairs = N * H * ((nb + 1) // 2) * 256
    keys = {"scan": (f"scan_mfma_kernel<{d}, {'true' if wl.fox else 'false'}>", pairs),
            "precond": (f"precond_mfma_kernel<{d}>", N * H * nb * 512),
            "causal_baseline": (f"causal_mfma_kernel<{d}>", pairs)}
    if wl.decode_steps:
        keys["decode"] = (f"decode_chunk_kernel<pa::bf16, pa::bf16, {d}, true>", None)
    return keys


def _source_sha(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _kname(raw):
    """Short kernel name, e.g. precond_mfma_kernel<64>, from a demangled
    signature or from a mangled one (whose template arguments are ints,
    bools and the library's element types)."""
    import re
    raw = raw.replace("(anonymous namespace)::", "")
    m = re.search(r"pa::(\w+(<[^()]*>)?)", raw)
    if m:
        return m.group(1)
    m = re.match(r"_ZN2pa(?:12_GLOBAL__N_1)?(\d+)", raw)
    if not m:
        return raw[:70]
    n = int(m.group(1))
    name, rest = raw[m.end():m.end() + n], raw[m.end() + n:]
    if not rest.startswith("I"):
        return name
    args, rest = [], rest[1:]
    while rest and rest[0] != "E":
        a = re.match(r"Li(-?\d+)E|Lb([01])E|NS_4bf16E|(f)", rest)
        if not a:
            break
        args.append(a.group(1) if a.group(1) is not None else
                    ("true" if a.group(2) == "1" else "false") if a.group(2) is not None else
                    "float" if a.group(3) else "pa::bf16")
        rest = rest[a.end():]
    return f"{name}<{', '.join(args)}>"


def _pmc_by_kernel(path):
    """Counter values per (kernel name, Grid_Size) of a rocprofv3 counter CSV."""
    import csv
    import re
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = _kname(r["Kernel_Name"])
            out.setdefault((name, int(r.get("Grid_Size") or 0)), []).append(
                float(r["Counter_Value"]))
    return out


def _values(rec, name, grid):
    return [v for (n, g), vs in rec.items() if n == name and (grid is None or g == grid)
            for v in vs]


def summarize_pmc(paths, workload):
    """HBM bytes per launch of the scan, the preconditioning, the beta = 0
    baseline and (with decode steps) the fused decode kernel at the workload's
    shape, from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reports for a device copy of known size."""
    fetch, write, cfetch, cwrite = (_pmc_by_kernel(p) for p in paths)
    copy_bytes = float(1 << 30)

    def copy_kib(rec):
        vals = [v for (k, _), vs in rec.items() if "copy" in k.lower() for v in vs]
        return sum(vals) / len(vals)

    f_scale = copy_bytes / (copy_kib(cfetch) * 1024)
    w_scale = copy_bytes / (copy_kib(cwrite) * 1024)
    res = {"workload": workload, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "kernels": {}}
    for key, (kname, grid) in kernel_keys(workload).items():
        fv, wv = _values(fetch, kname, grid), _values(write, kname, grid)
        if not fv or not wv:
            continue
        rb = sum(fv) / len(fv) * 1024 * f_scale
        wb = sum(wv) / len(wv) * 1024 * w_scale
        res["kernels"][key] = {"name": kname, "grid": grid, "dispatches": len(fv),
                               "read_bytes": rb,
                               "write_bytes": wb, "bytes": rb + wb,
                               "source": TRACKED_SOURCES[key],
                               "source_sha256": _source_sha(TRACKED_SOURCES[key])}
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def summarize_trace(path, top=24):
    """A markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv:
    per kernel the calls, average / minimum / maximum duration (us), total (ms)
    and share of the traced kernel time."""
    import csv
    import re
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = _kname(r["Name"])
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    print("| kernel | calls | avg us | min us | max us | total ms | % |")
    print("|---|---|---|---|---|---|---|")
    for n, c, a, lo, hi, t, pc in rows[:top]:
        print(f"| `{n}` | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} | {t:.3f} | {pc:.1f} |")


def causal_flops(N, H, L, d, B=64):
    """GEMM flops of the plain causal kernel: Q.K^T and P.V for every block
    pair c < b and for the (fully computed) diagonal tile."""
    nb = (L + B - 1) // B
    return N * H * (nb * (nb - 1) // 2 + nb) * 4 * B * B * d


def summarize_mfma(path, workload):
    """Matrix-core flops per dispatch from rocprofv3's SQ_INSTS_VALU_MFMA_MOPS_BF16
    (bf16 MFMA operations / 512) beside the flops the bench counts for the same
    launch: the long-context workload's scan, preconditioning and causal
    baseline, and the backward at the LM-layer shape (its four pair/block
    kernels plus the recomputed preconditioning against bwd_flops)."""
    import csv

    import workloads
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]) * 512))

    def mean(sub, grid=None):
        v = [x for n, g, x in rows if sub in n and (grid is None or g == grid)]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    spec = WORKLOADS[workload]
    wl = workloads.CONFIGS[spec["cfg"]]
    N, H, L, d = wl.N, wl.H, spec.get("L", wl.L), wl.d
    nb = (L + 63) // 64
    lm = workloads.CONFIGS["lm"]
    lnb = (lm.L + 63) // 64
    res = {"workload": workload, "counter": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512", "kernels": {}}
    for key, sub, grid, counted in (
            ("scan", "scan_mfma_kernel<64, true>", None, scan_flops(N, H, L, d)),
            ("precond", "precond_mfma_kernel", N * H * nb * 512, precond_flops(N, H, L, d)),
            ("causal_baseline", "causal_mfma_kernel", None, causal_flops(N, H, L, d))):
        m, n = mean(sub, grid)
        res["kernels"][key] = {"dispatches": n, "mfma_flops": m, "counted_flops": counted,
                               "ratio": None if m is None else round(m / counted, 4)}
    parts = {}
    for sub in ("bwd_key_b16_kernel", "bwd_query_b16_kernel", "bwd_chain_b16_kernel",
                "bwd_precond_b16_kernel"):
        parts[sub] = mean(sub)[0]
    parts["precond_mfma_kernel (recomputed)"] = mean("precond_mfma_kernel",
                                                     lm.N * lm.H * lnb * 512)[0]
    tot = sum(v for v in parts.values() if v is not None)
    counted = bwd_flops(lm.N, lm.H, lm.L, lm.d)
    res["kernels"]["backward_lm"] = {"parts": parts, "mfma_flops": tot, "counted_flops": counted,
                                     "ratio": round(tot / counted, 4)}
    out = os.path.join(ROOT, "profiles", f"mfma_{workload}.json")
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def measured_traffic(workload, key):
    """Counter-measured HBM bytes per launch, or None if not taken for this
    workload or if the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != _source_sha(rec["source"]):
        return None
    return rec["bytes"]


def decode_bytes(N, H, d, t, k_bytes, v_bytes):
    """HBM bytes one fused step at position t must move: read and write every
    cached key, read every cached value and log-f prefix entry."""
    return N * H * t * (2 * d * k_bytes + d * v_bytes + 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long", choices=sorted(WORKLOADS))
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration prefill measurements of the default run")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the decode steps one by one instead of replaying a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--summarize-mfma", metavar="MFMA_CSV",
                    help="write profiles/mfma_<workload>.json from a rocprofv3 "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 counter CSV and exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a bench run "
                         "and of a --calibrate-copy run into profiles/traffic_<workload>.json")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a markdown table of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the workload's prefill (and the beta = 0 baseline beside it) "
                         "without the front-end, backward and paged-decode measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dependent_position_encoding_amd as pa
    import workloads

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": src.numel() * 4,
                          "bytes_written": dst.numel() * 4, "dispatches": 3}))
        return
    pa.load_library()
    spec = WORKLOADS[args.workload]
    wl = workloads.CONFIGS[spec["cfg"]]
    if "L" in spec:
        wl = wl.replace(L=spec["L"])
    if args.decode_steps is not None:
        wl = wl.replace(decode_steps=args.decode_steps)
    N, H, L, d, T = wl.N, wl.H, wl.L, wl.d, wl.decode_steps
    print(f"[bench] workload {args.workload}: N={N} H={H} L={L} d={d} decode={T} "
          f"dtype={wl.dtype}", file=sys.stderr, flush=True)

    x = workloads.make_inputs(wl, device=dev)
    pre = {n: (x[n][:, :, :L].contiguous() if x[n] is not None else None) for n in x}
    tok = {n: [x[n][:, :, t].contiguous() for t in range(L, L + T)] if x[n] is not None else None
           for n in x}
    cache = pa.Cache(N, H, L + T, d, dtype=wl.dtype, gate=wl.fox, device=dev) if T else None
    ws = torch.empty(pa.fwd_workspace_bytes(N, H, L, d, wl.dtype, with_cache=T > 0),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(pre["q"])
    lse = torch.empty(N, H, L, dtype=torch.float32, device=dev)
    dws = torch.empty(max(pa.decode_workspace_bytes(cache, L + T), 1) if T else 1,
                      dtype=torch.uint8, device=dev)
    ot = torch.empty(N, H, d, dtype=wl.dtype, device=dev)
    lt = torch.empty(N, H, dtype=torch.float32, device=dev)

    E = lambda: torch.cuda.Event(enable_timing=True)

    def decode_loop():
        for i in range(T):
            pa.decode_step(cache, L + i, tok["q"][i], tok["k"][i], tok["v"][i], tok["w"][i],
                           tok["beta"][i], tok["logf"][i] if wl.fox else None,
                           scale=wl.scale, workspace=dws, out=(ot, lt))

    # The decode loop is launch-bound on the host (two kernels per token), so
    # it is captured once into a HIP graph and replayed: one submission per
    # 256 tokens.  The graph holds only the library's kernels (no memsets).
    graph = None
    if T and not args.no_graph:
        pa.fwd(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], logf=pre["logf"],
               scale=wl.scale, cache=cache, workspace=ws, out=(o, lse))
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            decode_loop()                                  # warm the binding on this stream
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_loop()
        torch.cuda.synchronize()

    def step(record):
        evs = [E() for _ in range(4)] if record else None
        pa.fwd(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], logf=pre["logf"],
               scale=wl.scale, cache=cache, workspace=ws, out=(o, lse), events=evs)
        dev_ev = []
        if T:
            if record:
                a, b = E(), E()
                a.record()
            if graph is not None:
                graph.replay()
            else:
                decode_loop()
            if record:
                b.record()
                dev_ev.append((a, b))
        return evs, dev_ev

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    recs = []
    t0, t1 = E(), E()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        recs.append(step(True))
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps

    pre_ms = np.mean([r[0][0].elapsed_time(r[0][1]) for r in recs])
    scan_ms = np.mean([r[0][1].elapsed_time(r[0][2]) for r in recs])
    align_ms = np.mean([r[0][2].elapsed_time(r[0][3]) for r in recs])
    fwd_ms = pre_ms + scan_ms + align_ms
    dec_ms = [float(np.mean([r[1][0][0].elapsed_time(r[1][0][1]) for r in recs]))] if T else []

    f_scan = scan_flops(N, H, L, d)
    f_pre = precond_flops(N, H, L, d)
    f_dec = sum(8.0 * N * H * (L + i + 1) * d for i in range(T))
    kb = 2 if cache is not None and cache.k_dtype == torch.bfloat16 else 4
    vb = 2 if wl.dtype == torch.bfloat16 else 4
    b_dec = sum(decode_bytes(N, H, d, L + i, kb, vb) for i in range(T))
    dec_total_ms = float(sum(dec_ms))

    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    # Headline: the prefill's executed matrix-core flops (scan + preconditioning)
    # over the whole prefill as a caller pays for it, cache alignment included
    # (its own d x d products are not counted, so this understates the rate).
    value = (f_scan + f_pre) / (fwd_ms * 1e-3) / 1e12
    scan_tf = f_scan / (scan_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "value_definition": "prefill executed TFLOP/s: scan_flops + precond_flops over the whole "
                            "prefill (preconditioning + scan + cache alignment), timed inside the "
                            "measured steps; decode is reported under 'decode'",
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": args.workload, "batch": N, "heads": H, "seq_len": L,
                   "head_dim": d, "decode_steps": T, "forget_gate": wl.fox,
                   "block": 64, "parallelism": "single GPU"},
        "prefill": {
            "ms": round(fwd_ms, 4), "precond_ms": round(pre_ms, 4),
            "scan_ms": round(scan_ms, 4), "cache_align_ms": round(align_ms, 4),
            "executed_TFLOP_s": round(value, 3),
            "fa_eq_TFLOP_s": round(fa_eq_flops(N, H, L, d) / (fwd_ms * 1e-3) / 1e12, 3),
            "tokens_per_s": round(N * L / (fwd_ms * 1e-3), 1),
            "frac_of_peak": round(value / peak, 4),
            "without_cache_alignment": {
                "ms": round(pre_ms + scan_ms, 4),
                "executed_TFLOP_s": round((f_scan + f_pre) / ((pre_ms + scan_ms) * 1e-3) / 1e12, 3),
                "frac_of_peak": round((f_scan + f_pre) / ((pre_ms + scan_ms) * 1e-3) / 1e12 / peak, 4),
                "tokens_per_s": round(N * L / ((pre_ms + scan_ms) * 1e-3), 1)},
            "timing": "library phase events on the launch stream, mean over the timed steps",
        },
        "roofline": {
            "kernel": "scan (right-to-left block scan with online softmax)",
            "bound": "mfma", "achieved": round(scan_tf, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(scan_tf / peak, 4), "traffic": measured_traffic(args.workload, "scan"),
            "algorithmic_note": "flops as counted by scan_flops(); traffic = HBM bytes per launch",
        },
    }
    if T:
        gbs = b_dec / (dec_total_ms * 1e-3) / 1e9
        out["decode"] = {
            "us_per_token_step": round(dec_total_ms / T * 1e3, 2),
            "GB_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "loop": "HIP graph of the 256 fused steps" if graph is not None else "eager launches",
        }
        out["roofline_decode"] = {
            "kernel": "fused decode step (rewrite + append + split-K attention, with its combine)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(args.workload, "decode"),
            "algorithmic_bytes_first_step": decode_bytes(N, H, d, L, kb, vb),
        }
        out["unfused_decode"] = unfused_rates(pa, cache, tok, L, wl, dws, ot, lt, kb, vb)
        out["decode_cache_cold"] = cold_decode_rate(pa, pre, cache, tok, L, wl, ws, dws, ot, lt,
                                                    kb, vb)
    if not args.prefill_only:
        out["prefill_reps"] = prefill_reps(pa, pre, wl, cache, ws, o, lse)
    if args.workload == "long" and not args.no_configs and not args.prefill_only:
        out["prefill_by_config"] = prefill_by_config(pa, dev)
    out["beta0_baseline"] = causal_baseline(pa, pre, wl, out["prefill"])
    if not args.prefill_only:
        out["front_end"] = front_end_rate(pa, wl, dev)
        out["backward"] = backward_rate(pa, dev)
        out["paged_decode"] = paged_decode_rate(pa, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds, N * (L + T) / (ms_step * 1e-3))
    print(json.dumps(out), flush=True)


BY_CONFIG = ("tiny", "flipflop", "lm", "fox2048", "fox4096", "fox8192")


def prefill_by_config(pa, dev, names=BY_CONFIG, budget_ms=400.0):
    """Prefill (no cache) at every workload shape: the library's phase events
    (preconditioning, scan) around each call, after two warm calls; enough
    calls to fill about `budget_ms` (at least 5, at most 50), medians.  Beside
    it the beta = 0 causal kernel at the same shape where it applies (bf16,
    d in {32, 64}), timed alike."""
    import numpy as np
    import torch

    import workloads
    res = {}
    for name in names:
        spec = WORKLOADS[name]
        wl = workloads.CONFIGS[spec["cfg"]]
        if "L" in spec:
            wl = wl.replace(L=spec["L"])
        N, H, L, d = wl.N, wl.H, wl.L, wl.d
        x = workloads.make_inputs(wl, device=dev, L=L)
        ws = torch.empty(pa.fwd_workspace_bytes(N, H, L, d, wl.dtype), dtype=torch.uint8,
                         device=dev)
        o = torch.empty_like(x["q"])
        lse = torch.empty(N, H, L, dtype=torch.float32, device=dev)
        run = lambda evs=None: pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"],
                                      logf=x["logf"], scale=wl.scale, workspace=ws,
                                      out=(o, lse), events=evs)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        reps = int(min(50, max(5, budget_ms / max(a.elapsed_time(b), 1e-3))))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for e in evs:
            run(e)
        torch.cuda.synchronize()
        pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
        scan_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
        tot_ms = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
        bf = wl.dtype == torch.bfloat16
        peak = PEAK_BF16_TFLOPS if bf else PEAK_F32_TFLOPS
        fl = scan_flops(N, H, L, d) + precond_flops(N, H, L, d)
        tf = fl / (tot_ms * 1e-3) / 1e12
        row = {"shape": {"batch": N, "heads": H, "seq_len": L, "head_dim": d,
                         "dtype": "bf16" if bf else "f32", "forget_gate": wl.fox},
               "reps": reps, "ms": round(tot_ms, 4), "precond_ms": round(pre_ms, 4),
               "scan_ms": round(scan_ms, 4),
               "executed_TFLOP_s": round(tf, 3),
               "fa_eq_TFLOP_s": round(fa_eq_flops(N, H, L, d) / (tot_ms * 1e-3) / 1e12, 3),
               "frac_of_peak": round(tf / peak, 4),
               "peak": "bf16 dense matrix" if bf else "fp32 vector",
               "scan_frac_of_peak": round(scan_flops(N, H, L, d) / (scan_ms * 1e-3) / 1e12 / peak, 4),
               "tokens_per_s": round(N * L / (tot_ms * 1e-3), 1)}
        if bf and d in (32, 64):
            for _ in range(2):
                pa.causal_attn(x["q"], x["k"], x["v"], scale=wl.scale, out=(o, lse))
            ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for c0, c1 in ce:
                c0.record()
                pa.causal_attn(x["q"], x["k"], x["v"], scale=wl.scale, out=(o, lse))
                c1.record()
            torch.cuda.synchronize()
            cms = float(np.median([c0.elapsed_time(c1) for c0, c1 in ce]))
            row["beta0_baseline_ms"] = round(cms, 4)
            row["beta0_baseline_fa_eq_TFLOP_s"] = round(
                fa_eq_flops(N, H, L, d) / (cms * 1e-3) / 1e12, 3)
            row["path_over_baseline_time"] = round(tot_ms / cms, 3)
        res[name] = row
        print(f"[bench] prefill {name}: {tot_ms:.3f} ms ({pre_ms:.3f} + {scan_ms:.3f}), "
              f"{tf:.1f} TFLOP/s = {tf / peak:.3f} of peak", file=sys.stderr, flush=True)
        del x, ws, o, lse
        torch.cuda.empty_cache()
    return res


def prefill_reps(pa, pre, wl, cache, ws, o, lse, reps=20):
    """Whole-prefill time (preconditioning, scan and, with a cache, its
    alignment) over `reps` back-to-back calls after three warm ones, each
    bracketed by its own events: median and minimum."""
    import numpy as np
    import torch
    run = lambda: pa.fwd(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], logf=pre["logf"],
                         scale=wl.scale, cache=cache, workspace=ws, out=(o, lse))
    for _ in range(3):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in evs]
    return {"reps": reps, "median_ms": round(float(np.median(t)), 4),
            "min_ms": round(float(np.min(t)), 4), "includes_cache_alignment": cache is not None}


def cold_decode_rate(pa, pre, cache, tok, L, wl, ws, dws, ot, lt, kb, vb, steps=32,
                     scratch_bytes=512 << 20):
    """Fused decode steps with the caches cold: before each step a 512 MiB
    scratch buffer (twice the size of the Infinity Cache) is either written
    (fill) or read (sum), so no cached key or value is left in any cache.  The
    written variant also leaves the Infinity Cache full of dirty scratch lines
    that the step's own traffic must write back to HBM; the read variant leaves
    clean lines only.  The cache is re-aligned from the prompt before each
    variant; each step is bracketed by its own events (the flush is outside
    them); eager launches, mean over `steps` steps."""
    import torch
    N, H, d = cache.N, cache.H, cache.d
    steps = min(steps, len(tok["q"]))
    scratch = torch.empty(scratch_bytes // 4, dtype=torch.float32, device=cache.device)
    scratch.fill_(1.0)
    acc = torch.empty((), dtype=torch.float32, device=cache.device)
    by = sum(decode_bytes(N, H, d, L + i, kb, vb) for i in range(steps))
    res = {"scratch_bytes_between_steps": scratch_bytes, "steps": steps}
    for mode in ("after_write", "after_read"):
        pa.fwd(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], logf=pre["logf"],
               scale=wl.scale, cache=cache, workspace=ws)
        evs = []
        for i in range(steps):
            if mode == "after_write":
                scratch.fill_(float(i + 2))
            else:
                torch.sum(scratch, dim=0, out=acc)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pa.decode_step(cache, L + i, tok["q"][i], tok["k"][i], tok["v"][i], tok["w"][i],
                           tok["beta"][i], tok["logf"][i] if wl.fox else None,
                           scale=wl.scale, workspace=dws, out=(ot, lt))
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs)
        gbs = by / (ms * 1e-3) / 1e9
        res[mode] = {"us_per_token_step": round(ms / steps * 1e3, 2), "GB_s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del scratch
    return res


def unfused_rates(pa, cache, tok, n, wl, dws, ot, lt, kb, vb, reps=20):
    """The unfused decode pieces at n cached keys, each replayed `reps` times
    from a HIP graph: path_kv_update alone (reads and writes every cached key)
    and path_decode alone (reads every key, value and gate prefix, then the
    combine).  Rates use the algorithmic bytes of each call."""
    import torch
    N, H, d = cache.N, cache.H, cache.d
    E = lambda: torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = E(), E()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "GB_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                "bytes": nbytes}

    g_bytes = 4 if cache.gcache is not None else 0
    upd = rate(lambda: pa.kv_update(cache, n, tok["w"][0], tok["beta"][0]), 2 * N * H * n * d * kb)
    dec = rate(lambda: pa.decode(cache, n, tok["q"][0], scale=wl.scale, workspace=dws, out=(ot, lt)),
               N * H * n * (d * kb + d * vb + g_bytes))
    return {"keys": n, "cache_update": upd, "decode_attention": dec,
            "note": "path_kv_update over n keys; path_decode over n keys (split-K + combine)"}


def front_end_rate(pa, wl, dev, R=32, reps=10):
    """The parameter front-end (path_param_fwd: w, beta, log f from a layer
    input of width H*d, rank R) at the workload's token count, replayed from a
    HIP graph (median of five replays after three warm ones).  Algorithmic
    bytes: the input x, the weights, and the outputs w, beta, log f; the
    projected intermediate's round trip through the workspace is reported
    beside them."""
    import torch
    import workloads
    N, H, L, d = wl.N, wl.H, wl.L, wl.d
    Dm = H * d
    p = workloads.make_frontend_inputs(N, L, Dm, R, H, d, wl.dtype, gate=wl.fox, device=dev)
    esz = 2 if wl.dtype == torch.bfloat16 else 4
    ws = torch.empty(pa.param_workspace_bytes(N, L, Dm, R, H, d, wl.dtype, wl.fox),
                     dtype=torch.uint8, device=dev)
    w = torch.empty(N, H, L, d, dtype=wl.dtype, device=dev)
    beta = torch.empty(N, H, L, dtype=torch.float32, device=dev)
    logf = torch.empty(N, H, L, dtype=torch.float32, device=dev) if wl.fox else None
    fn = lambda: pa.param_fwd(**p, H=H, d=d, workspace=ws, out=(w, beta, logf))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / reps)
    ms = sorted(times)[len(times) // 2]
    ngate = 2 if wl.fox else 1
    alg = (N * L * Dm * esz + (R * Dm + H * d * R + ngate * H * Dm) * esz + H * d * 12
           + N * H * L * d * esz + ngate * N * H * L * 4)
    rp = (R + ngate * H + 31) // 32 * 32
    gbs = alg / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "tokens_per_s": round(N * L / (ms * 1e-3), 1),
            "shape": {"tokens": N * L, "width": Dm, "rank": R, "heads": H, "head_dim": d,
                      "gate": wl.fox},
            "bound": "hbm", "GB_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": alg, "intermediate_bytes": 2 * N * L * rp * 4}


def paged_decode_rate(pa, dev, S=32, H=32, d=64, page=64, steps=16, seed=7):
    """Fused decode steps over a paged cache for a batch of S sequences of
    mixed lengths (seeded, uniform in [1024, 8192] cached keys), bf16 with the
    forget gate, pages assigned in a shuffled order.  One captured step
    (path_paged_decode_step advances the device lengths itself) is replayed
    `steps` times; the rate uses the algorithmic bytes of every step (read and
    write each cached key, read each value and gate prefix)."""
    import numpy as np
    import torch
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 8193, size=S)
    max_keys = int(lens.max()) + steps + 1        # one warm step, then `steps`
    need = (lens + 1 + steps + page - 1) // page  # pages of each final length
    stride = int(need.max())
    num_pages = int(need.sum())
    perm = rng.permutation(num_pages)
    table = np.zeros((S, stride), dtype=np.int32)
    at = 0
    for s in range(S):
        table[s, :need[s]] = perm[at:at + need[s]]
        at += need[s]
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    cache = pa.PagedCache(num_pages, page, H, d, dtype=torch.bfloat16, gate=True, device=dev)
    cache.kpages.copy_(torch.randn(cache.kpages.shape, generator=g, device=dev) * d ** -0.25)
    cache.vpages.copy_(torch.randn(cache.vpages.shape, generator=g, device=dev))
    cache.gpages.copy_(-torch.rand(cache.gpages.shape, generator=g, device=dev).cumsum(2) * 0.05)
    tab = torch.from_numpy(table).to(dev)
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    q = torch.randn(S, H, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(S, H, d, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(S, H, d, generator=g, device=dev).to(torch.bfloat16)
    w = torch.nn.functional.normalize(torch.randn(S, H, d, generator=g, device=dev), dim=-1)
    w = w.to(torch.bfloat16)
    beta = 2 * torch.sigmoid(torch.randn(S, H, generator=g, device=dev))
    logf = torch.nn.functional.logsigmoid(3 + torch.randn(S, H, generator=g, device=dev))
    o = torch.empty_like(q)
    lse = torch.empty(S, H, dtype=torch.float32, device=dev)
    ws = torch.empty(pa.paged_decode_workspace_bytes(S, H, d, torch.bfloat16, max_keys),
                     dtype=torch.uint8, device=dev)

    def launch():
        pa.paged_decode_step(cache, tab, seq, max_keys, q, k, v, w, beta, logf,
                             workspace=ws, out=(o, lse))

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        launch()                                  # warm the binding (one real step)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    torch.cuda.synchronize()
    start = lens + 1                              # cached keys at the first timed step
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert seq.cpu().numpy().tolist() == (lens + 1 + steps).tolist()
    assert torch.isfinite(o.float()).all()
    per_key = 2 * d * 2 + d * 2 + 4
    total = sum(float(H * (start + i).sum() * per_key) for i in range(steps))
    gbs = total / (ms * 1e-3) / 1e9
    return {"shape": {"sequences": S, "heads": H, "head_dim": d, "page_size": page,
                      "lengths": "uniform [1024, 8192] (seeded)",
                      "mean_cached_keys": round(float(start.mean()), 1)},
            "us_per_step": round(ms / steps * 1e3, 2), "GB_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "loop": "HIP graph of one step, replayed (device lengths advance)"}


def backward_rate(pa, dev, reps=3):
    """The backward pass (path_attn_bwd) at the LM-layer training shape (batch
    4, 24 heads, 4096 tokens, d = 64, bf16, scale 1, synthetic inputs of that
    workload), on the forward's own o and lse and a random dL/do: median of
    `reps` timed calls after a warm one; the forward timed alike beside it."""
    import torch
    import workloads
    wl = workloads.CONFIGS["lm"]
    x = workloads.make_inputs(wl, device=dev)
    N, H, L, d = x["q"].shape
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    do = torch.randn(x["q"].shape, generator=g, device=dev).to(wl.dtype)
    fwd = lambda: pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"],
                         scale=wl.scale)
    o, lse = fwd()
    ws = torch.empty(pa.bwd_workspace_bytes(N, H, L, d, wl.dtype), dtype=torch.uint8,
                     device=dev)
    bwd = lambda: pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], o, lse, do,
                         scale=wl.scale, workspace=ws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    ms, fwd_ms = timed(bwd), timed(fwd)
    fl = bwd_flops(N, H, L, d)
    tf = fl / (ms * 1e-3) / 1e12
    return {"shape": {"batch": N, "heads": H, "seq_len": L, "head_dim": d, "dtype": "bf16",
                      "forget_gate": wl.fox},
            "ms": round(ms, 3), "executed_TFLOP_s": round(tf, 2),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "executed_flops": fl,
            "fwd_ms": round(fwd_ms, 3), "bwd_over_fwd": round(ms / fwd_ms, 2),
            "tokens_per_s": round(N * L / (ms * 1e-3), 1),
            "workspace_GB": round(ws.numel() / 1e9, 3)}


def causal_baseline(pa, pre, wl, prefill):
    """Time the library's plain causal attention kernel (beta = 0, no gate) at
    the same shape: the FlashAttention-style baseline PaTH is compared with."""
    import numpy as np
    import torch
    N, H, L, d = pre["q"].shape
    o = torch.empty_like(pre["q"])
    lse = torch.empty(N, H, L, dtype=torch.float32, device=pre["q"].device)
    for _ in range(2):
        pa.causal_attn(pre["q"], pre["k"], pre["v"], scale=wl.scale, out=(o, lse))
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pa.causal_attn(pre["q"], pre["k"], pre["v"], scale=wl.scale, out=(o, lse))
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    fa = fa_eq_flops(N, H, L, d)
    return {"kernel": "path_causal_attn_fwd (plain causal softmax attention)",
            "ms": round(ms, 4), "fa_eq_TFLOP_s": round(fa / (ms * 1e-3) / 1e12, 3),
            "frac_of_peak": round(fa / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "path_prefill_over_baseline_time": round((prefill["precond_ms"] + prefill["scan_ms"]) / ms, 3)}


def cpu_baseline(wl, x, seconds, gpu_tokens_per_s):
    """Time the fp64 oracle on random query rows of 4 heads of this workload.
    Rows are uniform over the whole sequence, so the mean cost of a sampled
    row is the mean cost of a row of the full job; tokens/s is rows/s."""
    import numpy as np

    import oracle
    import workloads

    Ltot = x["q"].shape[2]
    job_rows = wl.N * wl.H * Ltot
    if job_rows <= 1 << 15:
        # a small job is timed whole: every row of every (batch, head) slice
        f64 = {n: (workloads.as_slices_f64(v) if v is not None else None) for n, v in x.items()}
        cores = oracle.num_threads()
        t = time.perf_counter()
        oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"], wl.scale)
        el = time.perf_counter() - t
        oracle.set_num_threads(1)
        try:
            t = time.perf_counter()
            oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                            wl.scale)
            el1 = time.perf_counter() - t
        finally:
            oracle.set_num_threads(cores)
        return {"value": round(job_rows / el, 1),
                "unit": "tokens/s (query rows of the full job per second)",
                "cores": cores, "kind": "oracle",
                "sample": f"the full job: all {job_rows} rows of {wl.N * wl.H} slices, fp64 walk, "
                          f"{el:.3f} s",
                "single_thread_tokens_per_s": round(job_rows / el1, 1),
                "single_thread_sample": f"the full job, {el1:.3f} s",
                "full_job_s": round(el, 4), "cpu_model": _cpu_model(),
                "gpu_tokens_per_s_same_job": round(gpu_tokens_per_s, 1)}
    heads = [0, 1, 2, 3][: wl.N * wl.H]
    f64 = {n: (workloads.as_slices_f64(v, heads) if v is not None else None) for n, v in x.items()}
    rng = np.random.default_rng(0)
    # calibrate on a small batch, then size the timed sample to ~`seconds`
    probe = rng.integers(0, Ltot, (len(heads), 8))
    t = time.perf_counter()
    oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"], wl.scale, rows=probe)
    rate = probe.size / max(time.perf_counter() - t, 1e-6)
    nrows = int(max(8, min(200000, rate * seconds / len(heads))))
    rows = rng.integers(0, Ltot, (len(heads), nrows))
    t = time.perf_counter()
    oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"], wl.scale, rows=rows)
    el = time.perf_counter() - t
    tps = rows.size / el
    cores = oracle.num_threads()
    # the same walk on one thread, sized to about a tenth of the timed sample's time
    rows1 = rng.integers(0, Ltot, (len(heads), max(4, nrows // (10 * max(cores, 1)))))
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                        wl.scale, rows=rows1)
        el1 = time.perf_counter() - t
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(tps, 1), "unit": "tokens/s (query rows of the full job per second)",
            "cores": cores, "kind": "oracle",
            "sample": f"{rows.size} random query rows (uniform over all {Ltot} positions) of "
                      f"{len(heads)} heads, fp64 walk, {el:.1f} s",
            "single_thread_tokens_per_s": round(rows1.size / el1, 1),
            "single_thread_sample": f"{rows1.size} rows, {el1:.1f} s",
            "extrapolated_full_job_s": round(job_rows / tps, 1),
            "extrapolated_note": f"all {job_rows} rows of the job at the sampled rate "
                                 "(sampled rows are uniform over positions, so their mean "
                                 "cost is a full-job row's)",
            "cpu_model": _cpu_model(),
            "gpu_tokens_per_s_same_job": round(gpu_tokens_per_s, 1)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
