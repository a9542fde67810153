"""Benchmark of the fused adaLN row-normalisation kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-kernels]

A step is one pass of the hot path over the FLUX.1-like adaLN workload
(1, 4608, 3072): the plain LayerNorm + modulate site and the gated-residual
site, two launches through the C ABI.  W untimed steps, then K timed steps
bracketed by torch.cuda.synchronize(); inputs are resident in HBM and rotate
over enough independent buffer sets (>= 1 GiB in total) that no launch finds
its data in the 256 MB Infinity Cache.  Every launch is bracketed by HIP
events on the stream it runs on, which gives each kernel's average duration.

Prints ONE JSON line: the step's throughput (algorithmic GB/s = bytes every
launch must move / time), the roofline of the dominant kernel, the CPU oracle
timed on this host's cores as a reported baseline, and (unless --no-kernels)
per-kernel GB/s and rows/s for every workload the kernels are checked on.
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

import torch  # noqa: E402

import dit_adaln_row_amd as dn  # noqa: E402
from dit_adaln_row_amd import inputs as gen  # noqa: E402
from dit_adaln_row_amd.workloads import HEADLINE, WORKLOADS  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30          # >= 4x the 256 MB Infinity Cache
METRIC = "achieved HBM GB/s (% of MI355X peak) and rows/s per fused norm+modulate kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "ln_modulate": "row_kernels.hip", "gated_ln_modulate": "row_kernels.hip",
    "rms_modulate": "row_kernels.hip", "qk_layernorm": "qk_kernel.hip",
    "rmsnorm_silu_bias": "wan_kernels.hip", "conv_bias_epilogue": "wan_kernels.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# argument marshalling for raw C-ABI calls (done once, outside the timed loop)
# ---------------------------------------------------------------------------

def _p(t):
    return None if t is None else t.data_ptr()


def make_call(lib, launch, t, stream):
    """(cfunc, args) for one launch of a workload on tensor set t."""
    e, rows, cols = launch.entry, launch.rows, launch.cols
    if e == "ln_modulate":
        out = torch.empty_like(t["x"])
        return lib.ln_modulate, (_p(t["x"]), _p(t["scale"]), _p(t["shift"]), _p(out), rows, cols,
                                 rows, cols, launch.eps, None, None, None, stream), out
    if e == "gated_ln_modulate":
        h, out = torch.empty_like(t["update"]), torch.empty_like(t["update"])
        return lib.gated_ln_modulate, (_p(t["update"]), _p(t["residual"]), _p(t["gate"]),
                                       _p(t["scale"]), _p(t["shift"]), _p(h), _p(out), rows, cols,
                                       rows, cols, launch.eps, None, None, None, stream), (h, out)
    if e == "rms_modulate":
        gated = launch.extra.get("gated", False)
        xn = "update" if gated else "x"
        out = torch.empty_like(t[xn])
        h = torch.empty_like(t[xn]) if gated else None
        return lib.rms_modulate, (_p(t[xn]), _p(t["weight"]), _p(t["scale"]), _p(t["shift"]),
                                  _p(out), _p(t["residual"]) if gated else None,
                                  _p(t["gate"]) if gated else None, _p(h), rows, cols, rows, cols,
                                  launch.eps, None, None, stream), (h, out)
    if e == "qk_layernorm":
        qo, ko = torch.empty_like(t["q"]), torch.empty_like(t["k"])
        return lib.qk_layernorm, (_p(t["q"]), _p(t["k"]), _p(qo), _p(ko), rows // 2, rows // 2,
                                  128, launch.eps, None, None, stream), (qo, ko)
    if e == "rmsnorm_silu_bias":
        out = torch.empty_like(t["x"])
        return lib.rmsnorm_silu_bias, (_p(t["x"]), _p(t["bias"]), _p(t["gamma"]), _p(out), rows,
                                       cols, launch.eps, None, None, stream), out
    raise KeyError(e)


def rotation_sets(w, device):
    """Enough independent input/output sets that their total is >= 1 GiB."""
    per_set = w.algorithmic_bytes()
    n = max(2, -(-ROTATE_BYTES // per_set))
    return [gen.make(w, device=device, seed_offset=i) for i in range(n)]


def check_status(st, what):
    if st != 0:
        raise RuntimeError(f"{what}: {dn.load().ditnorm_status_string(st).decode()}")


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def time_step_loop(calls_per_set, steps, warmup):
    """calls_per_set[s] = [(fn, args, name), ...] for rotation set s.  Returns
    (wall seconds for `steps` steps, {name: [event ms per launch]})."""
    nsets = len(calls_per_set)
    names = [c[2] for c in calls_per_set[0]]
    for i in range(warmup):
        for fn, args, name in calls_per_set[i % nsets]:
            check_status(fn(*args), name)
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for fn, args, name in calls_per_set[(warmup + i) % nsets]:
            a, b = ev[name][i]
            a.record()
            st = fn(*args)
            b.record()
            if st != 0:
                check_status(st, name)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in names}
    return t1 - t0, per


def time_kernel(calls, iters=200, warmup=20):
    """Per-launch event times (ms) of one launch kind over rotating sets; a
    spin kernel first lets the host queue the launches ahead of the GPU."""
    for i in range(warmup):
        fn, args = calls[i % len(calls)]
        check_status(fn(*args), "warmup")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)
    for i in range(iters):
        fn, args = calls[i % len(calls)]
        ev[i][0].record()
        fn(*args)
        ev[i][1].record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def kernel_source_hash(entry):
    src = os.path.join(ROOT, "dit_adaln_row_amd", "csrc", KERNEL_SOURCES[entry])
    hs = hashlib.sha256()
    for f in (src, os.path.join(ROOT, "dit_adaln_row_amd", "csrc", "device_common.hpp")):
        hs.update(open(f, "rb").read())
    return hs.hexdigest()[:16]


def traffic_for(workload, launch):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}/{launch.name}"
    r = rec.get("kernels", {}).get(key)
    if not r or r.get("source_hash") != kernel_source_hash(launch.entry):
        return None
    return r.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on this host's cores
# ---------------------------------------------------------------------------

def cpu_baseline(w, min_seconds=8.0):
    import concurrent.futures as cf

    import oracle
    oracle.build()
    threads = max(1, min(16, os.cpu_count() or 1))
    t = {k: (gen.to_u16(v) if v.dtype == torch.bfloat16 else v.numpy())
         for k, v in gen.make(w).items()}

    def chunks(rows):
        step = -(-rows // (threads * 4))
        return [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]

    def run_launch(l, ex):
        if l.entry == "ln_modulate":
            f = lambda b: oracle.ln_modulate(t["x"][b[0]:b[1]], t["scale"], t["shift"], l.eps)
        elif l.entry == "gated_ln_modulate":
            f = lambda b: oracle.gated_ln_modulate(t["update"][b[0]:b[1]], t["residual"][b[0]:b[1]],
                                                   t["gate"], t["scale"], t["shift"], l.eps)
        else:
            raise KeyError(l.entry)
        list(ex.map(f, chunks(l.rows)))

    reps = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while True:
            for l in w.launches:
                run_launch(l, ex)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or reps >= 50:
                break
    gbps = w.algorithmic_bytes() * reps / el / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full {w.key} step ({' + '.join(l.name for l in w.launches)}, "
                      f"{w.rows()} rows) x {reps} repetitions, {el:.1f} s wall, rows split over "
                      f"{threads} threads; the oracle is single-threaded C, unchanged",
            "rows_per_s": round(w.rows() * reps / el, 1)}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-kernels", action="store_true")
    ap.add_argument("--only", default=None, help="time only this workload's kernels (profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Rows are independent; see DESIGN.md for how the "
              f"path would shard.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")

    lib = dn.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream

    wkey = args.only or HEADLINE
    w = WORKLOADS[wkey]
    log(f"[bench] workload {w.key}: generating rotation sets")
    sets = rotation_sets(w, dev)
    calls = []
    keep = []
    for t in sets:
        row = []
        for l in w.launches:
            fn, a, outs = make_call(lib, l, t, stream)
            keep.append(outs)
            row.append((fn, a, l.name))
        calls.append(row)
    torch.cuda.synchronize()
    log(f"[bench] {len(sets)} rotation sets of {w.algorithmic_bytes() / 1e6:.1f} MB; "
        f"warmup {args.warmup}, steps {args.steps}")
    wall, per = time_step_loop(calls, args.steps, args.warmup)
    log("[bench] timed loop done")
    step_bytes = w.algorithmic_bytes()
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    kinfo = {}
    for l in w.launches:
        ms = sum(per[l.name]) / len(per[l.name])
        kinfo[l.name] = {"avg_ms": ms, "gbps": l.algorithmic_bytes() / (ms * 1e-3) / 1e9,
                         "bytes": l.algorithmic_bytes(), "rows": l.rows}
    dom = max(w.launches, key=lambda l: l.algorithmic_bytes() * kinfo[l.name]["avg_ms"])
    dk = kinfo[dom.name]
    traffic = traffic_for(w.key, dom)
    roofline = {"kernel": dom.name, "bound": "hbm", "achieved": round(dk["gbps"], 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dk["gbps"] / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": dom.algorithmic_bytes(),
                "avg_launch_ms": round(dk["avg_ms"], 5)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "accumulate": "f64 statistics, f32 elementwise ops rounded to bf16 per op",
        "data": "synthetic (seeded, distributions of the workload description)",
        "config": {"workload": w.key, "description": w.description,
                   "launches": [l.name for l in w.launches], "rows_per_step": w.rows(),
                   "bytes_per_step": step_bytes, "rotation_sets": len(sets)},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(w.rows() / (wall / args.steps), 1),
        "per_launch": {n: {"avg_ms": round(v["avg_ms"], 5), "gbps": round(v["gbps"], 1),
                           "pct_peak": round(100 * v["gbps"] / PEAK_HBM_GBPS, 2),
                           "rows_per_s": round(v["rows"] / (v["avg_ms"] * 1e-3), 1)}
                       for n, v in kinfo.items()},
        "roofline": roofline,
    }
    del sets, calls, keep
    torch.cuda.empty_cache()

    if not args.no_kernels and args.only is None:
        result["kernels"] = per_kernel_table(lib, dev, stream)
    if not args.no_cpu and args.only is None:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


def per_kernel_table(lib, dev, stream):
    """Median per-launch GB/s and rows/s of every workload's launches (200
    timed launches over rotating buffer sets each; copy kernel for context)."""
    table = {}
    for key, w in WORKLOADS.items():
        log(f"[bench] kernels: {key}")
        sets = rotation_sets(w, dev)
        for l in w.launches:
            calls, keep = [], []
            for t in sets:
                fn, a, outs = make_call(lib, l, t, stream)
                calls.append((fn, a))
                keep.append(outs)
            times = time_kernel(calls)
            med = times[len(times) // 2]
            gbps = l.algorithmic_bytes() / (med * 1e-3) / 1e9
            table[f"{key}/{l.name}"] = {
                "median_us": round(med * 1e3, 2), "p10_us": round(times[len(times) // 10] * 1e3, 2),
                "p90_us": round(times[9 * len(times) // 10] * 1e3, 2), "gbps": round(gbps, 1),
                "pct_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                "rows_per_s": round(l.rows / (med * 1e-3), 1), "bytes": l.algorithmic_bytes()}
            del keep
        del sets
        torch.cuda.empty_cache()
    # plain 16-byte copy moving 256 MB (read + write), the practical ceiling
    n = 128 << 20
    srcs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(4)]
    dsts = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(4)]
    calls = [(lib.ditnorm_copy, (_p(s), _p(d), n, stream)) for s, d in zip(srcs, dsts)]
    times = time_kernel(calls)
    med = times[len(times) // 2]
    gbps = 2 * n / (med * 1e-3) / 1e9
    table["copy_256MB"] = {"median_us": round(med * 1e3, 2), "gbps": round(gbps, 1),
                           "pct_peak": round(100 * gbps / PEAK_HBM_GBPS, 2), "bytes": 2 * n}
    return table


if __name__ == "__main__":
    main()
