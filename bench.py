"""Benchmark of the fused adaLN row-normalisation kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-kernels]

A step is one pass of the hot path over the FLUX.1-like adaLN workload
(1, 4608, 3072): the plain LayerNorm + modulate site and the gated-residual
site, two launches through the C ABI.  At least W untimed steps run first,
and at least WARMUP_FLOOR_MS of them in wall time whatever W is: in a fresh
process the first ~60 ms of back-to-back launches run up to 7% slower (the
gated launch measured 21.5 us after 20 warm-up steps, 20.4 after 200, 20.1
after 2000 and in every later loop).  Then K timed steps, bracketed by
torch.cuda.synchronize(), timed by HIP events recorded on the stream the
launches go to.  Inputs are resident in HBM and rotate over enough
independent buffer sets (>= 1 GiB for every launch) that no launch finds its
data in the 256 MB Infinity Cache.  Each launch kind runs as a burst between
HIP events, which gives each kernel's average duration.

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
WARMUP_FLOOR_MS = 200.0         # least wall time of warm-up steps before the timed loop
ROTATE_BYTES = 1 << 30          # >= 4x the 256 MB Infinity Cache
METRIC = "achieved HBM GB/s (% of MI355X peak) and rows/s per fused norm+modulate kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "ln_modulate": "row_kernels.hip", "gated_ln_modulate": "row_kernels.hip",
    "ln_modulate_folded": "row_kernels.hip",
    "rms_modulate": "row_kernels.hip", "qk_layernorm": "qk_kernel.hip",
    "rmsnorm_silu_bias": "wan_kernels.hip", "conv_bias_epilogue": "wan_kernels.hip",
    "modulate_scale_shift": "elementwise.hip", "residual_gate_add": "elementwise.hip",
    "ln_modulate_backward": "backward.hip",
}
DTYPE_CODES = {"bf16": 0, "f16": 1, "f32": 2}


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
    if e == "ln_modulate_folded":
        out = torch.empty_like(t["x"])
        return lib.ln_modulate_folded, (_p(t["x"]), _p(t["scale"]), _p(t["shift"]), _p(out), rows,
                                        cols, rows, cols, launch.eps, None, None, stream), out
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
    a, b, c = (t[n] for n in launch.inputs)
    if e == "ln_modulate_backward":        # inputs: x, scale, d_out
        rpb = launch.extra["rows_per_batch"]
        nb = rows // rpb
        d_x = torch.empty_like(a)
        d_scale = torch.empty((nb, cols), dtype=torch.float32, device=a.device)
        d_shift = torch.empty((nb, cols), dtype=torch.float32, device=a.device)
        dt = DTYPE_CODES[launch.extra.get("dtype", "bf16")]
        ws_bytes = lib.ln_modulate_backward_workspace_bytes(rows, cols, rpb, dt)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a.device)
        return lib.ln_modulate_backward, (_p(a), _p(b), _p(c), _p(d_x), _p(d_scale), _p(d_shift),
                                          rows, cols, rpb, cols, launch.eps, _p(ws), ws_bytes,
                                          None, None, dt, stream), (d_x, d_scale, d_shift, ws)
    if e == "conv_bias_epilogue":          # inputs: x, bias, h
        out = torch.empty_like(a)
        dt = DTYPE_CODES[launch.extra.get("dtype", "bf16")]
        bdt = DTYPE_CODES[launch.extra.get("bias_dtype", "f32")]
        return lib.conv_bias_epilogue, (_p(a), _p(b), _p(c), _p(out), rows, cols, dt, bdt,
                                        stream), out
    if e in ("modulate_scale_shift", "residual_gate_add"):
        # modulate: x, scale, shift; gate add: update, residual, gate
        out = torch.empty_like(a)
        return getattr(lib, e), (_p(a), _p(b), _p(c), _p(out), rows, cols, rows, cols,
                                 DTYPE_CODES[launch.extra["dtype"]], stream), out
    raise KeyError(e)


def rotation_sets(w, device):
    """Enough independent input/output sets that every launch of the workload,
    timed on its own, cycles through >= 1 GiB -- four times the 256 MB
    Infinity Cache (at most 64 sets: the 1 MB workload stays cache-resident,
    and is launch-bound)."""
    per_set = min(l.algorithmic_bytes() for l in w.launches)
    n = min(64, max(2, -(-ROTATE_BYTES // per_set)))
    return [gen.make(w, device=device, seed_offset=i) for i in range(n)]


def check_status(st, what):
    if st != 0:
        raise RuntimeError(f"{what}: {dn.load().ditnorm_status_string(st).decode()}")


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def time_step_loop(calls_per_set, steps, warmup, floor_ms=WARMUP_FLOOR_MS):
    """calls_per_set[s] = [(fn, args, name), ...]: the launches of one step on
    rotation set s.  Runs at least `warmup` untimed steps and at least
    `floor_ms` of them in wall time, then `steps` timed steps.  Inside the
    timed region each launch kind runs as one back-to-back burst (the K plain
    launches, then the K gated launches, every launch on its own rotating
    buffer set), with a HIP event on the launch stream before, between and
    after the bursts: the step time is the first-to-last event interval / K,
    and a kind's average launch duration is its burst interval / K, which is
    what rocprofv3 reports as the kernel's average duration.  Returns a dict:
    seconds (event time of the K steps), wall_seconds (host clock between the
    two synchronisations), per ({name: average ms per launch}), warmup_steps
    and warmup_ms (what the warm-up ran)."""
    nsets = len(calls_per_set)
    names = [c[2] for c in calls_per_set[0]]
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < floor_ms:
        for fn, args, name in calls_per_set[i % nsets]:
            check_status(fn(*args), name)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()  # the wall clock then follows the GPU's work
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for j, name in enumerate(names):
        for k in range(steps):
            fn, args, _ = calls_per_set[(i + k) % nsets][j]
            st = fn(*args)
            if st != 0:
                check_status(st, name)
        ev[j + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {n: ev[j].elapsed_time(ev[j + 1]) / steps for j, n in enumerate(names)}
    return {"seconds": ev[0].elapsed_time(ev[-1]) * 1e-3, "wall_seconds": t1 - t0, "per": per,
            "warmup_steps": i, "warmup_ms": warm_ms}


def time_kernel(calls, iters=100, reps=5, warmup=20, warm_ms=50.0):
    """Median over `reps` bursts of `iters` back-to-back launches (rotating
    buffer sets) of the per-launch time in ms; also the fastest and slowest
    burst.  The warm-up runs at least `warmup` launches and `warm_ms` of
    wall time, so that each kernel is timed on a settled GPU (the table
    follows the CPU baseline, which leaves the GPU idle for seconds)."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < warm_ms * 1e-3:
        for _ in range(20):
            fn, args = calls[i % len(calls)]
            check_status(fn(*args), "warmup")
            i += 1
        torch.cuda.synchronize()
    out = []
    for r in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(iters):
            fn, args = calls[i % len(calls)]
            fn(*args)
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / iters)
    return sorted(out)


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

def _cpu_info():
    """The host CPU as /proc/cpuinfo names it (first processor's entries)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k in ("model name", "vendor_id", "cpu family", "model", "stepping",
                     "cache size") and k not in info:
                info[k] = v
    except OSError:
        pass
    return info


def _cpu_model():
    i = _cpu_info()
    name = i.get("model name", "unknown")
    ids = ", ".join(f"{k} {i[k]}" for k in ("cpu family", "model", "stepping") if k in i)
    return f"{name} ({i.get('vendor_id', '?')}; {ids}; cache {i.get('cache size', '?')})"


def _cpu_quota():
    """The cgroup's CPU quota in CPUs (cgroup v2 cpu.max), or None."""
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        return None if q == "max" else round(int(q) / int(period), 2)
    except (OSError, ValueError):
        return None


def host_threads():
    """(threads for the CPU legs, CPUs this process may run on).  Every CPU in
    the process's affinity mask, but no more than the CPU share a job here is
    given when one is set (OMP_NUM_THREADS), so that the threads do not
    oversubscribe the share."""
    aff = len(os.sched_getaffinity(0))
    n = aff
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n), aff


def _oracle_call(oracle, l, t, lo, hi):
    """The oracle on rows [lo, hi) of launch l (whole batches for the backward)."""
    e = l.entry
    x = t[l.inputs[0]]
    if e == "ln_modulate":
        return oracle.ln_modulate(x[lo:hi], t["scale"], t["shift"], l.eps)
    if e == "ln_modulate_folded":
        return oracle.ln_modulate_folded(x[lo:hi], t["scale"], t["shift"], l.eps)
    if e == "gated_ln_modulate":
        return oracle.gated_ln_modulate(x[lo:hi], t["residual"][lo:hi], t["gate"], t["scale"],
                                        t["shift"], l.eps)
    if e == "rms_modulate":
        if l.extra.get("gated"):
            return oracle.rms_modulate(x[lo:hi], t["weight"], t["scale"], t["shift"], l.eps,
                                       residual=t["residual"][lo:hi], gate=t["gate"])
        return oracle.rms_modulate(x[lo:hi], t["weight"], t["scale"], t["shift"], l.eps)
    if e == "qk_layernorm":  # rows are q rows then k rows: half of the slice from each
        return oracle.qk_layernorm(t["q"][lo // 2:hi // 2], t["k"][lo // 2:hi // 2], l.eps)
    if e == "rmsnorm_silu_bias":
        return oracle.rmsnorm_silu_bias(x[lo:hi], t["bias"], t["gamma"], l.eps)
    if e == "conv_bias_epilogue":
        return oracle.conv_bias_epilogue_dt(x[lo:hi], t[l.inputs[1]], t[l.inputs[2]][lo:hi],
                                            l.extra.get("dtype", "bf16"),
                                            l.extra.get("bias_dtype", "f32"))
    if e == "modulate_scale_shift":
        return oracle.modulate_dt(x[lo:hi], t[l.inputs[1]], t[l.inputs[2]], l.extra["dtype"])
    if e == "residual_gate_add":
        return oracle.gate_residual_dt(x[lo:hi], t[l.inputs[1]][lo:hi], t[l.inputs[2]],
                                       l.extra["dtype"])
    if e == "ln_modulate_backward":
        rpb = l.extra["rows_per_batch"]
        fn = oracle.ln_modulate_backward_f32 if l.extra.get("dtype") == "f32" else \
            oracle.ln_modulate_backward
        sc, dout = t[l.inputs[1]], t[l.inputs[2]]
        if hi - lo <= rpb:  # part of one batch: a batch of that many tokens
            return fn(x[lo:hi], sc[:1], dout[lo:hi], l.eps, rows_per_batch=hi - lo)
        return fn(x[lo:hi], sc[lo // rpb:hi // rpb], dout[lo:hi], l.eps, rows_per_batch=rpb)
    raise KeyError(e)


def _keep_freed_memory():
    """glibc: serve large allocations from the heap and keep freed memory, so
    that the oracle's fresh output arrays do not page-fault on every call and
    the CPU timings measure its arithmetic."""
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-1, 1 << 30)  # M_TRIM_THRESHOLD
        libc.mallopt(-3, 1 << 30)  # M_MMAP_THRESHOLD
    except (OSError, AttributeError):
        pass


def _host_tensors(w, cap=None):
    """Host copies of a workload's inputs; with cap, 2-D tensors hold only
    their first cap rows (same distributions and seeds; a timing sample)."""
    if cap is None:
        return {k: (gen.to_u16(v) if v.dtype in (torch.bfloat16, torch.float16) else v.numpy())
                for k, v in gen.make(w).items()}
    out = {}
    for tt in w.tensors:
        shape = tt.shape if len(tt.shape) < 2 else (min(tt.shape[0], cap),) + tuple(tt.shape[1:])
        v = gen.normal(shape, tt.mu, tt.sigma, w.seed(tt.name), tt.kind)
        out[tt.name] = gen.to_u16(v) if v.dtype in (torch.bfloat16, torch.float16) else v.numpy()
    return out


def cpu_baseline(w, runs=5, run_seconds=2.5, single_runs=3, single_seconds=1.0):
    """The oracle on the host's cores: the whole headline step, rows split
    over threads, repeated for about run_seconds per run, median of `runs`
    runs; and single-threaded on a row sample (the first 1/8 of each launch's
    rows), median of `single_runs` runs of about single_seconds."""
    import concurrent.futures as cf
    import statistics

    import oracle
    oracle.build()
    _keep_freed_memory()
    threads, affinity = host_threads()
    t = _host_tensors(w)

    def chunks(rows):
        step = -(-rows // (threads * 4))
        return [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]

    rates, row_rates, total_reps, total_s = [], [], 0, 0.0
    with cf.ThreadPoolExecutor(threads) as ex:
        for _ in range(runs):
            reps, t0 = 0, time.perf_counter()
            while True:
                for l in w.launches:
                    list(ex.map(lambda b, l=l: _oracle_call(oracle, l, t, b[0], b[1]),
                                chunks(l.rows)))
                reps += 1
                el = time.perf_counter() - t0
                if el >= run_seconds or reps >= 5000:
                    break
            rates.append(w.algorithmic_bytes() * reps / el / 1e9)
            row_rates.append(w.rows() * reps / el)
            total_reps += reps
            total_s += el
    single, single_rows = [], []
    for _ in range(single_runs):
        n1, el1, b1, r1 = 0, 0.0, 0, 0
        t0 = time.perf_counter()
        while el1 < single_seconds and n1 < 5000:
            for l in w.launches:
                n = max(1, l.rows // 8)
                _oracle_call(oracle, l, t, 0, n)
                b1 += l.algorithmic_bytes() * n / l.rows
                r1 += n
            n1 += 1
            el1 = time.perf_counter() - t0
        single.append(b1 / el1 / 1e9)
        single_rows.append(r1 / el1)
    return {"value": round(statistics.median(rates), 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full {w.key} step ({' + '.join(l.name for l in w.launches)}, "
                      f"{w.rows()} rows), median of {runs} runs of about {run_seconds} s "
                      f"({total_reps} repetitions, {total_s:.1f} s in all), rows split over "
                      f"{threads} threads; the oracle is single-threaded C, unchanged",
            "runs_gbps": [round(r, 3) for r in rates],
            "rows_per_s": round(statistics.median(row_rates), 1),
            "threads": threads, "host_cores": affinity, "host_cpus_online": os.cpu_count(),
            "cpu_quota": _cpu_quota(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "single_thread": {"value": round(statistics.median(single), 3), "unit": "GB/s",
                              "rows_per_s": round(statistics.median(single_rows), 1),
                              "sample": f"the first 1/8 of each launch's rows, median of "
                                        f"{single_runs} runs of about {single_seconds} s"},
            "cpu_model": _cpu_model()}


def cpu_oracle_table(seconds=0.5, skip=()):
    """The oracle beside every workload's launches: GB/s-equivalent (the
    launch's algorithmic bytes per row) on a row sample, single-threaded and
    over the host's threads, each timed for about `seconds`."""
    import concurrent.futures as cf

    import oracle
    oracle.build()
    _keep_freed_memory()
    threads, _ = host_threads()
    table = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        for key, w in WORKLOADS.items():
            if key in skip:
                continue
            log(f"[bench] oracle: {key}")

            def sample_rows(l):
                rpb = l.extra.get("rows_per_batch", 1)
                n = max(1, l.rows // 16)
                if 1 < rpb <= n:  # whole batches (else one batch's first n tokens)
                    n -= n % rpb
                return n

            t = _host_tensors(w, cap=max(sample_rows(l) for l in w.launches))
            for l in w.launches:
                rpb = l.extra.get("rows_per_batch", 1)
                n = sample_rows(l)
                per_row = l.algorithmic_bytes() / l.rows
                row = {}
                for mode in ("single", "threads"):
                    if mode == "single":
                        parts = [(0, n)]
                    elif rpb > 1 and n <= rpb:  # one batch: not split
                        continue
                    else:
                        step = -(-n // threads)
                        if rpb > 1:
                            step = -(-step // rpb) * rpb
                        parts = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
                    run = lambda l=l, parts=parts: list(
                        ex.map(lambda b: _oracle_call(oracle, l, t, b[0], b[1]), parts))
                    run()  # untimed: first-touch of the outputs
                    reps, t0 = 0, time.perf_counter()
                    while True:
                        run()
                        reps += 1
                        el = time.perf_counter() - t0
                        if el >= seconds:
                            break
                    row[mode] = {"gbps": round(per_row * n * reps / el / 1e9, 3),
                                 "rows_per_s": round(n * reps / el, 1)}
                row["sample_rows"] = n
                table[f"{key}/{l.name}"] = row
            del t
    return {"threads": threads, "cpu_model": _cpu_model(), "launches": table}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-ms", type=float, default=WARMUP_FLOOR_MS,
                    help="least wall time of the warm-up steps (0 for counter runs, whose "
                         "every dispatch is serialised)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-kernels", action="store_true")
    ap.add_argument("--only", default=None, help="time only this workload's kernels (profiling)")
    ap.add_argument("--calib", action="store_true",
                    help="also launch the 16-byte copy kernel over 128 MB (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "NAME"),
                    help="CPU only: summarise a rocprofv3 --kernel-trace --stats run into profiles/NAME.txt")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "NAME"),
                    help="CPU only: turn FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json")
    ap.add_argument("--cmd", default="", help="the profiled command, recorded in the summary")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace, args.cmd)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.cmd)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Rows are independent, so the path shards by rows "
              f"across GPUs with no communication in the forward.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")

    lib = dn.load()
    log("[bench] source_hashes " + json.dumps({e: kernel_source_hash(e) for e in KERNEL_SOURCES}))
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
    tl = time_step_loop(calls, args.steps, args.warmup, args.warmup_ms)
    per = tl["per"]
    log(f"[bench] timed loop done (warm-up {tl['warmup_steps']} steps, {tl['warmup_ms']:.0f} ms)")
    step_bytes = w.algorithmic_bytes()
    sec = tl["seconds"]
    ms_per_step = sec / args.steps * 1e3
    value = step_bytes / (sec / args.steps) / 1e9

    kinfo = {}
    for l in w.launches:
        ms = per[l.name]
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
        "warmup_steps_run": tl["warmup_steps"], "warmup_ms": round(tl["warmup_ms"], 1),
        "timing": "HIP events on the launch stream around the K timed steps",
        "wall_ms_per_step": round(tl["wall_seconds"] / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "accumulate": "f64 statistics, f32 elementwise ops rounded to bf16 per op",
        "data": "synthetic (seeded, distributions of the workload description)",
        "config": {"workload": w.key, "description": w.description,
                   "launches": [l.name for l in w.launches], "rows_per_step": w.rows(),
                   "bytes_per_step": step_bytes, "rotation_sets": len(sets)},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(w.rows() / (sec / args.steps), 1),
        "per_launch": {n: {"avg_ms": round(v["avg_ms"], 5), "gbps": round(v["gbps"], 1),
                           "pct_peak": round(100 * v["gbps"] / PEAK_HBM_GBPS, 2),
                           "rows_per_s": round(v["rows"] / (v["avg_ms"] * 1e-3), 1)}
                       for n, v in kinfo.items()},
        "roofline": roofline,
    }
    del sets, calls, keep
    torch.cuda.empty_cache()
    if args.calib:
        copy_calibration(lib, dev, stream)

    if not args.no_kernels and args.only is None:
        result["kernels"] = per_kernel_table(lib, dev, stream)
    if not args.no_cpu and args.only is None:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w)
        result["cpu_baseline"]["per_launch"] = cpu_oracle_table()
    print(json.dumps(result), flush=True)


def copy_time_us(lib, dev, stream, moved_bytes, cache):
    """Median launch time of the library's plain copy moving `moved_bytes`
    (half read, half written), over rotating buffers of >= 1 GiB."""
    half = max(16, int(moved_bytes // 2) // 16 * 16)
    if half in cache:
        return cache[half]
    nsets = max(2, min(64, -(-(1 << 30) // (2 * half))))
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev),
             torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
    calls = [(lib.ditnorm_copy, (_p(a), _p(b), half, stream)) for a, b in bufs]
    times = time_kernel(calls)
    cache[half] = times[len(times) // 2] * 1e3
    del bufs
    return cache[half]


def per_kernel_table(lib, dev, stream):
    """Per-launch GB/s and rows/s of every workload's launches: the median of
    5 bursts of 100 back-to-back launches over rotating buffer sets, beside
    the plain copy kernel moving the same bytes (the practical ceiling, for
    context; `pct_of_copy` = copy time / launch time)."""
    table = {}
    copies = {}
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
            del keep
            cu = copy_time_us(lib, dev, stream, l.algorithmic_bytes(), copies)
            entry = {
                "median_us": round(med * 1e3, 2), "min_us": round(times[0] * 1e3, 2),
                "max_us": round(times[-1] * 1e3, 2), "gbps": round(gbps, 1),
                "pct_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                "rows_per_s": round(l.rows / (med * 1e-3), 1), "bytes": l.algorithmic_bytes(),
                "copy_us": round(cu, 2), "pct_of_copy": round(100 * cu / (med * 1e3), 1)}
            if l.algorithmic_bytes() * len(sets) < (256 << 20):
                entry["note"] = "launch-bound: the rotating sets stay cache-resident"
            table[f"{key}/{l.name}"] = entry
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


CALIB_BYTES = 128 << 20   # bytes read (and written) by one calibration copy launch


def copy_calibration(lib, dev, stream, launches=8):
    srcs = [torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev) for _ in range(4)]
    dsts = [torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev) for _ in range(4)]
    for i in range(launches):
        check_status(lib.ditnorm_copy(_p(srcs[i % 4]), _p(dsts[i % 4]), CALIB_BYTES, stream), "copy")
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/ (CPU only)
# ---------------------------------------------------------------------------

def _kernel_label(name):
    """Launch kind of a demangled kernel name."""
    if "ditnorm::row_mixed_kernel<" in name:
        # row_mixed_kernel<NV, RMS, GATED, P, WPB, REMFIRST, FOLD>
        args = [a.strip() for a in name.split("_kernel<", 1)[1].split(">", 1)[0].split(",")]
        rms, gated = args[1] == "true", args[2] == "true"
        fold = len(args) >= 7 and args[6] == "true"
        if fold:
            return "ln_modulate_folded"
        return {(False, False): "ln_modulate", (False, True): "gated_ln_modulate",
                (True, False): "rms_modulate", (True, True): "gated_rms_modulate"}[(rms, gated)]
    if "ditnorm::row_kernel<" in name or "ditnorm::row_wave_kernel<" in name:
        # row_kernel<NT, NV, RMS, GATED, FOLD> / row_wave_kernel<NV, FULL, RMS, GATED, MODE, FOLD>
        args = [a.strip() for a in name.split("_kernel<", 1)[1].split(">", 1)[0].split(",")]
        rms, gated = args[2] == "true", args[3] == "true"
        if args[-1] == "true" and len(args) in (5, 6):
            return "ln_modulate_folded"
        return {(False, False): "ln_modulate", (False, True): "gated_ln_modulate",
                (True, False): "rms_modulate", (True, True): "gated_rms_modulate"}[(rms, gated)]
    for key in ("bwd_fused_kernel", "bwd_tree_kernel"):
        if f"ditnorm::{key}" in name:
            return key
    if "ditnorm::elementwise_kernel<" in name:
        # elementwise_kernel<OP, DT, U>
        op, dt = (a.strip() for a in name.split("_kernel<", 1)[1].split(">", 1)[0].split(",")[:2])
        return ("modulate_scale_shift" if op == "0" else "residual_gate_add") + \
            ("_bf16" if dt == "0" else "_f16")
    if "ditnorm::epilogue_kernel<" in name:
        # epilogue_kernel<DT, F32BIAS, RES, U>
        dt = name.split("_kernel<", 1)[1].split(",")[0].strip()
        return "conv_bias_epilogue" + {"0": "", "1": "_f16", "2": "_f32"}[dt]
    for key, label in (("qk_kernel", "qk_layernorm"), ("wan_kernel", "rmsnorm_silu_bias"),
                       ("copy_kernel", "copy")):
        if f"ditnorm::{key}" in name:
            return label
    return None


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def summarize_trace(d, name, cmd):
    import csv
    files = _csvs(d, "kernel_stats.csv")
    if not files:
        sys.exit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# rocprofv3 kernel trace summary: {name}", f"# command: {cmd}", "",
             f"{'kernel':<70} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        n = r["Name"]
        lab = _kernel_label(n)
        short = (lab + "  " if lab else "") + n[:60]
        lines.append(f"{short:<70} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    out = os.path.join(ROOT, "profiles", f"{name}.txt")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(open(out).read())


def _pmc_means(d, counter):
    """{kernel label: mean counter value (KiB) per dispatch} from counter_collection.csv."""
    import csv
    files = _csvs(d, "counter_collection.csv")
    if not files:
        sys.exit(f"no counter_collection.csv under {d}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            lab = _kernel_label(r["Kernel_Name"])
            if lab:
                acc.setdefault(lab, []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _run_hashes(run_dir):
    """Kernel-source hashes the profiled bench run printed (in <run_dir>.log)."""
    try:
        for line in open(run_dir.rstrip("/") + ".log"):
            if "[bench] source_hashes " in line:
                return json.loads(line.split("[bench] source_hashes ", 1)[1])
    except OSError:
        pass
    sys.exit(f"{run_dir}.log has no source_hashes line: cannot tell which kernels were measured")


def summarize_pmc(fetch_dir, write_dir, workload, cmd):
    fetch = _pmc_means(fetch_dir, "FETCH_SIZE")
    write = _pmc_means(write_dir, "WRITE_SIZE")
    hashes = _run_hashes(fetch_dir)
    if hashes != _run_hashes(write_dir):
        sys.exit("the FETCH and WRITE runs measured different kernel sources")
    w = WORKLOADS[workload]
    f_cal = CALIB_BYTES / (fetch["copy"][0] * 1024.0)
    w_cal = CALIB_BYTES / (write["copy"][0] * 1024.0)
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {"kernels": {}}
    lines = [f"# HBM traffic per launch from rocprofv3 counters: {workload}",
             f"# command (two runs, --pmc FETCH_SIZE then --pmc WRITE_SIZE): {cmd}",
             f"# calibration: a plain 16-byte copy of {CALIB_BYTES} bytes reads "
             f"{fetch['copy'][0] * 1024:.0f} B by FETCH_SIZE (factor {f_cal:.4f}) and writes "
             f"{write['copy'][0] * 1024:.0f} B by WRITE_SIZE (factor {w_cal:.4f})", "",
             f"{'launch':<22} {'dispatches':>10} {'fetch_MB':>10} {'write_MB':>10} {'hbm_MB':>10} "
             f"{'algo_MB':>10} {'ratio':>7}"]
    for l in w.launches:
        lab = l.label()
        if l.entry == "ln_modulate_backward":
            # one call = the fused row / token pass and the tree levels:
            # every kernel's bytes over the number of calls
            parts = ("bwd_fused_kernel", "bwd_tree_kernel")
            if "bwd_fused_kernel" not in fetch or "bwd_fused_kernel" not in write:
                continue
            calls_f, calls_w = fetch["bwd_fused_kernel"][1], write["bwd_fused_kernel"][1]
            fb = sum(fetch[k][0] * fetch[k][1] for k in parts if k in fetch) / calls_f * 1024.0 * f_cal
            wb = sum(write[k][0] * write[k][1] for k in parts if k in write) / calls_w * 1024.0 * w_cal
            lab = "bwd_fused_kernel"
        elif lab not in fetch or lab not in write:
            continue
        else:
            fb = fetch[lab][0] * 1024.0 * f_cal
            wb = write[lab][0] * 1024.0 * w_cal
        algo = l.algorithmic_bytes()
        rec["kernels"][f"{workload}/{l.name}"] = {
            "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
            "hbm_bytes_per_launch": round(fb + wb), "algorithmic_bytes": algo,
            "ratio": round((fb + wb) / algo, 4), "calibration": {"fetch": f_cal, "write": w_cal},
            "source_hash": hashes[l.entry], "command": cmd}
        lines.append(f"{l.name:<22} {fetch[lab][1]:>10} {fb / 1e6:>10.2f} {wb / 1e6:>10.2f} "
                     f"{(fb + wb) / 1e6:>10.2f} {algo / 1e6:>10.2f} {(fb + wb) / algo:>7.3f}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    out = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
