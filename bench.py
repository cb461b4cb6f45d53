#!/usr/bin/env python3
"""Benchmark of the fused BF16 GEMM + reduce-scatter (one TP=8 rank's share).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large_prefill]

A step is one fused run of the whole hot path (GEMM tiles, routed BF16
epilogue with ready flags, reducers summing this rank's slice with the 7 peer
partials) over inputs already resident in HBM.  Prints ONE JSON line:
fused TFLOP/s (value), its fraction of the MI355X dense BF16 MFMA peak, the
overlap efficiency 1 - (T_fused - T_gemm) / T_reduce against the same GEMM and
the standalone reduce kernel run alone, a roofline object for the fused kernel,
and the CPU oracle timed on the host cores as a baseline.  The headline
workload is the large prefill shape (M = 32768), the largest of the metric's
range M = 512..32768; with --sweep (the default) the other benchmark shapes
are timed too and reported under "sweep", each with its own roofline fraction.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA (AMD published figure)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (AMD published figure)
METRIC = "fused GEMM+RS TFLOP/s (% bf16 MFMA peak) + overlap efficiency, M=512..32768"
DEFAULT_WORKLOAD = "large_prefill"
SWEEP = ("o_proj", "down_proj", "mixtral_down", "large_prefill")


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_gemm_reduce_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-sweep", dest="sweep", action="store_false")
    p.add_argument("--no-cpu", dest="cpu", action="store_false")
    p.add_argument("--no-check", dest="check", action="store_false")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--tile", default="auto")
    p.add_argument("--reducers", type=int, default=-1,
                   help="dedicated reducer workgroups: -1 the plan's default, -2 the adaptive controller")
    p.add_argument("--reduce-mode", default="auto", choices=["auto", "tail", "coresident", "stream", "adaptive"],
                   help="where the fused launch sums the slice without dedicated reducers")
    p.add_argument("--tile-stores", default="auto", choices=["auto", "device", "nt"],
                   help="cache policy of the routed tile stores (nt: non-temporal hint; auto: the library's choice)")
    p.add_argument("--cold", action="store_true",
                   help="also time the fused, GEMM-only and reduce launches with cold caches (a 512 MiB "
                        "buffer written before each launch)")
    p.add_argument("--sweep-out", default=None, help="also write per-config lines here")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run only a plain copy of known size and a few fused launches of --workload "
                        "(the program a rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE pass runs)")
    p.add_argument("--split-sweep", metavar="OUT_JSON",
                   help="time the fused launch of --workload over the compute/reducer split (dedicated "
                        "reducer workgroups R), the flag padding and the in-loop reducer slots, write "
                        "the table to OUT_JSON and exit")
    p.add_argument("--allreduce-sweep", metavar="OUT_JSON",
                   help="time GEMM + all-reduce (gemm_rs_run_allreduce: the reduce-scatter whose sum also "
                        "replicates the reduced slice to the 7 peers) on every benchmark shape, write "
                        "OUT_JSON and exit")
    p.add_argument("--allgather-sweep", metavar="OUT_JSON",
                   help="time all-gather + GEMM (the column-parallel layer) per layer shape, write OUT_JSON")
    p.add_argument("--timeline", metavar="OUT_MD",
                   help="trace one fused launch per reduce placement (tail, stream, adaptive) and write a "
                        "timeline summary of the GEMM's releases and the slice sum's stamps")
    p.add_argument("--counter-probe", action="store_true",
                   help="for rocprofv3 --pmc: two GEMM-only launches, two fused launches and two hipBLASLt "
                        "GEMMs of the workload, each synchronized")
    p.add_argument("--counters-from", nargs="+", metavar="COUNTER_CSV",
                   help="markdown table of the per-kernel mean of every counter in rocprofv3 counter CSVs")
    p.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                   help="print a markdown table of a rocprofv3 --stats kernel_stats.csv and exit")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn the counter_collection.csv of the two --traffic-probe passes into "
                        "profiles/traffic_<workload>.json and exit (no GPU needed)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Case:
    """Device inputs/outputs and a handle for one benchmark shape."""

    def __init__(self, name, args, rank=0):
        self.args = args
        import numpy as np
        import torch

        import synthetic
        from tensor_gemm_reduce_amd import gemm_rs as gr

        self.cfg = cfg = synthetic.CONFIGS[name]
        self.name = name
        self.rank = rank
        x, w, peers = synthetic.make_inputs(cfg, "normal")
        self.host_inputs = (x, w, peers)
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        self.x, self.w = d(x), d(w)
        self.peers = [d(p) for p in peers]
        z = lambda: torch.empty((cfg.S, cfg.N), dtype=torch.int16, device="cuda")
        self.send = [z() for _ in range(7)]
        self.local = z()
        self.out = z()
        self.op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, tile=args.tile,
                            num_reducers=args.reducers, reduce_mode=args.reduce_mode,
                            tile_stores=args.tile_stores)
        # where the fused launch sums the slice elsewhere than after the last
        # tile, the same launch with the sum after the last tile is timed beside it
        self.op_tail = None
        if self.op.info.reduce_mode != gr.REDUCE_TAIL:
            self.op_tail = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=rank, tile=args.tile,
                                     num_reducers=max(args.reducers, -1), reduce_mode="tail",
                                     tile_stores=args.tile_stores)
        self.gr = gr

    def run(self, mode):
        self.op.run(mode, self.x, self.w, self.send, self.peers, self.out, self.local)

    def run_tail(self):
        self.op_tail.run(self.gr.MODE_FUSED, self.x, self.w, self.send, self.peers, self.out, self.local)

    def matmul(self):
        import torch

        return torch.nn.functional.linear(self.x.view(torch.bfloat16), self.w.view(torch.bfloat16))


def time_each(fn, warmup, iters):
    """Per-launch durations (us) from event pairs on the current stream (host
    launch overhead included: for probes only)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) * 1e3 for s, e in ev]


class Replay:
    """fn captured `n` times back to back into one HIP graph.  The library keeps
    its run state on the device, so every replay is n new runs; replaying
    removes the host launch gaps that would dominate microsecond kernels."""

    def __init__(self, fn, n):
        import torch

        self.n = n
        fn()  # warm the code path outside capture
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for _ in range(n):
                fn()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()


def time_replays(fn, warmup, iters, per_graph=10):
    """Median over ceil(iters / per_graph) replays of the per-launch time (us)
    of a graph of per_graph back-to-back launches."""
    import torch

    g = Replay(fn, per_graph)
    reps = max(1, -(-iters // per_graph))
    for _ in range(max(1, -(-warmup // per_graph))):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for s, e in ev:
        s.record(stream)
        g.replay()
        e.record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) * 1e3 / per_graph for s, e in ev]


def time_interleaved(fns, warmup_s=0.3, rounds=20, per_graph=10):
    """Per-launch times (us) of several launch sequences measured side by side:
    each is captured as a graph of per_graph launches; the graphs are replayed
    in turn for about warmup_s seconds (clocks and caches settle), then for
    `rounds` rounds, each replaying every graph once (the order rotates from
    round to round) between events.  Returns {name: [us per launch, ...]}."""
    import torch

    graphs = {k: Replay(f, per_graph) for k, f in fns.items()}
    names = list(graphs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warmup_s:
        for k in names:
            graphs[k].replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = {k: [] for k in names}
    for r in range(rounds):
        order = names[r % len(names):] + names[:r % len(names)]
        for k in order:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            graphs[k].replay()
            e.record(stream)
            ev[k].append((s, e))
    torch.cuda.synchronize()
    return {k: [s.elapsed_time(e) * 1e3 / per_graph for s, e in v] for k, v in ev.items()}


def time_cold(fns, rounds=20, flush_bytes=512 << 20):
    """Per-launch times (us) with cold caches: before every launch a
    flush_bytes buffer (twice the 256 MiB last-level cache) is written on the
    same stream, outside the events that bracket the launch.  Launches are
    eager (one launch per event pair), in rotating order."""
    import torch

    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    names = list(fns)
    stream = torch.cuda.current_stream()
    for k in names:  # first launches (and the adaptive split's timing) untimed
        flush.fill_(0)
        fns[k]()
    torch.cuda.synchronize()
    ev = {k: [] for k in names}
    for r in range(rounds):
        order = names[r % len(names):] + names[:r % len(names)]
        for k in order:
            flush.fill_(r & 0xFF)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fns[k]()
            e.record(stream)
            ev[k].append((s, e))
    torch.cuda.synchronize()
    del flush
    return {k: [s.elapsed_time(e) * 1e3 for s, e in v] for k, v in ev.items()}


def summary(us):
    q = statistics.quantiles(us, n=10) if len(us) >= 2 else [us[0]] * 9
    return {"median_us": statistics.median(us), "mean_us": statistics.fmean(us), "p10_us": q[0],
            "p90_us": q[-1]}


def measure_case(c: Case, warmup, iters):
    gr = c.gr
    cfg = c.cfg
    fns = {
        "fused": lambda: c.run(gr.MODE_FUSED),
        "gemm": lambda: c.run(gr.MODE_GEMM_ONLY),
        "reduce": lambda: c.run(gr.MODE_REDUCE_ONLY),
        "seq": lambda: c.run(gr.MODE_SEQUENTIAL),
        "matmul": c.matmul,
    }
    if c.op_tail is not None:
        fns["fused_tail"] = c.run_tail
    t = time_interleaved(fns, rounds=max(4, -(-iters // 10)))
    fused, gemm, red, seq, mm = (summary(t[k]) for k in ("fused", "gemm", "reduce", "seq", "matmul"))
    st = c.op.status()
    if st != gr.OK:
        raise RuntimeError(f"{c.name}: device status {gr.gemm_rs_strerror(st)}")
    tf, tg, tr = fused["median_us"], gemm["median_us"], red["median_us"]
    extra = {}
    if c.op_tail is not None:
        tail = summary(t["fused_tail"])
        extra = {"T_fused_tail_us": tail, "overlap_tail": 1.0 - (tail["median_us"] - tg) / tr}
    if c.args.cold:
        tc = time_cold({k: fns[k] for k in ("fused", "gemm", "reduce")}, rounds=max(5, -(-iters // 10)))
        cf, cg, cr = (statistics.median(tc[k]) for k in ("fused", "gemm", "reduce"))
        if c.op.status() != gr.OK:
            raise RuntimeError(f"{c.name}: device status after the cold runs")
        extra["cold"] = {"T_fused_us": cf, "T_gemm_us": cg, "T_reduce_us": cr,
                         "fused_tflops": cfg.flops / cf * 1e-6, "overlap": 1.0 - (cf - cg) / cr}
    return {
        "shape": {"M": cfg.M, "N": cfg.N, "K_local": cfg.K_local, "tp": cfg.tp},
        "launch": c.op.info.as_dict(),
        "T_fused_us": fused, "T_gemm_us": gemm, "T_reduce_us": red, "T_seq_us": seq,
        "T_torch_linear_us": mm,
        "fused_tflops": cfg.flops / tf * 1e-6,
        "fused_pct_peak": 100.0 * cfg.flops / tf * 1e-6 / PEAK_BF16_TFLOPS,
        # the fused kernel's average launch duration (events around graph
        # replays of back-to-back launches) against the dense BF16 peak
        "roofline_frac": cfg.flops / tf * 1e-6 / PEAK_BF16_TFLOPS,
        "gemm_only_tflops": cfg.flops / tg * 1e-6,
        "reduce_gbs": cfg.reduce_bytes / tr * 1e-3,
        "reduce_pct_hbm": 100.0 * cfg.reduce_bytes / tr * 1e-3 / PEAK_HBM_GBS,
        "overlap": 1.0 - (tf - tg) / tr,
        "speedup_vs_sequential": seq["median_us"] / tf,
        "reduce_mode": {0: "auto", 1: "tail", 2: "coresident", 3: "stream", 4: "adaptive"}[c.op.info.reduce_mode],
        **extra,
    }


def check_case(c: Case, rows_per=3):
    """Untimed parity check on sampled rows against the oracle: `out` equals
    the oracle's slice sum of the GPU's local partial, and both the local
    slice and `out` are within 1e-2 of the FP64 reference and no worse than
    1.1x the unfused path's error (the vendor GEMM with BF16 output, then the
    slice sum)."""
    import numpy as np

    import oracle

    x, w, peers = c.host_inputs
    cfg = c.cfg
    c.run(c.gr.MODE_FUSED)
    import torch

    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, cfg.S - 1], rng.integers(0, cfg.S, rows_per)])).astype(np.int64)
    host = lambda t: t.cpu().numpy().view(np.uint16)
    local = host(c.local)[rows]
    out = host(c.out)[rows]
    prows = [p[rows] for p in peers]
    want_out = oracle.slice_sum(local, prows, tp=8)
    ref = oracle.ref_f64(x, w, None, tp=8, rank=c.rank, rows=rows)
    ref_out = oracle.ref_f64(x, w, peers, tp=8, rank=c.rank, rows=rows)
    err = lambda bits, r: float(np.max(np.abs(oracle.bf16_to_f32(bits) - r)) / np.max(np.abs(r)))
    err_local, err_out = err(local, ref), err(out, ref_out)
    # the unfused path: the vendor GEMM with BF16 output, then the slice sum
    y = c.matmul()[c.rank * cfg.S + torch.from_numpy(rows).cuda()]
    y_local = y.view(torch.int16).cpu().numpy().view(np.uint16)
    unf_local, unf_out = err(y_local, ref), err(oracle.slice_sum(y_local, prows, tp=8), ref_out)
    ok = (bool(np.array_equal(out, want_out)) and err_local <= 1e-2 and err_out <= 1e-2
          and err_local <= 1.1 * unf_local and err_out <= 1.1 * unf_out)
    return {"ok": ok, "rows": int(rows.size), "local_max_rel_err": err_local,
            "unfused_local_max_rel_err": unf_local, "out_max_rel_err": err_out,
            "unfused_out_max_rel_err": unf_out}


def cpu_baseline(c: Case, seconds):
    """The oracle as it stands, on the host cores, over whole rows of the same
    workload until about `seconds` have elapsed."""
    import numpy as np

    import oracle

    x, w, peers = c.host_inputs
    cfg = c.cfg
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(cores, int(omp)) if omp and omp.isdigit() else cores
    oracle.lib()
    t_total, rows_done, reps = 0.0, 0, 0
    S = cfg.S
    chunk = max(1, min(S, 64))
    start = 0
    while t_total < seconds and reps < 10_000:
        rows = (np.arange(chunk) + start) % S
        t0 = time.perf_counter()
        # whole path for these slice rows: all 8 destination row blocks of the
        # GEMM (routing) in one call (W is transposed once per call), the BF16
        # rounding and the slice sum
        part = oracle.f32_to_bf16(oracle.gemm_f32acc(x, w, rows=np.concatenate([d * S + rows for d in range(8)])))
        locals_ = part[c.rank * chunk:(c.rank + 1) * chunk]
        oracle.slice_sum(locals_, [p[rows] for p in peers], tp=8)
        t_total += time.perf_counter() - t0
        rows_done += chunk
        start += chunk
        reps += 1
    flops = 2.0 * rows_done * 8 * cfg.N * cfg.K_local
    return {"value": flops / t_total * 1e-12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} slice rows x 8 destination blocks of {c.name} (GEMM, BF16 rounding, "
                      f"routing, slice sum; one oracle GEMM call per {chunk} slice rows, which converts and "
                      f"transposes W once) in {t_total:.1f} s",
            "seconds": t_total}


def load_traffic(workload):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return t


COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes
TRAFFIC_LAUNCHES = 4


def traffic_probe(args):
    """A device-to-device copy of COPY_BYTES (the calibration kernel), then
    TRAFFIC_LAUNCHES fused launches of the workload, each synchronized."""
    import torch

    from tensor_gemm_reduce_amd import gemm_rs as gr

    src = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    c = Case(args.workload, args)
    for _ in range(TRAFFIC_LAUNCHES):
        c.run(gr.MODE_FUSED)
        torch.cuda.synchronize()
    log(f"traffic probe done: copy {COPY_BYTES} B, {TRAFFIC_LAUNCHES} fused launches of {args.workload}")


def counter_probe(args):
    """Two launches each of the GEMM-only kernel, the fused kernel and
    hipBLASLt's GEMM of the same product, each synchronized."""
    import torch

    from tensor_gemm_reduce_amd import gemm_rs as gr

    c = Case(args.workload, args)
    for fn in (lambda: c.run(gr.MODE_GEMM_ONLY), lambda: c.run(gr.MODE_FUSED), c.matmul):
        for _ in range(2):
            fn()
            torch.cuda.synchronize()
    log(f"counter probe done: {args.workload}")


def counters_from(paths):
    """Per-kernel means of rocprofv3 counter-collection CSVs (one table row
    per kernel and counter pass), for kernels that ran at least 100 us."""
    import collections
    import csv

    acc = collections.OrderedDict()
    for path in paths:
        per = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            e = per.setdefault(key, {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
        for (_, name), e in per.items():
            if e["dur"] < 100:
                continue
            short = name if len(name) <= 90 else name[:40] + "..." + name[-47:]
            a = acc.setdefault(short, {})
            for k, v in e.items():
                a.setdefault(k, []).append(v)
    for name, a in acc.items():
        print(f"**{name}**\n")
        print("| counter | mean per launch |")
        print("|---|---|")
        for k, v in a.items():
            print(f"| {'duration us (under counters)' if k == 'dur' else k} | {sum(v) / len(v):.4g} |")
        print()


def traffic_from(args):
    """HBM bytes per fused launch from the FETCH_SIZE and WRITE_SIZE passes,
    each scaled by what the same counter reads for the copy of known size."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "fused_kernel" not in r["Kernel_Name"]]
        fused = [float(r["Counter_Value"]) for r in rows if "fused_kernel" in r["Kernel_Name"]]
        if not copy or not fused:
            raise SystemExit(f"{path}: no {counter} rows for the copy and the fused kernel")
        # the copy is the largest other dispatch; later launches of the fused
        # kernel see warm caches, as in the timed runs
        return max(copy), statistics.median(fused[1:] if len(fused) > 1 else fused)

    copy_f, fused_f = per_kernel(args.traffic_from[0], "FETCH_SIZE")
    copy_w, fused_w = per_kernel(args.traffic_from[1], "WRITE_SIZE")
    # counters are in KiB; the copy reads and writes COPY_BYTES each
    k_fetch = copy_f * 1024.0 / COPY_BYTES
    k_write = copy_w * 1024.0 / COPY_BYTES
    t = {"workload": args.workload, "source_digest": source_digest(),
         "fetch_bytes": fused_f * 1024.0 / k_fetch, "write_bytes": fused_w * 1024.0 / k_write,
         "fetch_kib_raw": fused_f, "write_kib_raw": fused_w,
         "copy_fetch_factor": k_fetch, "copy_write_factor": k_write, "copy_bytes": COPY_BYTES}
    out = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t))


SPLIT_KNOBS = (
    [dict(reduce_mode="tail")] + [dict(num_reducers=r) for r in (2, 4, 8, 12, 16, 24, 32, 64)]
    + [dict(reduce_mode="stream"), dict(reduce_mode="adaptive")]
    + [dict(reduce_mode="tail", flag_stride=32), dict(num_reducers=8, flag_stride=32)]
    + [dict(reduce_mode="tail", tile_stores=0), dict(num_reducers=8, tile_stores=0)]
    + [dict(reduce_mode="tail", tile_stores=1), dict(num_reducers=8, tile_stores=1)]
    + [dict(reduce_mode="tail", flag_protocol=1), dict(num_reducers=8, flag_protocol=1)]
)


def split_sweep(args):
    """Fused launch times of one workload over the reducer placements and the
    flag layout, side by side with the GEMM-only launch and the standalone
    reduce (one set of buffers, one handle per setting).  Every setting's
    `out` must equal the default setting's bit for bit (same sum order)."""
    import torch

    from tensor_gemm_reduce_amd import gemm_rs as gr

    base = Case(args.workload, args)
    cfg = base.cfg
    ops = []
    for kw in SPLIT_KNOBS:
        try:
            op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=base.rank, tile=args.tile, **kw)
        except gr.GemmRSError as e:  # (the stream needs the 256x256 tile)
            log(f"[{args.workload}] {kw}: {e}")
            continue
        ops.append((kw, op))
    run = lambda op, mode: op.run(mode, base.x, base.w, base.send, base.peers, base.out, base.local)
    base.run(gr.MODE_FUSED)
    torch.cuda.synchronize()
    want = base.out.clone()
    same = []
    for kw, op in ops:
        base.out.zero_()
        run(op, gr.MODE_FUSED)
        torch.cuda.synchronize()
        same.append(bool(torch.equal(base.out, want)))
    fns = {"gemm": lambda: base.run(gr.MODE_GEMM_ONLY), "reduce": lambda: base.run(gr.MODE_REDUCE_ONLY)}
    for i, (kw, op) in enumerate(ops):
        fns[f"k{i}"] = (lambda o: (lambda: run(o, gr.MODE_FUSED)))(op)
    t = time_interleaved(fns, rounds=max(4, args.steps // 20))
    tg, tr = statistics.median(t["gemm"]), statistics.median(t["reduce"])
    rows = []
    for i, (kw, op) in enumerate(ops):
        st = op.status()
        tf = statistics.median(t[f"k{i}"])
        rows.append({**kw, "flag_stride": kw.get("flag_stride", 1),
                     "tile_stores": op.info.tile_stores,
                     "flag_protocol": kw.get("flag_protocol", 0),
                     "compute_wgs": op.info.compute_wgs, "reducer_wgs": op.info.reducer_wgs,
                     "T_fused_us": tf, "fused_tflops": cfg.flops / tf * 1e-6,
                     "overlap": 1.0 - (tf - tg) / tr, "out_matches_default": same[i],
                     "status": gr.gemm_rs_strerror(st)})
        log(f"[{args.workload}] {kw}: {tf:.1f} us, overlap {rows[-1]['overlap']:.2f}, same={same[i]}, "
            f"status={rows[-1]['status']}")
    res = {"workload": args.workload, "T_gemm_us": tg, "T_reduce_us": tr, "launch": base.op.info.as_dict(),
           "rows": rows, "source_digest": source_digest()}
    with open(args.split_sweep, "w") as f:
        json.dump(res, f, indent=1)
    if not all(same) or any(r["status"] != gr.gemm_rs_strerror(gr.OK) for r in rows):
        raise RuntimeError("a setting changed the result or reported an error")


def timeline_summary(op, cfg, kernel_us):
    """Per-launch figures from a traced fused run's slot log and slice-sum
    stamps (100 MHz counter; times in us from the launch's first workgroup)."""
    import numpy as np

    log_, _, stamps, launch = op.debug_read(sums=True)
    info = op.info
    t0 = int(launch[0])
    rel = lambda v: ((np.asarray(v, np.int64) - t0) % (1 << 32)) / 100.0
    release = rel(log_[:, 2])              # per schedule slot
    flag_of_slot = log_[:, 0].astype(np.int64)
    gemm_end = float(release.max())
    ts, ipt = info.tiles_per_slice, info.bm * info.bn // 512
    own_first = op.cfg.rank * ts
    slot_of_flag = {int(f): q for q, f in enumerate(flag_of_slot)}
    own_release = np.array([release[slot_of_flag[own_first + t]] for t in range(ts)])
    acq, done, items = rel(stamps[:, 1]), rel(stamps[:, 2]), stamps[:, 3].astype(np.int64)
    launch_end = float(rel(launch[2]))
    G = info.compute_wgs
    rounds = []
    for r in range((info.tiles + G - 1) // G):
        sl = slice(r * G, min((r + 1) * G, info.tiles))
        lo, hi = float(release[sl].min()), float(release[sl].max())
        prev = rounds[-1]["release_last_us"] if rounds else 0.0
        in_win = (done > prev) & (done <= hi)
        rounds.append({"round": r, "release_first_us": lo, "release_last_us": hi,
                       "own_tiles_released": int(np.sum((own_release > prev) & (own_release <= hi))),
                       "sum_items_done_pct": 100.0 * float(items[in_win].sum()) / max(1, ts * ipt)})
    before = 100.0 * float(items[done <= gemm_end].sum()) / max(1, ts * ipt)
    return {"kernel_us": kernel_us, "launch_span_us": launch_end, "gemm_last_release_us": gemm_end,
            "sum_before_gemm_end_pct": before, "sum_end_after_gemm_us": float(done.max()) - gemm_end,
            "median_release_to_acquire_us": float(np.median(acq - own_release)),
            "median_acquire_to_done_us": float(np.median(done - acq)),
            "items_ok": bool(np.all(items == ipt)), "rounds": rounds}


def timeline(args):
    """One traced fused launch per reduce placement of a workload, after an
    untraced timing of the same placement; writes a markdown summary."""
    import torch

    from tensor_gemm_reduce_amd import gemm_rs as gr

    base = Case(args.workload, args)
    cfg = base.cfg
    rows = {}
    for mode in ("tail", "stream", "adaptive"):
        try:
            op = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=base.rank, tile=args.tile, reduce_mode=mode,
                           debug_flags=gr.DEBUG_TRACE)
            plain = gr.GemmRS(cfg.M, cfg.N, cfg.K_local, rank=base.rank, tile=args.tile, reduce_mode=mode)
        except gr.GemmRSError as e:
            log(f"[{args.workload}] {mode}: {e}")
            continue
        run = lambda o: o.run(gr.MODE_FUSED, base.x, base.w, base.send, base.peers, base.out, base.local)
        t = time_interleaved({"k": lambda: run(plain)}, rounds=8)
        for _ in range(3):
            run(op)
        torch.cuda.synchronize()
        if op.status() != gr.OK:
            raise RuntimeError(f"{mode}: device status {gr.gemm_rs_strerror(op.status())}")
        rows[mode] = timeline_summary(op, cfg, statistics.median(t["k"]))
        log(f"[{args.workload}] {mode}: " + json.dumps({k: v for k, v in rows[mode].items() if k != "rounds"}))
    cmd = " ".join(["python3", "bench.py"] + sys.argv[1:])
    L = [f"# Slice-sum timeline, {args.workload}", "",
         f"Command (on the GPU host, from the repository root): `{cmd}`", "",
         "One traced fused launch per reduce placement (after three warm-up launches), read back with "
         "`gemm_rs_debug_read`: the slot log's release times and the slice-sum stamps of the own tiles "
         "(100 MHz counter; times in us from the launch's first workgroup start). `kernel us` is the same "
         "placement's untraced launch time (interleaved graph replays). `sum before GEMM end` is the share "
         "of the slice's items in own tiles whose last sum store precedes the GEMM's last tile release.",
         f"Library source digest: {source_digest()}.", "",
         "| placement | kernel us | GEMM last release us | launch span us | sum before GEMM end | "
         "sum end after GEMM us | median release to acquire us | median acquire to done us |",
         "|---|---|---|---|---|---|---|---|"]
    for mode, r in rows.items():
        L.append(f"| {mode} | {r['kernel_us']:.1f} | {r['gemm_last_release_us']:.1f} | {r['launch_span_us']:.1f} | "
                 f"{r['sum_before_gemm_end_pct']:.1f}% | {r['sum_end_after_gemm_us']:.1f} | "
                 f"{r['median_release_to_acquire_us']:.1f} | {r['median_acquire_to_done_us']:.1f} |")
    for mode, r in rows.items():
        L += ["", f"Per GEMM round, {mode} (rounds of {base.op.info.compute_wgs} slots; the sum's items counted "
                  "in the round whose release window holds their last store):", "",
              "| round | first release us | last release us | own tiles released | sum items done |",
              "|---|---|---|---|---|"]
        for x in r["rounds"]:
            L.append(f"| {x['round']} | {x['release_first_us']:.1f} | {x['release_last_us']:.1f} | "
                     f"{x['own_tiles_released']} | {x['sum_items_done_pct']:.1f}% |")
        tail_pct = 100.0 - sum(x["sum_items_done_pct"] for x in r["rounds"])
        L.append(f"| after | | | | {tail_pct:.1f}% |")
    with open(args.timeline, "w") as f:
        f.write("\n".join(L) + "\n")
    if not all(r["items_ok"] for r in rows.values()):
        raise RuntimeError("an own tile's item count is off")


def allreduce_sweep(args):
    """GEMM + all-reduce per benchmark shape: the fused launch with the gather
    stores, side by side with the GEMM-only launch, the standalone reduce with
    the gather stores, the reduce-scatter alone (fused, no gather) and
    hipBLASLt's GEMM.  Algorithmic bytes of the all-reduce's sum: 8 reads and
    1 + 7 writes of 2 bytes per slice element, 4*M*N."""
    import torch

    rows = {}
    for name in SWEEP:
        c = Case(name, args)
        cfg = c.cfg
        gr = c.gr
        gather = [torch.empty_like(c.out) for _ in range(7)]
        ar = lambda mode: c.op.run(mode, c.x, c.w, c.send, c.peers, c.out, c.local, gather=gather)
        ar(gr.MODE_FUSED)
        torch.cuda.synchronize()
        same = all(torch.equal(g, c.out) for g in gather)
        t = time_interleaved({"fused_ar": lambda: ar(gr.MODE_FUSED), "gemm": lambda: c.run(gr.MODE_GEMM_ONLY),
                              "reduce_ar": lambda: ar(gr.MODE_REDUCE_ONLY), "fused_rs": lambda: c.run(gr.MODE_FUSED),
                              "matmul": c.matmul}, rounds=max(4, args.steps // 20))
        st = c.op.status()
        med = {k: statistics.median(v) for k, v in t.items()}
        ar_bytes = 4.0 * cfg.M * cfg.N
        rows[name] = {
            "shape": {"M": cfg.M, "N": cfg.N, "K_local": cfg.K_local},
            "T_fused_ar_us": med["fused_ar"], "T_gemm_us": med["gemm"], "T_reduce_ar_us": med["reduce_ar"],
            "T_fused_rs_us": med["fused_rs"], "T_torch_linear_us": med["matmul"],
            "fused_ar_tflops": cfg.flops / med["fused_ar"] * 1e-6,
            "fused_ar_pct_peak": 100.0 * cfg.flops / med["fused_ar"] * 1e-6 / PEAK_BF16_TFLOPS,
            "reduce_ar_gbs": ar_bytes / med["reduce_ar"] * 1e-3,
            "overlap_ar": 1.0 - (med["fused_ar"] - med["gemm"]) / med["reduce_ar"],
            "speedup_vs_unfused": (med["matmul"] + med["reduce_ar"]) / med["fused_ar"],
            "gather_equals_out": same, "status": gr.gemm_rs_strerror(st),
        }
        log(f"[{name}] all-reduce: " + json.dumps({k: rows[name][k] for k in
                                                   ("T_fused_ar_us", "T_gemm_us", "T_reduce_ar_us", "overlap_ar",
                                                    "gather_equals_out")}))
        del c, gather
        torch.cuda.empty_cache()
    with open(args.allreduce_sweep, "w") as f:
        json.dump({"rows": rows, "source_digest": source_digest()}, f, indent=1)
    if not all(r["gather_equals_out"] and r["status"] == "success" for r in rows.values()):
        raise RuntimeError("an all-reduce run reported an error or a gather buffer differs from out")


AG_SWEEP = ("ag_qkv", "ag_gate_up", "ag_mixtral_w13", "ag_large_prefill")


def allgather_sweep(args):
    """All-gather + GEMM (the column-parallel layer) per layer shape: the fused
    launch side by side with the GEMM over an already gathered buffer, the
    standalone all-gather copy, the two in sequence and hipBLASLt's GEMM on
    the gathered activations.  Algorithmic bytes of the all-gather: the tp-1
    peer slices read and written, 2 * (tp-1) * S * K * 2."""
    import numpy as np
    import torch

    import synthetic
    from tensor_gemm_reduce_amd import gemm_rs as gr

    rows = {}
    for name in AG_SWEEP:
        cfg = synthetic.AG_CONFIGS[name]
        xs, w = synthetic.make_ag_inputs(cfg, "normal")
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        xs_d = [d(x) for x in xs]
        w_d = d(w)
        xg = torch.empty((cfg.M, cfg.K), dtype=torch.int16, device="cuda")
        y = torch.empty((cfg.M, cfg.N), dtype=torch.int16, device="cuda")
        op = gr.GemmRS(cfg.M, cfg.N, cfg.K, rank=0, tile=args.tile)
        run = lambda mode: op.run_allgather(mode, xs_d, w_d, xg, y)
        run(gr.MODE_FUSED)
        torch.cuda.synchronize()
        gathered_ok = all(torch.equal(xg[i * cfg.S:(i + 1) * cfg.S], xs_d[i]) for i in range(cfg.tp))
        mm = lambda: torch.nn.functional.linear(xg.view(torch.bfloat16), w_d.view(torch.bfloat16))
        t = time_interleaved({"fused": lambda: run(gr.MODE_FUSED), "gemm": lambda: run(gr.MODE_GEMM_ONLY),
                              "copy": lambda: run(gr.MODE_REDUCE_ONLY), "seq": lambda: run(gr.MODE_SEQUENTIAL),
                              "matmul": mm}, rounds=max(4, args.steps // 20))
        st = op.status()
        med = {k: statistics.median(v) for k, v in t.items()}
        rows[name] = {
            "shape": {"M": cfg.M, "N": cfg.N, "K": cfg.K}, "launch": op.info.as_dict(),
            "T_fused_us": med["fused"], "T_gemm_us": med["gemm"], "T_copy_us": med["copy"], "T_seq_us": med["seq"],
            "T_torch_linear_us": med["matmul"],
            "fused_tflops": cfg.flops / med["fused"] * 1e-6,
            "fused_pct_peak": 100.0 * cfg.flops / med["fused"] * 1e-6 / PEAK_BF16_TFLOPS,
            "copy_gbs": cfg.gather_bytes / med["copy"] * 1e-3,
            "overlap": 1.0 - (med["fused"] - med["gemm"]) / med["copy"],
            "speedup_vs_sequential": med["seq"] / med["fused"],
            "gathered_ok": gathered_ok, "status": gr.gemm_rs_strerror(st),
        }
        log(f"[{name}] all-gather: " + json.dumps({k: rows[name][k] for k in
                                                   ("T_fused_us", "T_gemm_us", "T_copy_us", "overlap",
                                                    "gathered_ok")}))
        op.close()
        del xs_d, w_d, xg, y
        torch.cuda.empty_cache()
    with open(args.allgather_sweep, "w") as f:
        json.dump({"rows": rows, "source_digest": source_digest()}, f, indent=1)
    if not all(r["gathered_ok"] and r["status"] == "success" for r in rows.values()):
        raise RuntimeError("an all-gather run reported an error or gathered wrong rows")


def stats_summary(path):
    """Markdown table of rocprofv3's per-kernel statistics (durations in us)."""
    import csv

    rows = list(csv.DictReader(open(path)))
    print("| kernel | calls | average us | min us | max us |")
    print("|---|---|---|---|---|")
    for r in rows:
        name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} |")


def main():
    args = parse()
    if args.counters_from:
        counters_from(args.counters_from)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of a TP=8 layer on a single GPU; --gpus {args.gpus} "
              "is not supported (the library runs one GPU; sharding across GPUs is a design only).", file=sys.stderr)
        sys.exit(2)
    import torch

    from tensor_gemm_reduce_amd import gemm_rs as gr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    if args.traffic_probe:
        traffic_probe(args)
        return
    if args.counter_probe:
        counter_probe(args)
        return
    if args.split_sweep:
        split_sweep(args)
        return
    if args.timeline:
        timeline(args)
        return
    if args.allreduce_sweep:
        allreduce_sweep(args)
        return
    if args.allgather_sweep:
        allgather_sweep(args)
        return
    c = Case(args.workload, args)
    cfg = c.cfg
    check = check_case(c) if args.check else None
    log(f"[{args.workload}] parity check: {check}")

    # timed region: exactly K fused steps (one replay of a graph of K
    # back-to-back launches), synchronized on both sides; HIP events on the
    # replay stream give the average launch duration
    steps = Replay(lambda: c.run(gr.MODE_FUSED), args.steps)
    for _ in range(max(1, -(-args.warmup // args.steps))):
        steps.replay()
    torch.cuda.synchronize()
    # and at least 0.3 s of the same work, so that clocks have settled
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.3:
        steps.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    steps.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = c.op.status()
    if st != gr.OK:
        raise RuntimeError(f"device status {gr.gemm_rs_strerror(st)}")
    mean_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    ms_per_step = wall / args.steps * 1e3
    value = cfg.flops * args.steps / wall * 1e-12
    log(f"[{args.workload}] fused: {mean_us:.2f} us/launch (events), {ms_per_step * 1e3:.2f} us/step (wall)")

    m = measure_case(c, args.warmup, args.steps)
    log(f"[{args.workload}] " + json.dumps({k: m[k] for k in ("fused_tflops", "overlap", "reduce_gbs")}))

    traffic = load_traffic(args.workload)
    achieved = cfg.flops / mean_us * 1e-6
    roofline = {
        "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS,
        "traffic": (traffic["fetch_bytes"] + traffic["write_bytes"]) if traffic else None,
        "kernel": f"fused_kernel ({c.op.info.bm}x{c.op.info.bn} tile)", "algorithmic_flops_per_launch": cfg.flops,
        "avg_launch_us": mean_us,
    }
    cpu = cpu_baseline(c, args.cpu_seconds) if args.cpu else None

    sweep = {}
    if args.sweep:
        for name in SWEEP:
            if name == args.workload:
                sweep[name] = dict(m, parity=check)
                continue
            try:
                sc = Case(name, args)
                sweep[name] = measure_case(sc, args.warmup, args.steps)
                sweep[name]["parity"] = check_case(sc) if args.check else None
                del sc
                torch.cuda.empty_cache()
                log(f"[{name}] " + json.dumps({k: sweep[name][k] for k in
                                               ("fused_tflops", "fused_pct_peak", "overlap", "reduce_gbs")}))
            except Exception as e:  # report, keep the headline line
                sweep[name] = {"error": repr(e)}
                log(f"[{name}] error: {e!r}")
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            json.dump({args.workload: m, **sweep, "source_digest": source_digest()}, f, indent=1)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {cfg.description}; M={cfg.M} N={cfg.N} "
                               f"K_local={cfg.K_local} tp={cfg.tp}, rank 0, bf16 in / fp32 accumulate",
                   "global_batch": cfg.M, "parallelism": "tp8 (one rank simulated)"},
        "pct_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "overlap": m["overlap"],
        "T_fused_us": m["T_fused_us"]["median_us"], "T_gemm_us": m["T_gemm_us"]["median_us"],
        "T_reduce_us": m["T_reduce_us"]["median_us"],
        "reduce_gbs": m["reduce_gbs"],
        "reduce_mode": m["reduce_mode"],
        "tile_stores": {gr.STORES_DEVICE: "device", gr.STORES_NONTEMPORAL: "nt"}[c.op.info.tile_stores],
        "cold": m.get("cold"),
        "T_fused_tail_us": (m.get("T_fused_tail_us") or {}).get("median_us"),
        "overlap_tail": m.get("overlap_tail"),
        "parity": check,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": {k: ({"fused_tflops": v.get("fused_tflops"), "fused_pct_peak": v.get("fused_pct_peak"),
                       "roofline_frac": v.get("roofline_frac"),
                       "overlap": v.get("overlap"), "T_fused_us": v.get("T_fused_us", {}).get("median_us"),
                       "T_gemm_us": v.get("T_gemm_us", {}).get("median_us"),
                       "T_reduce_us": v.get("T_reduce_us", {}).get("median_us"),
                       "reduce_gbs": v.get("reduce_gbs"),
                       "T_torch_linear_us": v.get("T_torch_linear_us", {}).get("median_us"),
                       "reduce_mode": v.get("reduce_mode"),
                       "T_fused_tail_us": (v.get("T_fused_tail_us") or {}).get("median_us"),
                       "overlap_tail": v.get("overlap_tail"),
                       "cold": v.get("cold"),
                       "parity_ok": (v.get("parity") or {}).get("ok")} if "error" not in v else v)
                  for k, v in sweep.items()},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "hip": torch.version.hip},
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
