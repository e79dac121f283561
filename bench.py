"""Benchmark of the DualQuant BCD solver on one MI355X.

Default workload: the whole Llama-3.1-8B linear-layer set (32 layers x q,
k, v, o, gate, up, down; 224 matrices, 6.98 G bf16 weights, 13.96 GB,
resident in HBM; N(0, 0.02^2) with 1 % outlier columns x 20; INT4 codes,
G = 64, fp16 block and column scales, T = 20 iterations). A step solves
every matrix of the set (absmax start, T iterations, packed codes; one
dq_solve each), the matrices spread over --streams streams.

value = set elements * T / step time: weight elements per second per BCD
iteration, whole job (start and packing included). The roofline entry is
for the dominant kernel, the BCD pass, on the dominant shape (gate/up,
14336 x 4096, 54 % of the set's elements): its algorithmic bytes per
launch (one read of W plus a read and a write of the block scales and the
column scales) over its average duration, measured in this run with events
on the stream it runs on, around the T passes of solves of one resident
gate matrix after the timed steps. cpu_baseline times the float64 oracle (test
infrastructure, never on the product path) on the whole of layer 0 with a
pool of worker processes.

--workload NAME selects a single-matrix workload instead (other shapes and
formats; --init colnorm starts each solve from the column-norm start), with
the same step (one whole solve) and the roofline of its own pass kernel, or
an activation workload act_... (a step is one dq_rescale_quantize_act of a
whole token batch; metric: activation elements/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
(defaults: K = 10 timed steps after W = 2 warm-up steps for the layer set;
K = 100 after W = 200 for a single matrix or an activation batch).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def alg_bytes_per_elem(w_bytes: int, a_bytes: int, G: int, rows: int) -> float:
    """One read of W, a read and a write of the block scales, a read and a
    write of the column scales (2 bytes each, amortized over the rows)."""
    return w_bytes + 2.0 * a_bytes / G + 4.0 / rows


def cpu_baseline(wl, data, budget_s: float = 30.0):
    """Time the float64 oracle on the same workload (whole matrix when it
    fits the budget, else a prefix of whole column stripes)."""
    from oracle import dualquant as D
    from calibration_free_bit_amd import synth

    W = synth.bf16_to_f64(data) if data.dtype.name == "uint16" else data.astype("float64")
    fmt = D.FORMATS[wl.fmt]
    # calibrate on 2 stripes, then size the sample
    G = fmt.group
    t0 = time.perf_counter()
    D.solve(W[:, :2 * G], fmt, wl.iters)
    rate = 2 * G * W.shape[0] * wl.iters / (time.perf_counter() - t0)
    n_str = W.shape[1] // G
    k = max(2, min(n_str, int(budget_s * 0.6 * rate / (G * W.shape[0] * wl.iters))))
    Ws = W[:, :k * G]
    # repeat the sample until about 10 s of CPU work have been timed
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while reps == 0 or dt < 10.0:
        D.solve(Ws, fmt, wl.iters)
        reps += 1
        dt = time.perf_counter() - t0
    sample = (f"float64 numpy oracle, {'whole matrix' if k == n_str else f'first {k} of {n_str} column stripes'}"
              f" ({Ws.shape[0]}x{Ws.shape[1]}), T={wl.iters}, {reps} solve(s) in {dt:.1f} s")
    return {"value": Ws.size * wl.iters * reps / dt, "unit": "elements/s", "cores": 1,
            "kind": "oracle", "sample": sample}


def kernel_source_hash() -> str:
    """Hash of the HIP sources; counter-based traffic is reported only while
    it matches the hash recorded with the counters."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "calibration_free_bit_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def profile_stem(workload: str) -> str:
    """File stem of a workload's rocprofv3 summaries in profiles/: the
    profiled kernel, then the workload."""
    if workload.startswith("act_"):
        return "act_quant_" + workload[len("act_"):]
    return f"bcd_pass_{workload}"


def counters_json(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{profile_stem(workload)}_counters.json")


def recorded_traffic(workload: str):
    """Bytes moved per pass launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE measurement, or None if absent or taken on other sources."""
    try:
        rec = json.load(open(counters_json(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def recorded_valu(workload: str):
    """VALU lane operations per pass launch from the committed rocprofv3
    SQ_INSTS_VALU measurement (wave instructions x 64), or None."""
    try:
        rec = json.load(open(counters_json(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    v = rec.get("valu_insts_per_launch")
    return None if v is None else 64.0 * v


#: Non-packed VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
#: (one wave64 instruction per SIMD every 4 cycles).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def copy_calibration(nbytes: int = 256 << 20, reps: int = 3):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of the profiled kernels."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


SET_WORKLOAD = "llama31_8b_int4_g64_bf16"


def _make_set_matrix(item):
    from calibration_free_bit_amd import synth
    l, p, name, spec, seed = item
    return l, p, synth.make_matrix(spec, seed).data


#: Columns per task of the set's oracle baseline (whole stripes of G = 64).
SET_BASELINE_CHUNK_COLS = 512


def _oracle_chunk(task):
    """Worker of the set's oracle baseline: the float64 oracle on one column
    block (whole stripes) of one matrix, T iterations; returns its elements."""
    from calibration_free_bit_amd import synth
    from oracle import dualquant as D
    bits, iters = task
    W = synth.bf16_to_f64(bits)
    D.solve(W, D.FORMATS["int4_g64"], iters)
    return W.size


def set_cpu_baseline(pool, n_proc: int, layer0, iters: int):
    """The float64 oracle on the whole of layer 0 (its seven matrices, 218 M
    weights), split into blocks of whole column stripes -- which the method
    solves independently of each other, so the blocks together are exactly
    the layer's solve -- on a pool of n_proc worker processes (forked before
    the GPU was touched). Reported as elements/s per iteration; the full set
    is 32 such layers ("x32 extrapolated" for its time)."""
    tasks = []
    for name, bits in layer0:
        for c0 in range(0, bits.shape[1], SET_BASELINE_CHUNK_COLS):
            tasks.append((name, bits[:, c0:c0 + SET_BASELINE_CHUNK_COLS]))
    # largest blocks first, so the pool drains evenly
    tasks.sort(key=lambda t: -t[1].size)
    t0 = time.perf_counter()
    n = sum(pool.imap_unordered(_oracle_chunk, [(b, iters) for _, b in tasks], chunksize=1))
    dt = time.perf_counter() - t0
    rate = n * iters / dt
    shapes = ", ".join(f"{nm} {b.shape[0]}x{b.shape[1]}" for nm, b in layer0)
    return {"value": rate, "unit": "elements/s", "cores": n_proc, "kind": "oracle",
            "sample": f"float64 numpy oracle on all of layer 0 ({shapes}; {n} weights) in "
                      f"{len(tasks)} blocks of up to {SET_BASELINE_CHUNK_COLS} columns, T={iters}, "
                      f"{n_proc} worker processes (host affinity {len(os.sched_getaffinity(0))} cores), "
                      f"{dt:.1f} s; x32 extrapolated, the whole set would take "
                      f"{32 * n * iters / rate:.0f} s"}


def baseline_workers() -> int:
    """Worker processes for host-side work: the cores this process may run
    on, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_set(args):
    """The whole Llama-3.1-8B linear set on one GPU, spread over streams."""
    import multiprocessing as mp

    import numpy as np

    from calibration_free_bit_amd import synth
    items = synth.llama_layer_specs()
    # host generation and the oracle baseline in worker processes forked
    # before the GPU is touched
    n_proc = baseline_workers()
    pool = mp.get_context("fork").Pool(n_proc)
    t_gen = time.perf_counter()
    host = {}
    for l, p, data in pool.imap_unordered(_make_set_matrix, items, chunksize=1):
        host[(l, p)] = data
    t_gen = time.perf_counter() - t_gen
    T = 20
    baseline = None
    if not args.no_cpu_baseline:
        layer0 = [(name, host[(l, p)]) for (l, p, name, _, _) in items if l == 0]
        baseline = set_cpu_baseline(pool, n_proc, layer0, T)
    pool.close()
    pool.join()

    import torch
    from calibration_free_bit_amd import dq
    fmt = dq.FORMATS["int4_g64"]
    solvers = []
    for (l, p, name, spec, seed) in items:
        W = torch.from_numpy(host.pop((l, p)).view(np.int16)).to("cuda:0")
        solvers.append(dq.Solver(W, fmt))
    torch.cuda.synchronize()
    elems = sum(s.W.numel() for s in solvers)
    streams = [torch.cuda.Stream() for _ in range(args.streams)]
    cur = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dq.solve_on_streams(solvers, T, streams)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(cur)
    for _ in range(args.steps):
        dq.solve_on_streams(solvers, T, streams)
    e1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    value = elems * T / (step_ms * 1e-3)
    b_step = alg_bytes_per_elem(2, 2, fmt.group, 4096)
    step_gbs = value * b_step / 1e9  # whole step, start and packing included

    # the dominant kernel on the dominant shape: the T passes of a solve of
    # layer 0's gate matrix (14336 x 4096) from the absmax start, alone on
    # the current stream, timed with events on that stream around
    # dq_bcd_iterate(T) (each T includes one final column update)
    gate = solvers[[k for k, it in enumerate(items) if it[2] == "gate"][0]]
    M, N = gate.W.shape
    reps = max(3, args.steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r0, r1 in ev:
        gate.init()
        r0.record(cur)
        gate.iterate(T)
        r1.record(cur)
    torch.cuda.synchronize()
    pass_s = sum(r0.elapsed_time(r1) for r0, r1 in ev) * 1e-3 / (reps * T)
    b_pass = alg_bytes_per_elem(2, 2, fmt.group, M)
    achieved = b_pass * M * N / pass_s / 1e9
    dom = f"int4_g64_{M}x{N}_bf16"
    out = {
        "metric": "weight elements/s per BCD iteration",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32-requant/f64-sums",
        "data": "synthetic (seeded, numpy PCG64)",
        "config": {"workload": SET_WORKLOAD, "matrices": len(solvers), "elements": elems,
                   "format": "int4_g64", "iters": T, "streams": args.streams,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(dom),
                     "kernel": f"bcd_pass_kernel on the gate/up shape {M}x{N} INT4-G64 (layer 0 gate)",
                     "alg_bytes_per_elem": b_pass, "avg_launch_us": pass_s * 1e6,
                     "launches": reps * T, "counters": f"profiles/{profile_stem(dom)}_counters.json"},
        "valu": valu_entry(recorded_valu(dom), pass_s, M * N),
        "whole_step": {"achieved": step_gbs, "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                       "alg_bytes_per_elem": b_step,
                       "note": "every kernel of the set, overlapped on the streams"},
        "breakdown_ms": {"wall_per_step": wall * 1e3 / args.steps, "host_generation_s": t_gen},
    }
    if baseline is not None:
        out["cpu_baseline"] = baseline
    print(json.dumps(out))


def _step_counts(args, steps: int, warmup: int) -> None:
    """Fill in the workload's default step counts and check them."""
    args.steps = steps if args.steps is None else args.steps
    args.warmup = warmup if args.warmup is None else args.warmup
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: single matrix 100 timed steps after 200 warm-up steps (the
    # clocks settle within the warm-up; together ~0.1 s of device time);
    # the layer set 10 after 2
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=SET_WORKLOAD)
    ap.add_argument("--streams", type=int, default=2, help="streams of the Llama set workload")
    ap.add_argument("--init", choices=("rtn", "colnorm"), default="rtn",
                    help="start of a single-matrix solve: absmax (default) or the column-norm start")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (for scaling byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark measures one GPU; "
              "the solver shards by column stripes with no communication",
              file=sys.stderr)
        sys.exit(2)

    from calibration_free_bit_amd import synth as _synth
    known = [SET_WORKLOAD, *_synth.WORKLOADS, *_synth.ACT_WORKLOADS]
    if args.workload not in known:
        print(f"bench.py: unknown workload {args.workload!r}; one of: {', '.join(known)}",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == SET_WORKLOAD:
        _step_counts(args, steps=10, warmup=2)
        run_set(args)
        return
    if args.workload.startswith("act_"):
        _step_counts(args, steps=100, warmup=200)
        run_act(args)
        return
    _step_counts(args, steps=100, warmup=200)

    import numpy as np
    import torch

    from calibration_free_bit_amd import dq, synth

    wl = synth.WORKLOADS[args.workload]
    fmt = dq.FORMATS[wl.fmt]
    m = synth.make_matrix(wl.spec, wl.seeds[0])
    data = m.data
    host = torch.from_numpy(data.view(np.int16) if data.dtype == np.uint16 else data)
    W = host.to("cuda:0")
    s = dq.Solver(W, fmt)
    M, N = W.shape
    T = wl.iters
    st = torch.cuda.current_stream()
    colnorm = args.init == "colnorm"
    init = s.init_colnorm if colnorm else s.init

    def step():
        if colnorm:  # the column-norm start, then the same iterations and packing
            s.init_colnorm()
            s.iterate(T)
            s.pack()
        else:
            s.solve(T)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: K whole steps back to back (one dq_solve each for
    # the absmax start)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(st)
    for _ in range(args.steps):
        step()
    e_end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / args.steps

    # breakdown, outside the timed region: the same work as separate calls
    # with events between them (the pass time for the roofline comes from
    # here)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        e = ev[k]
        e[0].record(st)
        init()
        e[1].record(st)
        s.iterate(T)
        e[2].record(st)
        s.pack()
        e[3].record(st)
    torch.cuda.synchronize()
    init_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    iter_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    pack_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    elems = M * N
    value = elems * T / (step_ms * 1e-3)
    pass_s = iter_ms * 1e-3 / T
    w_bytes = 2 if fmt_w_bf16(data) else 4
    a_bytes = 2 if fmt.a_fmt == dq.SCALE_FP16 else 1
    b_alg = alg_bytes_per_elem(w_bytes, a_bytes, fmt.group, M)
    achieved = b_alg * elems / pass_s / 1e9

    out = {
        "metric": "weight elements/s per BCD iteration",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32-requant/f64-sums",
        "data": "synthetic (seeded, numpy PCG64)",
        "config": {"workload": wl.name, "rows": M, "cols": N, "format": wl.fmt,
                   "group": fmt.group, "iters": T, "seed": wl.seeds[0], "init": args.init,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(wl.name),
                     "kernel": "bcd_pass_kernel", "alg_bytes_per_elem": b_alg,
                     "avg_launch_us": pass_s * 1e6},
        "valu": valu_entry(recorded_valu(wl.name), pass_s, elems),
        "breakdown_ms": {"init": init_ms, "iterate": iter_ms, "pack": pack_ms,
                         "wall_per_step": wall * 1e3 / args.steps},
        "iterate_elements_per_s_per_iter": elems / pass_s,
        "us_per_iter": iter_ms * 1e3 / T,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, data)
    print(json.dumps(out))


def act_bytes_per_elem(code_bits: int, a_bytes: int, G: int, tokens: int) -> float:
    """One read of X (bf16), the codes and the per-token block scales
    written, the column scales read (2 bytes, amortized over the tokens)."""
    return 2.0 + code_bits / 8.0 + a_bytes / G + 2.0 / tokens


def act_cpu_baseline(aw, X, bbits, budget_s: float = 10.0):
    """The float64 oracle on a prefix of the tokens, repeated for about
    budget_s seconds."""
    from calibration_free_bit_amd import synth
    from oracle import dualquant as D

    fmt = D.FORMATS[aw.fmt]
    b = bbits.view("float16").astype("float64")
    k = min(aw.tokens, 256)
    Xs = synth.bf16_to_f64(X[:k])
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while reps == 0 or dt < budget_s:
        D.rescale_quantize_act(Xs, b, fmt)
        reps += 1
        dt = time.perf_counter() - t0
    return {"value": Xs.size * reps / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 numpy oracle, the first {k} of {aw.tokens} tokens "
                      f"({k}x{aw.cols}), {reps} run(s) in {dt:.1f} s"}


def run_act(args):
    """Activation quantization with the column scales folded in
    (dq_rescale_quantize_act): one step quantizes the whole token batch."""
    import numpy as np
    import torch

    from calibration_free_bit_amd import dq, synth

    aw = synth.ACT_WORKLOADS[args.workload]
    fmt = dq.FORMATS[aw.fmt]
    X = synth.make_activations(aw.tokens, aw.cols, aw.seed)
    bbits = synth.make_col_scales(aw.cols, aw.seed + 1)
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
    bd = torch.from_numpy(bbits.view(np.int16)).to("cuda:0")
    xq = torch.empty((aw.tokens, aw.cols * fmt.code_bits // 8), dtype=torch.uint8, device="cuda:0")
    xs = torch.empty((aw.tokens, aw.cols // fmt.group), dtype=fmt.a_dtype, device="cuda:0")
    p = dq.problem(1, aw.cols, fmt, dq.W_BF16, aw.cols)
    st = torch.cuda.current_stream()

    def step():
        dq.rescale_quantize_act(p, Xd, aw.tokens, aw.cols, bd, xq, xs, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(st)
    for _ in range(args.steps):
        step()
    e_end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / args.steps
    elems = aw.tokens * aw.cols
    a_bytes = 2 if fmt.a_fmt == dq.SCALE_FP16 else 1
    b_alg = act_bytes_per_elem(fmt.code_bits, a_bytes, fmt.group, aw.tokens)
    # one kernel per step, launched back to back: the step time is the
    # launch time
    achieved = b_alg * elems / (step_ms * 1e-3) / 1e9
    out = {
        "metric": "activation elements/s",
        "value": elems / (step_ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32",
        "data": "synthetic (seeded, numpy PCG64)",
        "config": {"workload": aw.name, "tokens": aw.tokens, "cols": aw.cols, "format": aw.fmt,
                   "group": fmt.group, "seed": aw.seed, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(aw.name),
                     "kernel": "act_quant_kernel", "alg_bytes_per_elem": b_alg,
                     "avg_launch_us": step_ms * 1e3},
        "breakdown_ms": {"wall_per_step": wall * 1e3 / args.steps},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = act_cpu_baseline(aw, X, bbits)
    print(json.dumps(out))


def valu_entry(lane_ops, pass_s: float, elems: int):
    """The pass kernel against the VALU issue peak, the unit that binds it:
    recorded lane operations per launch over the launch time measured here."""
    if lane_ops is None:
        return None
    achieved = lane_ops / pass_s / 1e12
    return {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TOPS, "unit": "T lane-op/s",
            "frac": achieved / VALU_PEAK_TOPS, "lane_ops_per_elem": lane_ops / elems}


def fmt_w_bf16(data) -> bool:
    return data.dtype.name == "uint16"


if __name__ == "__main__":
    main()
