"""Collect the rocprofv3 evidence behind bench.py's roofline entry.

For a single-matrix or activation workload W (stem bcd_pass_W, or
act_quant_<...> for an activation workload act_<...>), each in its own
rocprofv3 process:
  1. --kernel-trace --stats of ``bench.py --workload W`` (per-kernel
     average durations);
  2. --pmc FETCH_SIZE, then --pmc WRITE_SIZE of the same command with 2
     timed steps (HBM bytes per dispatch, in KiB), then --pmc SQ_INSTS_VALU
     SQ_INSTS_SALU SQ_WAVES (instructions of the profiled kernel: the plain
     BCD pass, or the activation quantizer);
  3. the same two byte counters for ``bench.py --copy-calibration``, a plain
     device copy of 256 MiB, whose known bytes give the counters' scale
     factors;
and writes to OUT_DIR:
  STEM_kernel_trace.md   kernel-trace summary
  STEM_counters.json     traffic and instructions per launch + factors
  STEM_counters.md       the same, readable

For the Llama-3.1-8B set (the default workload) it writes the kernel trace
of the default bench command (``bench.py`` with 2 timed steps), with the
average of the pass launches bench.py times for its roofline entry (the
last ones of the run: T passes at a time on the gate matrix), and collects
1.-3. for the single-matrix workload of that shape,
int4_g64_14336x4096_bf16 (the same matrix recipe; layer 0's gate seed).

Usage (on a machine with the GPU; rocprofv3 on PATH):
  python profile_counters.py OUT_DIR [--workload W]
"""

from __future__ import annotations

import argparse
import csv
import json
import os
import subprocess
import sys
import tempfile
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
BENCH = os.path.join(ROOT, "bench.py")


def _shown(cmd):
    """The command as a reader reruns it: the repository as /root/repo, the
    interpreter as python3, the output folder as OUT."""
    txt = []
    for c in cmd:
        if c == sys.executable:
            c = "python3"
        elif c.startswith(ROOT):
            c = "/root/repo" + c[len(ROOT):]
        elif c.startswith("/tmp/dqprof_"):
            c = "OUT/" + os.path.basename(c)
        txt.append(c)
    return "cd /tmp && export TMPDIR=/tmp && " + " ".join(txt)


def _rocprof(args, prog, tag, work, timeout=300):
    """Run prog under rocprofv3; returns (output dir, shown command, stdout)."""
    out = os.path.join(work, tag)
    cmd = ["rocprofv3", *args, "-d", out, "-o", "run", "--output-format", "csv", "--",
           sys.executable, *prog]
    env = dict(os.environ, TMPDIR="/tmp")
    print("[profile]", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=timeout)
    if r.returncode not in (0,):
        print(r.stdout[-2000:], r.stderr[-4000:], flush=True)
        raise RuntimeError(f"rocprofv3 failed ({r.returncode}) for {tag}")
    print(f"[profile] {tag} done", flush=True)
    return out, _shown(cmd), r.stdout


def _find(root, suffix):
    for d, _, files in os.walk(root):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(d, f)
    raise FileNotFoundError(f"{suffix} under {root}")


def _matches(kernel_name: str, name_has: str) -> bool:
    """name_has in the kernel's name; for the pass kernel only its plain
    instantiation (fifth template argument, the pass mode, 0), not the first
    pass of a whole solve or the statistics variant."""
    if name_has not in kernel_name:
        return False
    if name_has == "bcd_pass_kernel":
        args = kernel_name.split("<", 1)[1].split(">(")[0].split(",")
        return args[4].strip() == "0"
    return True


def _counters(root, counter, name_has):
    """Per-dispatch values of one counter, for kernels whose name contains
    name_has (summed over the counter's dimensions)."""
    per = defaultdict(float)
    for r in csv.DictReader(open(_find(root, "counter_collection.csv"))):
        if r["Counter_Name"] == counter and _matches(r["Kernel_Name"], name_has):
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def _json_line(stdout: str):
    for line in reversed(stdout.splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    raise RuntimeError("bench.py printed no JSON line")


def _trace_table(tr, title, cmd):
    stats = list(csv.DictReader(open(_find(tr, "kernel_stats.csv"))))
    lines = [f"# Kernel trace: {title}", "", "Command:", "", f"    {cmd}", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} % |")
    return lines


def _dispatches(tr, name_has):
    """(start, end) in ns of every dispatch of the kernel, in dispatch order."""
    rows = []
    for r in csv.DictReader(open(_find(tr, "kernel_trace.csv"))):
        if _matches(r["Kernel_Name"], name_has):
            rows.append((int(r["Dispatch_Id"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    return [(a, b) for _, a, b in rows]


def profile_workload(name, out_dir, work):
    """Kernel trace and counters of a single-matrix or activation workload."""
    import bench  # for the source hash and the workload definitions
    from calibration_free_bit_amd import dq, synth
    if name in synth.ACT_WORKLOADS:
        aw = synth.ACT_WORKLOADS[name]
        kernel, what = "act_quant_kernel", "activation quantization"
        launch, unit = "launch", "activation element"
        M, N = aw.tokens, aw.cols
        fmt = dq.FORMATS[aw.fmt]
        b_alg = bench.act_bytes_per_elem(fmt.code_bits, 2 if fmt.a_fmt == dq.SCALE_FP16 else 1,
                                         fmt.group, M)
    else:
        wl = synth.WORKLOADS[name]
        kernel, what = "bcd_pass_kernel", "BCD solver"
        launch, unit = "pass launch", "weight element"
        M, N = wl.spec.rows, wl.spec.cols
        fmt = dq.FORMATS[wl.fmt]
        b_alg = bench.alg_bytes_per_elem(2 if wl.spec.dtype == "bf16" else 4,
                                         2 if fmt.a_fmt == dq.SCALE_FP16 else 1, fmt.group, M)
    stem = bench.profile_stem(name)
    bench_args = [BENCH, "--workload", name, "--no-cpu-baseline"]

    # 1. kernel trace
    tr, tr_cmd, _ = _rocprof(["--kernel-trace", "--stats"], bench_args, f"{stem}_trace", work)
    lines = _trace_table(tr, f"{what}, workload {name}", tr_cmd)
    open(os.path.join(out_dir, f"{stem}_kernel_trace.md"), "w").write("\n".join(lines) + "\n")

    # 2./3. byte counters, each counter in its own run
    res = {}
    cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d, c, _ = _rocprof(["--pmc", counter], bench_args + ["--steps", "2", "--warmup", "1"],
                           f"{stem}_{counter}", work, timeout=180)
        res[("pass", counter)] = _counters(d, counter, kernel)
        cmds[("pass", counter)] = c
        d, c, _ = _rocprof(["--pmc", counter], [BENCH, "--copy-calibration"], f"copy_{counter}", work,
                           timeout=180)
        res[("copy", counter)] = _counters(d, counter, "")
        cmds[("copy", counter)] = c

    # 4. VALU instruction count of the kernel (wave-level instructions;
    #    x64 lanes = lane operations), for its VALU roofline
    d, c, _ = _rocprof(["--pmc", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_WAVES"],
                       bench_args + ["--steps", "2", "--warmup", "1"], f"{stem}_valu", work, timeout=180)
    valu = _counters(d, "SQ_INSTS_VALU", kernel)
    salu = _counters(d, "SQ_INSTS_SALU", kernel)
    waves = _counters(d, "SQ_WAVES", kernel)
    cmds[("pass", "VALU")] = c

    copy_bytes = 256 << 20
    # the copy kernel is the largest dispatch of the calibration run
    f_copy = max(res[("copy", "FETCH_SIZE")]) * 1024.0
    w_copy = max(res[("copy", "WRITE_SIZE")]) * 1024.0
    fetch_factor = copy_bytes / f_copy
    write_factor = copy_bytes / w_copy
    pf = res[("pass", "FETCH_SIZE")]
    pw = res[("pass", "WRITE_SIZE")]
    fetch_kib = sum(pf) / len(pf)
    write_kib = sum(pw) / len(pw)
    traffic = fetch_kib * 1024.0 * fetch_factor + write_kib * 1024.0 * write_factor
    rec = {
        "workload": name,
        "source_hash": bench.kernel_source_hash(),
        "kernel": kernel,
        "dispatches": len(pf),
        "fetch_kib_per_launch": fetch_kib,
        "write_kib_per_launch": write_kib,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": f_copy / 1024.0,
        "copy_write_kib": w_copy / 1024.0,
        "fetch_factor": fetch_factor,
        "write_factor": write_factor,
        "traffic_bytes_per_launch": traffic,
        "traffic_bytes_per_element": traffic / (M * N),
        "alg_bytes_per_element": b_alg,
        "valu_insts_per_launch": sum(valu) / len(valu),
        "salu_insts_per_launch": sum(salu) / len(salu),
        "waves_per_launch": sum(waves) / len(waves),
        "valu_lane_ops_per_element": 64.0 * sum(valu) / len(valu) / (M * N),
        "commands": {f"{k[0]}_{k[1]}": v for k, v in cmds.items()},
    }
    json.dump(rec, open(os.path.join(out_dir, f"{stem}_counters.json"), "w"), indent=2)
    md = [f"# HBM byte counters: {kernel}, workload {name}", "",
          f"Per {launch} (average of {len(pf)} dispatches): FETCH_SIZE {fetch_kib:.0f} KiB, "
          f"WRITE_SIZE {write_kib:.0f} KiB.", "",
          f"Calibration: a plain 256 MiB device copy reads FETCH_SIZE {f_copy / 1024:.0f} KiB and "
          f"WRITE_SIZE {w_copy / 1024:.0f} KiB, so the factors are {fetch_factor:.4f} (fetch) and "
          f"{write_factor:.4f} (write).", "",
          f"Traffic per launch: {traffic / 1e6:.2f} MB = {traffic / (M * N):.3f} bytes per {unit} "
          f"(algorithmic: {b_alg:.4f}, ratio {traffic / (M * N) / b_alg:.3f}).", "",
          f"VALU: {rec['valu_insts_per_launch']:.4g} wave instructions per launch "
          f"({rec['valu_lane_ops_per_element']:.2f} lane operations per {unit}), "
          f"SALU {rec['salu_insts_per_launch']:.4g}, waves {rec['waves_per_launch']:.0f}.", "",
          "Commands:", ""]
    md += [f"    {v}" for v in cmds.values()]
    open(os.path.join(out_dir, f"{stem}_counters.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1), flush=True)


def profile_set(out_dir, work):
    """Kernel trace of the default bench command (the Llama-3.1-8B set),
    with the average of the pass launches its roofline entry times."""
    import bench
    stem = bench.profile_stem(bench.SET_WORKLOAD)
    tr, tr_cmd, stdout = _rocprof(["--kernel-trace", "--stats"],
                                  [BENCH, "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                                  f"{stem}_trace", work, timeout=600)
    res = _json_line(stdout)
    n = res["roofline"]["launches"]
    d = _dispatches(tr, "bcd_pass_kernel")[-n:]
    avg_us = sum(b - a for a, b in d) / len(d) / 1e3
    lines = _trace_table(tr, f"BCD solver, the Llama-3.1-8B set ({bench.SET_WORKLOAD})", tr_cmd)
    lines += ["", f"Roofline launches (the last {n} plain pass launches of the run: the T passes "
                  f"of solves of layer 0's gate matrix, 14336x4096, alone on one stream): average "
                  f"{avg_us:.2f} us in this trace; bench.py measured {res['roofline']['avg_launch_us']:.2f} us "
                  f"with events in the same run (its average includes one final column update per "
                  f"T passes).", "",
              f"Whole step: {res['ms_per_step']:.2f} ms, {res['value'] / 1e12:.3f} T elements/s per "
              f"iteration (under the profiler)."]
    open(os.path.join(out_dir, f"{stem}_kernel_trace.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[-3:]), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out_dir")
    ap.add_argument("--workload", default=None, help="default: the Llama-3.1-8B set")
    args = ap.parse_args()
    os.makedirs(args.out_dir, exist_ok=True)
    sys.path.insert(0, ROOT)
    import bench
    work = tempfile.mkdtemp(prefix="dqprof_", dir="/tmp")
    if args.workload in (None, bench.SET_WORKLOAD):
        profile_set(args.out_dir, work)
        profile_workload("int4_g64_14336x4096_bf16", args.out_dir, work)
    else:
        profile_workload(args.workload, args.out_dir, work)


if __name__ == "__main__":
    main()
