"""Collect the rocprofv3 evidence behind bench.py's roofline entry.

Runs, each in its own rocprofv3 process:
  1. --kernel-trace --stats of ``bench.py`` (per-kernel average durations);
  2. --pmc FETCH_SIZE, then --pmc WRITE_SIZE of ``bench.py`` (HBM bytes per
     dispatch, in KiB), then --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_WAVES
     (instructions issued by the profiled kernel: the BCD pass for a weight
     workload, the activation quantizer for an ``act_`` workload);
  3. the same two counters for ``bench.py --copy-calibration``, a plain
     device copy of 256 MiB, whose known bytes give the scale factors of
     the two counters.
and writes to OUT_DIR (STEM: bcd_pass_<workload>, or act_quant_<...> for
an activation workload act_<...>):
  STEM_kernel_trace.md   kernel-trace summary
  STEM_counters.json     traffic per launch + factors
  STEM_counters.md       the same, readable

Usage (on a machine with the GPU; rocprofv3 on PATH):
  python -m calibration_free_bit_amd.profile_counters OUT_DIR [--workload W]
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

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
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
    out = os.path.join(work, tag)
    cmd = ["rocprofv3", *args, "-d", out, "-o", "run", "--output-format", "csv", "--",
           sys.executable, *prog]
    env = dict(os.environ, TMPDIR="/tmp")
    print("[profile]", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=timeout)
    if r.returncode not in (0,):
        print(r.stdout[-2000:], r.stderr[-4000:], flush=True)
        raise RuntimeError(f"rocprofv3 failed ({r.returncode}) for {tag}")
    return out, _shown(cmd)


def _find(root, suffix):
    for d, _, files in os.walk(root):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(d, f)
    raise FileNotFoundError(f"{suffix} under {root}")


def _matches(kernel_name: str, name_has: str) -> bool:
    """name_has in the kernel's name; for the pass kernel only its plain
    instantiation (last template argument 0), not the first pass of a
    whole solve or the statistics variant."""
    if name_has not in kernel_name:
        return False
    if name_has == "bcd_pass_kernel":
        return kernel_name.split(">(")[0].endswith(", 0")
    return True


def _counters(root, counter, name_has):
    """Per-dispatch values of one counter, for kernels whose name contains
    name_has (summed over the counter's dimensions)."""
    per = defaultdict(float)
    for r in csv.DictReader(open(_find(root, "counter_collection.csv"))):
        if r["Counter_Name"] == counter and _matches(r["Kernel_Name"], name_has):
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out_dir")
    ap.add_argument("--workload", default="int4_g64_4096x4096_bf16")
    args = ap.parse_args()
    os.makedirs(args.out_dir, exist_ok=True)
    sys.path.insert(0, ROOT)
    import bench  # for the source hash and the workload definition
    from calibration_free_bit_amd import synth

    from calibration_free_bit_amd import dq
    if args.workload in synth.ACT_WORKLOADS:
        aw = synth.ACT_WORKLOADS[args.workload]
        kernel, what = "act_quant_kernel", "activation quantization"
        launch, unit = "launch", "activation element"
        M, N = aw.tokens, aw.cols
        fmt = dq.FORMATS[aw.fmt]
        b_alg = bench.act_bytes_per_elem(fmt.code_bits, 2 if fmt.a_fmt == dq.SCALE_FP16 else 1,
                                         fmt.group, M)
    else:
        wl = synth.WORKLOADS[args.workload]
        kernel, what = "bcd_pass_kernel", "BCD solver"
        launch, unit = "pass launch", "weight element"
        M, N = wl.spec.rows, wl.spec.cols
        fmt = dq.FORMATS[wl.fmt]
        b_alg = bench.alg_bytes_per_elem(2 if wl.spec.dtype == "bf16" else 4,
                                         2 if fmt.a_fmt == dq.SCALE_FP16 else 1, fmt.group, M)
    name = args.workload
    stem = bench.profile_stem(name)
    bench_args = [BENCH, "--workload", name, "--no-cpu-baseline"]
    work = tempfile.mkdtemp(prefix="dqprof_", dir="/tmp")

    # 1. kernel trace
    tr, tr_cmd = _rocprof(["--kernel-trace", "--stats"], bench_args,
                          "trace", work)
    stats = list(csv.DictReader(open(_find(tr, "kernel_stats.csv"))))
    lines = [f"# Kernel trace: {what}, workload {name}", "",
             "Command:", "", f"    {tr_cmd}", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} % |")
    open(os.path.join(args.out_dir, f"{stem}_kernel_trace.md"), "w").write(
        "\n".join(lines) + "\n")

    # 2./3. byte counters, each counter in its own run
    res = {}
    cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d, c = _rocprof(["--pmc", counter], bench_args + ["--steps", "2", "--warmup", "1"],
                        f"pass_{counter}", work, timeout=180)
        res[("pass", counter)] = _counters(d, counter, kernel)
        cmds[("pass", counter)] = c
        d, c = _rocprof(["--pmc", counter], [BENCH, "--copy-calibration"], f"copy_{counter}", work,
                        timeout=180)
        vals = _counters(d, counter, "")
        res[("copy", counter)] = vals
        cmds[("copy", counter)] = c

    # 4. VALU instruction count of the kernel (wave-level instructions;
    #    x64 lanes = lane operations), for its VALU roofline
    d, c = _rocprof(["--pmc", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_WAVES"],
                    bench_args + ["--steps", "2", "--warmup", "1"], "pass_valu", work, timeout=180)
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
        "valu_insts_per_launch": sum(valu) / len(valu),
        "salu_insts_per_launch": sum(salu) / len(salu),
        "waves_per_launch": sum(waves) / len(waves),
        "valu_lane_ops_per_element": 64.0 * sum(valu) / len(valu) / (M * N),
        "commands": {f"{k[0]}_{k[1]}": v for k, v in cmds.items()},
    }
    json.dump(rec, open(os.path.join(args.out_dir, f"{stem}_counters.json"), "w"), indent=2)
    md = [f"# HBM byte counters: {kernel}, workload {name}", "",
          f"Per {launch} (average of {len(pf)} dispatches): FETCH_SIZE {fetch_kib:.0f} KiB, "
          f"WRITE_SIZE {write_kib:.0f} KiB.", "",
          f"Calibration: a plain 256 MiB device copy reads FETCH_SIZE {f_copy / 1024:.0f} KiB and "
          f"WRITE_SIZE {w_copy / 1024:.0f} KiB, so the factors are {fetch_factor:.4f} (fetch) and "
          f"{write_factor:.4f} (write).", "",
          f"Traffic per launch: {traffic / 1e6:.2f} MB = {traffic / (M * N):.3f} bytes per {unit} "
          f"(algorithmic: {b_alg:.4f}).", "",
          f"VALU: {rec['valu_insts_per_launch']:.4g} wave instructions per launch "
          f"({rec['valu_lane_ops_per_element']:.2f} lane operations per {unit}), "
          f"SALU {rec['salu_insts_per_launch']:.4g}, waves {rec['waves_per_launch']:.0f}.", "",
          "Commands:", ""]
    md += [f"    {v}" for v in cmds.values()]
    open(os.path.join(args.out_dir, f"{stem}_counters.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
