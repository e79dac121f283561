"""bench.py's command line: the checks that run before any device work.

No GPU is needed: each case exits on the host with status 2 and a message
before torch touches a device.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = _run("--gpus", gpus, "--no-cpu-baseline")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("args", [("--steps", "0"), ("--warmup", "-1"),
                                  ("--workload", "llama31_8b_int4_g64_bf16", "--steps", "0")])
def test_bad_step_counts_are_refused(args):
    r = _run(*args, "--no-cpu-baseline")
    assert r.returncode == 2
    assert "--steps" in r.stderr
    assert r.stdout == ""


def test_default_step_counts():
    sys.path.insert(0, ROOT)
    import argparse

    import bench

    for steps, warmup, want in [(None, None, (100, 200)), (7, None, (7, 200)), (None, 0, (100, 0))]:
        ns = argparse.Namespace(steps=steps, warmup=warmup)
        bench._step_counts(ns, steps=100, warmup=200)
        assert (ns.steps, ns.warmup) == want


def test_profile_stems_name_kernel_and_workload():
    sys.path.insert(0, ROOT)
    import bench
    from calibration_free_bit_amd import synth

    stems = {}
    for name in list(synth.WORKLOADS) + list(synth.ACT_WORKLOADS):
        stem = bench.profile_stem(name)
        kernel = "act_quant_" if name in synth.ACT_WORKLOADS else "bcd_pass_"
        assert stem.startswith(kernel)
        assert stem.endswith(name.split("_", 1)[1] if name.startswith("act_") else name)
        stems[stem] = name
    assert len(stems) == len(synth.WORKLOADS) + len(synth.ACT_WORKLOADS)


@pytest.mark.parametrize("name", ["act_no_such_workload", "int4_g64_1x1_bf16"])
def test_unknown_workload_is_refused(name):
    r = _run("--workload", name, "--no-cpu-baseline")
    assert r.returncode == 2
    assert "unknown workload" in r.stderr
    assert r.stdout == ""
