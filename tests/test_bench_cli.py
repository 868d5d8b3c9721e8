"""The benchmark's command line, on the CPU (no GPU run): the one-GPU contract
and the byte accounting the JSON line is built from."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_names_every_workload_option():
    r = run_bench("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--steps", "--warmup", "--splits", "--layout", "--no-whole-pair", "--no-mix"):
        assert opt in r.stdout


def test_decode_kernel_label_follows_the_partition():
    whole = "one workgroup per (sequence, KV head) pair"
    assert whole in bench.decode_kernel_label(-1, 32, 2048)
    assert whole in bench.decode_kernel_label(0, 32, 512)          # short contexts: whole pairs
    assert "merge" in bench.decode_kernel_label(0, 32, 2048)       # the mha default: split + merge
    assert "merge" in bench.decode_kernel_label(0, 65, 100)        # more than 64 sequences
    assert "merge" in bench.decode_kernel_label(512, 32, 100)      # an explicit split count


def test_unknown_workload_is_refused():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode != 0
