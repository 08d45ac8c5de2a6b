"""The host worker pool of the slot-mode layer's CPU half, on the CPU only.

tests/host_pool_stress.cpp drives csrc/host_pool.hpp with jobs that
alternate between a few items and many; every item must run exactly once
with its own job's function.  Built twice with g++: optimised, and with the
thread sanitizer (a smaller run), which reports any data race between a job's
publication and a late worker of the previous job.
"""
import os
import subprocess

import pytest

from helpers import ROOT

SRC = os.path.join(ROOT, "tests", "host_pool_stress.cpp")
INC = os.path.join(ROOT, "bit_expert_ffn_router_amd", "csrc")


def _build(tmp_path, name, extra):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-pthread", "-I", INC, SRC, "-o", exe] + extra,
                   check=True)
    return exe


def test_pool_every_item_once(tmp_path):
    exe = _build(tmp_path, "stress", [])
    r = subprocess.run([exe, "8", "200000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_pool_under_thread_sanitizer(tmp_path):
    try:
        exe = _build(tmp_path, "stress_tsan", ["-fsanitize=thread"])
    except subprocess.CalledProcessError:
        pytest.skip("g++ cannot build with the thread sanitizer here")
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([exe, "6", "1500"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
