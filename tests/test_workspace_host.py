"""The per-stream workspace bookkeeping (csrc/workspace.h), on the host.

tests/workspace_sim.cpp instantiates the library's cache with a simulated
stream backend, runs concurrent callers through it and replays every stream's
queued operations: no call may use a freed or too-small buffer, no buffer may
be freed under an open call, and the calls on one stream must not interleave.
A caller that drops the lock between acquire and release (the bookkeeping that
had the race) is run too, and must be caught.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("ws") / "workspace_sim")
    r = subprocess.run([cxx, "-std=c++17", "-O1", "-pthread", "-Wall",
                        os.path.join(HERE, "workspace_sim.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, mode):
    return subprocess.run([exe, mode], capture_output=True, text=True, timeout=120)


def test_concurrent_callers_on_shared_streams(sim):
    r = run(sim, "ok")
    assert r.returncode == 0, r.stdout


def test_failed_allocation_holds_nothing(sim):
    r = run(sim, "fail")
    assert r.returncode == 0, r.stdout


def test_dropping_the_lock_early_is_caught(sim):
    r = run(sim, "early")
    assert r.returncode == 3, (r.returncode, r.stdout)
    assert "dead" in r.stdout or "free while" in r.stdout
