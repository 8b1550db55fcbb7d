"""Host code under the address and undefined-behaviour sanitizers (no GPU).

* The host-only planning unit of the library (argument checks, launch table,
  automatic choice, split-K plan: csrc/host_plan.cpp) with the address
  replay of tests/host_replay.cpp, which runs the kernels' own constexpr
  index functions (csrc/addr_math.hpp) over every tile of the benchmark's
  workloads and an edge sweep and checks every load against its matrix's
  rows and columns, every store against C's M x N window and every direct
  load's 32-bit lane offset.  A planted mistake (edge tiles left overhanging
  C) must be reported.
* The C oracle (test infrastructure) through tests/oracle_sanitized.c, on
  buffers allocated to exactly the extent each leading dimension implies.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_fp32_gemm_03_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not available")
    return path


def _build(cmd, out):
    r = subprocess.run(cmd + ["-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def _run(exe, *args, env=None):
    e = dict(os.environ)
    e.update({"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
              "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    e.update(env or {})
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=e)


@pytest.fixture(scope="module")
def replay_exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("replay") / "host_replay")
    cmd = [_compiler("g++"), "-std=c++17", *SAN, "-Wall", "-Wextra", "-Werror", "-I", CSRC,
           os.path.join(ROOT, "tests", "host_replay.cpp"), os.path.join(CSRC, "host_plan.cpp")]
    return _build(cmd, out)


def test_replay_every_address_of_the_workloads(replay_exe):
    r = _run(replay_exe)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert ", 0 failures" in r.stdout, r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]


def test_replay_reports_a_planted_mistake(replay_exe):
    r = _run(replay_exe, "--quick", "--plant-unclamped")
    assert r.returncode == 1, r.stdout[-2000:] + r.stderr[-2000:]
    assert "FAIL" in r.stdout and "direct load" in r.stdout, r.stdout[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    out = str(tmp_path / "oracle_san")
    cmd = [_compiler("gcc"), "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "gemm_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitized.c"), "-lm"]
    exe = _build(cmd, out)
    r = _run(exe, env={"OMP_NUM_THREADS": "4"})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert ": 0 failures" in r.stdout, r.stdout
