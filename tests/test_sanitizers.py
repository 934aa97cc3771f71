"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code (CPU only):

* the C-ABI library's host code (kvq_host.cpp: configuration checks, the precision-tail
  state machine, the decode split planner, every entry point's argument checks) linked
  with host stand-ins for the device layer (tests/sanitize/host_stubs.cpp, which also check
  each decode plan: every unit covered once, workgroups onto partial slots one to one),
  driven by tests/sanitize/host_driver.cpp;
* the oracle (oracle/kvq_oracle.c) driven by tests/sanitize/oracle_driver.c on exact-size
  heap buffers.

Each program prints "ok" and exits 0; any sanitizer report aborts it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _have(cc):
    return shutil.which(cc) is not None


def _build_run(tmp_path, cc, std, srcs, incs, extra=()):
    exe = str(tmp_path / "prog")
    cmd = [cc, std] + SAN + list(extra) + ["-I" + i for i in incs] + srcs + ["-o", exe]
    if cc == "gcc":
        cmd.append("-lm")
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.skipif(not _have("g++"), reason="no g++")
def test_host_library_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "mixed_precision_quantized_amd", "csrc")
    srcs = [os.path.join(csrc, "kvq_host.cpp"), os.path.join(HERE, "sanitize", "host_stubs.cpp"),
            os.path.join(HERE, "sanitize", "host_driver.cpp")]
    _build_run(tmp_path, "g++", "-std=c++17", srcs, [os.path.join(ROOT, "include"), csrc])


@pytest.mark.skipif(not _have("gcc"), reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    srcs = [os.path.join(ROOT, "oracle", "kvq_oracle.c"), os.path.join(HERE, "sanitize", "oracle_driver.c")]
    _build_run(tmp_path, "gcc", "-std=c11", srcs, [os.path.join(ROOT, "oracle")], ["-ffp-contract=off"])
