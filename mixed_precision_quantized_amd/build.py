"""Build libkvq.so (the HIP kernels for gfx950 plus the host C ABI) in-tree with hipcc.

Flags that fix the numerics of the encoders: correctly rounded fp32 division and square
root, no flush of subnormals, and no FMA contraction in the encode translation unit.
Packed fp32 instructions are disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
          "-Wno-unused-command-line-argument", "-I" + INCLUDE]

UNITS = [
    ("kvq_host.cpp", ["-ffp-contract=off"]),
    ("kvq_append.hip", ["-ffp-contract=off"]),
    ("kvq_decode.hip", []),
    ("kvq_decode_ws.hip", []),
    ("kvq_decode_ws_k2.hip", []),
    ("kvq_decode_ws_k3.hip", []),
    ("kvq_decode_ws_k4.hip", []),
    ("kvq_decode_ws_k5.hip", []),
    ("kvq_decode_ws_k6.hip", []),
    ("kvq_decode_ws_k8.hip", []),
    ("kvq_merge.hip", []),
    ("kvq_prefill.hip", []),
    ("kvq_debug.hip", ["-ffp-contract=off"]),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd[:3]) + " ...")
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every translation unit and link libkvq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    procs = []
    for src, extra in UNITS:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc"] + COMMON + extra + lang + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for cmd, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            raise RuntimeError("compile failed: " + cmd[-3])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
