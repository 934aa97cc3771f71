"""Build libkvq.so (the HIP kernels for gfx950 plus the host C ABI) in-tree with hipcc.

Flags that fix the numerics of the encoders: correctly rounded fp32 division and square
root, no flush of subnormals, and no FMA contraction in the encode translation unit.
Packed fp32 instructions are disabled for all device code.
"""
import os
import subprocess
import sys
import time

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

# longest first: the prefill kernels, then the fast decode kernel (one object per key format
# id 1..24, each against every value format), then the rest
UNITS = [("kvq_prefill.hip", [])]
UNITS += [("kvq_decode_ws_key.hip", ["-DKVQ_WS_FK=%d" % f], "kvq_decode_ws_key_f%d" % f) for f in range(1, 25)]
UNITS += [
    ("kvq_host.cpp", ["-ffp-contract=off"]),
    ("kvq_append.hip", ["-ffp-contract=off"]),
    ("kvq_decode.hip", []),
    ("kvq_decode_ws.hip", []),
    ("kvq_merge.hip", []),
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
    """Compile every translation unit and link libkvq.so; returns its path.  Each compiler's
    output goes to a log file next to its object (the kernel headers' inline-asm clobber
    warnings run to hundreds of KB per unit, more than a pipe holds)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    running = []                                  # (cmd, process, log file)

    def reap(block):
        while running:
            done = [r for r in running if r[1].poll() is not None]
            for cmd, p, log in done:
                running.remove((cmd, p, log))
                log.close()
                if p.returncode != 0:
                    with open(log.name) as f:
                        sys.stderr.write(f.read()[-20000:])
                    raise RuntimeError("compile failed: " + cmd[-3])
            if done or not block:
                return
            time.sleep(0.2)

    for unit in UNITS:
        src, extra = unit[0], unit[1]
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, (unit[2] if len(unit) > 2 else src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc"] + COMMON + extra + lang + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        while len(running) >= jobs:
            reap(True)
        log = open(obj + ".log", "w")
        running.append((cmd, subprocess.Popen(cmd, stdout=log, stderr=subprocess.STDOUT), log))
        objs.append(obj)
    while running:
        reap(True)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
