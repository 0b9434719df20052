"""Compile the gfx950 HIP sources in ``csrc/`` into ``libwhisper_enc.so`` next to this file, and
the measurement probe in ``csrc/probe/`` into ``libwenc_probe.so`` (used by the benchmark only).

``python -m speech_transformer_encoder_amd.build`` (or ``__graft_entry__.build()``) compiles every
``.hip`` source to an object with hipcc, in parallel, and links the objects into the shared
library.  hipcc cross-compiles for gfx950 without a GPU present.
"""

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwhisper_enc.so")
PROBE_LIB = os.path.join(HERE, "libwenc_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    # Packed fp32 VALU forms stay off: the kernels use plain fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _hipcc(srcs, lib, verbose):
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="wenc_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = [ex.submit(_run, [HIPCC, *FLAGS, *inc, "-c", s, "-o", o], verbose)
                    for s, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        tmp = lib + ".tmp"
        _run([HIPCC, *LINK_FLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB, verbose)
    return _hipcc(sources(), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
