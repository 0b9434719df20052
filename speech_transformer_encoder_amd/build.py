"""Compile the gfx950 HIP sources in ``csrc/`` into ``libwhisper_enc.so`` next to this file, and
the measurement probe in ``csrc/probe/`` into ``libwenc_probe.so`` (used by the benchmark only).

``python -m speech_transformer_encoder_amd.build`` (or ``__graft_entry__.build()``) runs hipcc
once over every ``.hip`` source.  hipcc cross-compiles for gfx950 without a GPU present.
"""

import glob
import os
import subprocess
import sys

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
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    # Packed fp32 VALU forms stay off: the kernels use plain fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wl,--no-undefined",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(srcs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB, verbose)
    return _hipcc(sources(), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
