"""Compile the HIP library libpn.so for gfx950 with hipcc (in-tree).

Packed fp32 VALU instructions are switched off for every HIP source
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpn.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("pn_kernels.hip", "pn_gemv_rows.hip", "pn_smallm.hip", "pn_probe.hip",
                                                               "pn_rotate.hip", "pn_prefill.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=None) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra or []) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
