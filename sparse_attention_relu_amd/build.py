"""Build libsparse_mla.so (release) and libsparse_mla_debug.so (SA_DEBUG:
device-side precondition checks) for gfx950 with hipcc (no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_mla.so")
DEBUG_LIB = os.path.join(HERE, "libsparse_mla_debug.so")
SOURCES = ["abi.hip", "indexer.hip", "topk.hip", "mla.hip", "cache.hip", "share.hip", "qproj.hip", "quant.hip", "debug.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=fast", "-munsafe-fp-atomics",
    # packed fp32 instructions stay off: ordinary fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # MFMA results in ordinary VGPRs: keeps the attention loop from shuttling
    # values through AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def _command(out: str, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc, *FLAGS, *extra, "-o", out, *srcs]


def build(verbose: bool = False, extra=()) -> str:
    """Compile both libraries (in parallel) and move them into place."""
    jobs = [(LIB, list(extra)), (DEBUG_LIB, ["-DSA_DEBUG", *extra])]
    procs = []
    for lib, ex in jobs:
        cmd = _command(lib + ".tmp", ex)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for lib, p in procs:
        text, _ = p.communicate()
        out = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(f"{os.path.basename(lib)}: hipcc failed ({p.returncode}):\n{out}")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("\n".join(failed))
    for lib, _ in procs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
