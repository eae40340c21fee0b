"""Build libfa.so in-tree with hipcc for gfx950.

Also builds libfa_serial.so, the race-check variant of the same sources
(``-DFA_SERIAL_PIPELINE``: every staged LDS copy completes, behind workgroup
barriers, before anything else runs).  Its outputs must equal libfa.so's bit
for bit; only the tests load it.

Usage: ``python -m exact_attention_103_amd.build`` (or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SERIAL_LIB = os.path.join(PKG, "libfa_serial.so")

SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_fp8_quant.hip", "fa_decode.hip", "fa_bwd.hip",
           "fa_noalloc.hip"]

# Packed fp32 VALU forms are switched off for the device code; hipcc's host
# pass warns that it does not know the feature, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-fno-honor-nans",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into libfa.so and libfa_serial.so (always
    recompiles both, in parallel)."""
    jobs = [(LIB, list(extra_flags)), (SERIAL_LIB, [*extra_flags, "-DFA_SERIAL_PIPELINE"])]
    procs = [_start(out, flags, verbose) for out, flags in jobs]
    for p in procs:
        _finish(*p, verbose)
    return LIB


def _start(out, extra_flags, verbose):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), \
        tmp, out


def _finish(proc, tmp, out, verbose):
    text, _ = proc.communicate()
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in text.splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(out)}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
