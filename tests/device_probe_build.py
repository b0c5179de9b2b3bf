"""Builds tests/_build/libss_device_probe.so from tests/device_probe.hip with
the library's own compiler flags (gfx950). Called by __graft_entry__.build()."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))
SRC = os.path.join(HERE, "device_probe.hip")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libss_device_probe.so")


def build(verbose=False):
    from speculative_decoding_verification_pipeline_amd import build as lib_build
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [lib_build.hipcc(), *lib_build.CFLAGS, "-shared", "-x", "hip", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=OUT_DIR)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
