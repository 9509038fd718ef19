"""Compile the HIP sources of the library into one shared object for gfx950.

Run as ``python -m mla_paged_latent_amd.build``; writes
``mla_paged_latent_amd/libmla_paged_latent.so`` next to this file, and the
measurement probes bench.py uses (achievable HBM read and MFMA rates) as
``libmla_probe.so`` beside it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_paged_latent.so")
SOURCES = ["cache_write.hip", "absorb_upv.hip", "decode.hip", "context.hip", "prefill.hip"]
PROBE_LIB = os.path.join(HERE, "libmla_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def flags(extra: list[str] | None = None) -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # keep packed-fp32 instructions out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"] + (extra or [])


def _link(sources: list[str], lib: str, verbose: bool) -> str:
    cc = hipcc()
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in sources:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, *flags(), "-shared", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source, link ``libmla_paged_latent.so`` and the probe library;
    returns the main library's path."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
