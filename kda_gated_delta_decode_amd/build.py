"""Build the KDA decode C-ABI library (libkda_decode.so) in-tree for gfx950.

    python -m kda_gated_delta_decode_amd.build [-v]

Compiles csrc/kda_decode.hip (decode kernels and launch entry points),
csrc/kda_prefill.hip (the chunked prefill), csrc/kda_probe.hip (bandwidth
probes) and csrc/kda_host.cpp (validation, addressing, sizing) with hipcc into
kda_gated_delta_decode_amd/libkda_decode.so.  Flags:
  --offload-arch=gfx950          MI355X only
  -ffp-contract=off              no implicit multiply-add fusion: every fused
                                 multiply-add in the kernels is an explicit
                                 fmaf, so fp32 and fp16 builds do identical
                                 arithmetic
  -target-feature -packed-fp32-ops   keep the compiler from forming packed
                                 fp32 instructions
  -amdgpu-kernarg-preload-count=14   preload the leading kernel arguments
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
LIB = os.path.join(PKG, "libkda_decode.so")
SOURCES = [os.path.join(CSRC, "kda_decode.hip"), os.path.join(CSRC, "kda_prefill.hip"),
           os.path.join(CSRC, "kda_probe.hip"), os.path.join(CSRC, "kda_host.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA decode library needs ROCm's hipcc")


def flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # kernels whose leading arguments are plain pointers and integers get
        # the first 14 argument dwords preloaded into scalar registers
        "-mllvm", "-amdgpu-kernarg-preload-count=14",
        # atomics stay as written: the optimizer's rewrite of a one-lane
        # atomic reads its result back at once, which would stall the
        # chained-row kernel's pair-counter increment (issued early, its
        # result used only at the end)
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-Wall",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that notice is expected and is filtered out of the log.
    noise = ("packed-fp32-ops' is not a recognized feature", "argument unused during compilation")
    log = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    return r.returncode, log


def build(verbose: bool = False) -> str:
    """Compile the library (always; a build check must compile).  Returns the
    path of the .so.  Each source compiles to its own object, in parallel
    (no device code crosses files), then one link; the output is written
    atomically."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    tmp = LIB + ".tmp%d" % os.getpid()
    compile_flags = [f for f in flags() if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="kda_build_") as work:
        objs = [os.path.join(work, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *compile_flags, "-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        logs = []
        for (rc, log), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (src, rc, log))
            logs.append(log)
        link = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, log = _run(link)
        if rc != 0:
            raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, log))
        logs.append(log)
    log = "\n".join(l for l in logs if l.strip())
    if verbose and log.strip():
        print(log)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
