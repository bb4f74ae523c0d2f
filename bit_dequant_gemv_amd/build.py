"""Build libqmoe.so (and the synthetic-input generator library) for gfx950.

Every HIP translation unit is compiled with hipcc for --offload-arch=gfx950 and
linked into a shared library next to its sources.  Packed-FP32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed: {' '.join(cmd)}")
    # hipcc's host pass does not know the packed-fp32 feature flag; drop that noise
    noise = [l for l in (r.stdout + r.stderr).splitlines()
             if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if verbose and noise:
        print("\n".join(noise))


def _library(srcs, out, extra, verbose, jobs, build_subdir="_build"):
    build_dir = os.path.join(os.path.dirname(out), build_subdir)
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in srcs:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *COMMON, *extra, *lang, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build_qmoe(verbose=False, jobs=None):
    csrc = os.path.join(HERE, "csrc")
    srcs = [os.path.join(csrc, f) for f in ("api.cpp", "kernels.hip", "ffn.hip", "layer.hip", "batched.hip",
                                            "gdn.hip", "attn.hip", "noalloc.hip", "stream.hip", "offload.cpp")]
    return _library(srcs, os.path.join(HERE, "libqmoe.so"),
                    ["-I", os.path.join(ROOT, "include"), "-I", csrc], verbose,
                    jobs or min(8, os.cpu_count() or 4))


def build_probe(verbose=False, jobs=None):
    """libqmoe_probe.so: the same sources with QMOE_PHASE_PROBE defined, so the fused
    layer records per-workgroup phase timestamps (bench.py --phase-probe reads them).
    Not part of the product build."""
    csrc = os.path.join(HERE, "csrc")
    srcs = [os.path.join(csrc, f) for f in ("api.cpp", "kernels.hip", "ffn.hip", "layer.hip", "batched.hip",
                                            "gdn.hip", "attn.hip", "noalloc.hip", "stream.hip", "offload.cpp")]
    return _library(srcs, os.path.join(HERE, "libqmoe_probe.so"),
                    ["-I", os.path.join(ROOT, "include"), "-I", csrc, "-DQMOE_PHASE_PROBE"], verbose,
                    jobs or min(8, os.cpu_count() or 4), build_subdir="_build_probe")


def build_synth(verbose=False, jobs=None):
    sdir = os.path.join(ROOT, "synth")
    return _library([os.path.join(sdir, "csrc", "synth.hip")], os.path.join(sdir, "libqmoe_synth.so"),
                    ["-ffp-contract=off"], verbose, 1)


def build_all(verbose=False):
    return [build_qmoe(verbose), build_synth(verbose)]


if __name__ == "__main__":
    if "--probe" in sys.argv:
        print("built", build_probe(verbose="-v" in sys.argv))
    else:
        for p in build_all(verbose="-v" in sys.argv):
            print("built", p)
