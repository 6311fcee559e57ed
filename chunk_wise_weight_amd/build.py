"""Build the HIP library libttt.so in-tree with hipcc for gfx950.

Run as ``python -m chunk_wise_weight_amd.build`` (or through the repository's
``__graft_entry__.build()``).  Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libttt.so")
SOURCES = ["inplace.hip", "lact.hip", "lact_bwd.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU forms anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 3) -> str:
    """Compile every source to an object (in parallel) and link libttt.so."""
    with tempfile.TemporaryDirectory(prefix="ttt_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        errors = []
        for cmd, p in procs:
            out, _ = p.communicate()
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                errors.append(f"{' '.join(cmd)}\n{out}")
            elif verbose and out.strip():
                print(out)
        if errors:
            raise RuntimeError("HIP build failed:\n" + "\n\n".join(errors))
        tmp_lib = LIB + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
