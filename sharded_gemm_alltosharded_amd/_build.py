"""Build libshardgemm.so (the HIP library behind include/shardgemm.h) in-tree
for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libshardgemm.so")
SOURCES = ["api.hip", "generic.hip", "tile.hip", "skinny.hip", "q4.hip", "q4_wide.hip", "q4s.hip", "layout.hip",
           "tile_dma.hip", "backward.hip", "q4tile.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code (the host pass warns it does
    # not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed", "-Wno-unknown-warning-option",
]

# Per-file flags.  The 4-bit streaming kernel scales every group's MFMA result
# on the vector unit; with the default register choice the MFMAs write the
# accumulation registers and each group then copies them to ordinary ones
# (about half of the loop's vector instructions).  The VGPR form of the MFMA
# removes the copies; it pays for 17 to 32 tokens (q4_wide.hip) and measured
# slower or no faster for fewer tokens, in the other 4-bit kernels and in the
# dense ones (and spills in tile.hip).
FILE_FLAGS = {
    "q4_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _objdir():
    d = os.path.join(HERE, "_build")
    os.makedirs(d, exist_ok=True)
    return d


HEADERS = [os.path.join(CSRC, "internal.h"), os.path.join(CSRC, "q4_stream.h"),
           os.path.join(os.path.dirname(HERE), "include", "shardgemm.h")]


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in [src, *HEADERS])


def build_library(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library;
    incremental=True recompiles only sources newer than their objects."""
    objdir = _objdir()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        if incremental and not _stale(os.path.join(CSRC, src), obj):
            continue
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text, file=sys.stderr)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True, incremental="--incremental" in sys.argv))
