"""Build step: compile the HIP sources under csrc/ into libpesti.so (gfx950).

Run as `python -m dequantize_mat_vec_amd.build`; the package entry script's
build() calls the same function.  hipcc cross-compiles for gfx950 without a
GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO = PKG_DIR.parent
SRC_DIR = PKG_DIR / "csrc"
INCLUDE_DIR = REPO / "include"
LIB_PATH = PKG_DIR / "libpesti.so"
ARCH = "gfx950"

# Packed float32 VALU ops are turned off for every device compilation; the
# host pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(SRC_DIR.glob("*.hip"))


def build(verbose: bool = False) -> Path:
    """Compile every source into libpesti.so (always recompiles)."""
    objs = []
    obj_dir = PKG_DIR / "_build"
    obj_dir.mkdir(exist_ok=True)
    procs = []
    for src in sources():
        obj = obj_dir / (src.stem + ".o")
        cmd = [hipcc(), *[f for f in HIP_FLAGS if f != "-shared"], "-c", "-I", str(INCLUDE_DIR),
               str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        msgs = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln
                and "is not a recognized feature" not in ln]
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and any(m.strip() for m in msgs):
            print("\n".join(msgs), flush=True)
    if failed:
        for src, text in failed:
            sys.stderr.write(f"--- {src.name}\n{text}\n")
        raise RuntimeError("HIP compilation failed")
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
