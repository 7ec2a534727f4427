"""Build libvsa_cube.so (gfx950) in-tree with hipcc.

    python -m block_sparse_video_cube_amd.build

Every source is compiled for gfx950 only.  Packed fp32 instructions are
switched off for the device code (the compiler otherwise forms them from
ordinary float code).
"""

from __future__ import annotations

import concurrent.futures
import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
OUT = os.path.join(PKG, "libvsa_cube.so")

SOURCES = ["api.hip", "permute.hip", "select.hip", "sta.hip", "attn_fwd.hip", "attn_lin.hip", "attn_bwd.hip", "quant.hip", "attn_fp8.hip", "linear.hip", "linear_bwd.hip", "linear_states.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            failed = True
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc compilation failed")
    tmp = OUT + ".tmp"
    rc, out = _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("hipcc link failed")
    # The library must load: an unresolved symbol (for example a kernel whose
    # host stub was not emitted) would otherwise only show at first use.
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"the linked library does not load: {e}") from e
    shutil.move(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
