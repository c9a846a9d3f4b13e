"""Build libkvstore.so (all HIP sources, gfx950) in the package directory.

    python -m attention_kv_store_amd.build            # release build
    python -m attention_kv_store_amd.build --verbose

Every HIP source is compiled with packed-fp32 instructions disabled for the
device (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass
prints a harmless "not a recognized feature" warning for that flag.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvstore.so")
SOURCES = ["api.hip", "store.hip", "rope.hip", "prefill.hip", "decode.hip", "calib.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def build(verbose: bool = False, out: str = LIB) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}",
    ]
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *common, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for src, pr in procs:
        log, _ = pr.communicate()
        log = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed = True
            sys.stderr.write(f"--- {src} failed ---\n{log}\n")
        elif verbose and log.strip():
            print(log)
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    main()
