"""Build libkvstore.so (all HIP sources, gfx950) in the package directory,
and beside it libkvstore_debug.so: the same kernels with the C ABI built with
KVS_DEBUG, whose calls first check the device-resident preconditions
(cu_seqlens_q, seqlens_k, table entries, slots) on the GPU and return
KVS_ERR_INVALID on a violation (loaded when the environment sets KVS_DEBUG=1),
libkvstore_calib.so: the benchmark's MFMA calibration kernel
(include/kvstore_calib.h), kept out of the attention library, and
libkvstore_phases.so: the attention library with the decode kernel's phase
timestamps (decode.hip built with KVS_PHASE_TIMES; bench.py --decode-phases).

    python -m attention_kv_store_amd.build            # both libraries
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
DEBUG_LIB = os.path.join(PKG, "libkvstore_debug.so")
SOURCES = ["api.hip", "store.hip", "rope.hip", "prefill.hip", "decode.hip", "mixed.hip"]
# the debug library: api.hip again with KVS_DEBUG, plus the check kernel
DEBUG_SOURCES = [("api.hip", "api_debug.o", ["-DKVS_DEBUG"]), ("validate.hip", "validate.o", [])]
# the benchmark's MFMA calibration kernel, a library of its own
CALIB_LIB = os.path.join(PKG, "libkvstore_calib.so")
CALIB_SOURCES = [("calib.hip", "calib.o", [])]
# the profiling library: decode.hip again with its phase probes
PHASES_LIB = os.path.join(PKG, "libkvstore_phases.so")
PHASES_SOURCES = [("decode.hip", "decode_phases.o", ["-DKVS_PHASE_TIMES"])]
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
    jobs = [(src, src.replace(".hip", ".o"), []) for src in SOURCES] + DEBUG_SOURCES + CALIB_SOURCES + PHASES_SOURCES
    for src, o, extra in jobs:
        obj = os.path.join(objdir, o)
        cmd = [hipcc(), *common, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
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
    release = objs[:len(SOURCES)]
    debug = [o for o in release if not o.endswith(os.sep + "api.o")] + objs[len(SOURCES):len(SOURCES) + len(DEBUG_SOURCES)]
    n0 = len(SOURCES) + len(DEBUG_SOURCES)
    calib = objs[n0:n0 + len(CALIB_SOURCES)]
    phases = [o for o in release if not o.endswith(os.sep + "decode.o")] + objs[n0 + len(CALIB_SOURCES):]
    out_dir = os.path.dirname(out)
    for lib_out, lib_objs in ((out, release), (os.path.join(out_dir, os.path.basename(DEBUG_LIB)), debug),
                              (os.path.join(out_dir, os.path.basename(CALIB_LIB)), calib),
                              (os.path.join(out_dir, os.path.basename(PHASES_LIB)), phases)):
        tmp = lib_out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib_out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    main()
