"""The decode kernel's phase-probe build (KVS_PHASE_TIMES, the profiling
library libkvstore_phases.so): its probes write through vector memory
instructions only -- the device assembly holds no scalar-memory store,
atomic or write-back -- and the product build has no probe at all.  CPU only
(hipcc cross-compiles for gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_kv_store_amd", "csrc")
SCALAR_WRITES = ("s_store_", "s_atomic_", "s_buffer_store", "s_buffer_atomic", "s_dcache_wb", "s_scratch_store")


def _device_asm(tmp_path, defines):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "decode.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", *defines, "--cuda-device-only", "-S",
           os.path.join(CSRC, "decode.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


def test_phase_probes_use_vector_stores_only(tmp_path):
    asm = _device_asm(tmp_path, ["-DKVS_PHASE_TIMES"])
    assert "s_memrealtime" in asm
    bad = [l.strip() for l in asm.splitlines() if any(x in l for x in SCALAR_WRITES)]
    assert not bad, bad[:5]


def test_product_build_has_no_probes(tmp_path):
    asm = _device_asm(tmp_path, [])
    assert "s_memrealtime" not in asm
    assert "g_phase_t" not in asm
