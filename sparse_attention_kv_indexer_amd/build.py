"""Build libdsa_indexer.so in-tree with hipcc for gfx950.

``python -m sparse_attention_kv_indexer_amd.build`` (or ``build()``) compiles
every HIP source under ``csrc/`` into one shared library next to this file,
and the bench's HBM read probes (``csrc/probe/``) into ``libdsa_probe.so``.
It needs hipcc but no GPU.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdsa_indexer.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PROBE_LIB_PATH = os.path.join(HERE, "libdsa_probe.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: keeps loop-carried accumulators out of
    # AGPRs (which would be copied in and out on every iteration)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is needed to build the HIP library)")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def probe_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile the library and the probe library; returns the library's path.
    Always recompiles."""
    _compile(LIB_PATH, sources(), verbose, extra_flags)
    _compile(PROBE_LIB_PATH, probe_sources(), verbose, extra_flags)
    return LIB_PATH


def _compile(out: str, srcs: list[str], verbose: bool, extra_flags: list[str] | None) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
