"""Build libmdn.so in-tree with hipcc for gfx950.

    python -m chunkwise_delta_rule_amd.build

Each HIP source is compiled to an object (in parallel), then linked into
``chunkwise_delta_rule_amd/libmdn.so``; the benchmark's ceiling kernels
(``csrc/peaks.hip``) go into ``libmdn_peaks.so`` beside it.  Packed-fp32
instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmdn.so")
PEAKS_LIB = os.path.join(PKG, "libmdn_peaks.so")
SOURCES = ["api.hip", "chunk_bwd.hip", "chunk_fwd.hip", "chunk_fused.hip", "decode.hip", "gates.hip",
           "layer_io.hip"]
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs where they fit: the kernels apply
    # VALU arithmetic to their accumulators every chunk, and AGPR-resident
    # accumulators would need a copy each way
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmdn")
    return path


# Kernels whose explicit vmcnt waits count only their own loads: a register
# spill would add scratch traffic to the same counter and break those waits,
# so these must compile without scratch.
NO_SCRATCH = {"chunk_fused.hip": ("chunk_fwd_fused_kernel", "chunk_fwd_seg_kernel"),
              "chunk_fwd.hip": ("chunk_scan_bf16_kernel",),
              "chunk_bwd.hip": ("bwd_scan_bf16_kernel", "bwd_rescan_bf16_kernel")}


def _check_no_scratch(src: str, remarks: str) -> None:
    names = NO_SCRATCH.get(src, ())
    current = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and current and any(n in current for n in names) and int(m.group(1)) > 0:
            raise RuntimeError(f"{src}: kernel {current} uses {m.group(1)} bytes/lane of scratch; "
                               "its vmcnt waits assume it has none")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    _check_no_scratch(src, res.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmdn.so and libmdn_peaks.so.
    Returns the path of libmdn.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
