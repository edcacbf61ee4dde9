"""Build libvca_attn.so, the HIP/C++ attention library, in-tree for gfx950.

    python -m varlen_causal_attention_amd.build

Compiles every source under csrc/ with hipcc (in parallel) and links one
shared library next to this file. Packed-fp32 instructions are disabled for
all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvca_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Kernel units are compiled once per element type: bf16 (namespace vca::bf)
# and fp16 (VCA_ELEM_F16, namespace vca::hf).
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_tiles.hip", "attn_bwd_roles.hip"]
HIP_SOURCES = ["attn_merge.hip", "attn_ring.hip", "attn_api.hip", "attn_timing.hip"]
CXX_SOURCES = ["attn_segments.cpp"]
# -amdgpu-mfma-vgpr-form=1: keep MFMA accumulators in VGPRs. The kernels keep
# their working set under the unified register budget; left to choose, the
# compiler parks accumulators in AGPRs and then shuttles hundreds of values
# per loop iteration between the two register files.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", "-Wno-unused-result"]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile(job) -> str:
    src, f16 = job
    obj = os.path.join(BUILD, os.path.basename(src) + (".f16" if f16 else "") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    defs = ["-DVCA_ELEM_F16"] if f16 else []
    cmd = [HIPCC, *COMMON, *VGPR_FORM, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True, asan_host_dir: str | None = None) -> str:
    """Build the library in-tree; with asan_host_dir, build instead a copy
    whose host code runs under AddressSanitizer (device code unchanged) into
    that directory, for the host-side tests:
        python -m varlen_causal_attention_amd.build --asan-host DIR
        VCA_ATTN_LIB=DIR/libvca_attn.so ASAN_OPTIONS=detect_leaks=0 \
          LD_PRELOAD=$(clang -print-file-name=libclang_rt.asan-x86_64.so) \
          python -m pytest tests/test_abi_host.py tests/test_dense_route.py"""
    global BUILD, LIB, COMMON
    if asan_host_dir:
        BUILD = os.path.join(os.path.abspath(asan_host_dir), "_build")
        LIB = os.path.join(os.path.abspath(asan_host_dir), "libvca_attn.so")
        COMMON = [c for c in COMMON if c != "-O3"] + [
            "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
            "-fno-omit-frame-pointer"]
    os.makedirs(BUILD, exist_ok=True)
    jobs = ([(s, False) for s in KERNEL_SOURCES] + [(s, True) for s in KERNEL_SOURCES]
            + [(s, False) for s in HIP_SOURCES + CXX_SOURCES])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = LIB + ".tmp"
    san = ["-Xarch_host", "-fsanitize=address"] if asan_host_dir else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--asan-host":
        build(asan_host_dir=sys.argv[2])
    else:
        build()
