"""Build libbitlinear.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m bit_gemm_02_amd.build   (or bit_gemm_02_amd.build.build()).
The library is written next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libbitlinear.so")
SOURCES = ["api.hip", "quant.hip", "decode.hip", "gemv.hip", "prefill.hip", "mixed.hip", "train.hip",
           "calib.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE semantics for the quantizers: no multiply-add contraction, correctly rounded fp32
    # division (the HIP default, stated explicitly), denormals kept.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # No packed-fp32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]

# Per-source additions.  The one-token kernels keep their MFMA accumulators in ordinary VGPRs:
# the decode-tile product accumulates four planes separately across wave-uniform branches, and
# in the accumulation registers the compiler copied all four in and out around every
# super-step (32 register moves per 16 weight rows x 256 weights, each read stalling on the
# MFMA that had just written it).
SOURCE_FLAGS = {
    "gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose: bool = False, output: str = LIBRARY, extra_flags=(), extra_link_flags=()) -> str:
    """Compile every source and link the shared library (to `output`, with `extra_flags` on
    every compile line and `extra_link_flags` on the link line); returns its path."""
    with tempfile.TemporaryDirectory(prefix="bitlinear_build_") as tmp:
        objs = [os.path.join(tmp, src.replace(".hip", ".o")) for src in SOURCES]

        def compile_one(src_obj):
            src, obj = src_obj
            cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, ()), *extra_flags, "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return src, subprocess.run(cmd, capture_output=True, text=True)

        # One hipcc process per source, several at a time (each is single-threaded).
        jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for src, r in pool.map(compile_one, zip(SOURCES, objs)):
                if r.returncode != 0:
                    raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        tmp_lib = output + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra_link_flags, *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
