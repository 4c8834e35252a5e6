"""Build libwq.so (HIP for gfx950) in-tree with hipcc.

    python -m bit_weight_only_wq_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwq.so")
SOURCES = ["wq_api.hip", "wq_quantize.hip", "wq_gemv.hip", "wq_gemv_lowbit.hip", "wq_gemv_nf4.hip", "wq_gemm_mfma.hip", "wq_gemm_xr.hip", "wq_kv.hip", "wq_dequant.hip", "wq_workspace.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # No packed fp32 instructions: they are kept out of every kernel here.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    from . import gen_nf4
    gen_nf4.write()                      # csrc/wq_nf4_levels.h (NF4 level table)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
