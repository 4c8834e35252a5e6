"""Build libwq.so (HIP for gfx950) and the read-stream probe libwq_probe.so
in-tree with hipcc: every source is compiled on its own (in parallel), then
linked.

    python -m bit_weight_only_wq_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwq.so")
PROBE_LIB = os.path.join(HERE, "libwq_probe.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["wq_api.hip", "wq_quantize.hip", "wq_gemv.hip", "wq_gemv_lowbit.hip", "wq_gemv_nf4.hip",
           "wq_gemm_mfma.hip", "wq_gemm_xr.hip", "wq_gemm_sk.hip", "wq_gemm_q4.hip", "wq_gemm_qs.hip", "wq_gemm_ts.hip", "wq_gemm_kw.hip", "wq_kv.hip", "wq_dequant.hip"]
PROBE_SOURCES = ["probe/wq_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # No packed fp32 instructions: they are kept out of every kernel here.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    return res.returncode, out


def _link(hipcc, sources, lib, jobs, verbose):
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = [os.path.join(OBJ_DIR, s.replace("/", "_").replace(".hip", ".o")) for s in sources]
    cmds = [[hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(HERE, "csrc", s), "-o", o]
            for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for s, (rc, out) in zip(sources, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = lib + ".tmp"
    rc, out = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"hipcc link of {os.path.basename(lib)} failed ({rc}):\n{out}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    from . import gen_nf4
    gen_nf4.write()                      # csrc/wq_nf4_levels.h (NF4 level table)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    _link(hipcc, PROBE_SOURCES, PROBE_LIB, jobs, verbose)
    return _link(hipcc, SOURCES, LIB, jobs, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
