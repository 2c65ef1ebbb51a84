"""Build librq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m mixed_precision_block_amd.build

Each translation unit compiles to _build/<name>.o in parallel, then one
shared library is linked next to this file.  The hardware probes that
bench.py --only probes runs (probes/probes.hip) become a second library,
libprobe.so, beside it; librq never loads it.  Always rebuilds.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librq.so")
PROBE_SRC = os.path.join(HERE, "probes", "probes.hip")
PROBE_LIB = os.path.join(HERE, "libprobe.so")
SOURCES = ["rq_api.hip", "quant_mx.hip", "gemm.hip", "gemm_pipe.hip", "gemv_nibble.hip", "norm_gate_kv.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the GPU feature flag
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        msg = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, msg

    def build_probes():
        tmp = PROBE_LIB + ".tmp"
        msg = _run([HIPCC, *FLAGS, "-shared", "-o", tmp, PROBE_SRC])
        os.replace(tmp, PROBE_LIB)
        return msg

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        probes = ex.submit(build_probes)
        for obj, msg in ex.map(compile_one, SOURCES):
            objs.append(obj)
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
        probe_msg = probes.result()
        if verbose and probe_msg.strip():
            print(probe_msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
