"""Builds libtq.so (host C++ + HIP kernels for gfx950) in the package directory.

Usage: python -m kv_cache_compression_turboquant_amd.build
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")

SOURCES = ["tq_host.cpp", "tq_encode128.hip", "tq_encode_prod128.hip", "tq_encode_mse32.hip", "tq_misc.hip", "tq_score128.hip", "tq_attn128.hip",
           "tq_general.hip", "tq_cache128.hip", "tq_split128.hip", "tq_peaks.hip", "tq_noalloc.hip", "tq_prefill128.hip",
           "tq_fwht128.hip", "tq_kvgen.hip", "tq_encode64.hip"]

# Packed FP32 VALU instructions are disabled for all device code.  MFMA results go to ordinary
# VGPRs rather than accumulation registers: the kernels post-process their accumulators with
# VALU code, and the AGPR form costs a copy in each direction per use (and, for the decode
# attention, one wave per SIMD of occupancy).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose=False, defines=(), out=None, tmp=None):
    """Compiles every source into libtq.so for gfx950; raises on failure.  `defines` (NAME=VALUE)
    override the kernels' compile-time tuning defaults; `out` / `tmp` redirect the library and
    the object directory."""
    objs = []
    out = out or LIB
    tmp = tmp or os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(tmp, src + ".o")
        objs.append(obj)
        cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-c",
               "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *["-D" + d for d in defines],
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        # the host pass does not know the device feature flag: drop that notice
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp_lib = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objs, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
