"""Build libsdverify.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m speculative_decoding_verification_sd_amd.build

Compiles every csrc/*.hip translation unit with hipcc and links one shared
library next to this file.  Packed-FP32 instruction selection is switched
off for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libsdverify.so"
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file flags.  Verify attention never carries NaN through its max/exp
# chain (masked scores are -inf and unused LDS rows are zeroed), so its
# translation unit drops NaN-quieting canonicalisations around fmax.
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
                "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


PROBES = os.path.join(HERE, "probes")
PROBE_LIB = "libsdprobe.so"


def build_probes(verbose: bool = False) -> str:
    """libsdprobe.so: bench.py's measurement kernels (MFMA throughput, wave
    placement), kept out of the verify-step library."""
    cc = hipcc()
    out = os.path.join(HERE, PROBE_LIB)
    srcs = sorted(os.path.join(PROBES, f) for f in os.listdir(PROBES) if f.endswith(".hip"))
    cmd = [cc, *COMMON_FLAGS, *DEVICE_FLAGS, "-shared", "-o", out + ".tmp", *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probes:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, extra_flags=(), out: str = None) -> str:
    cc = hipcc()
    out = out or os.path.join(HERE, LIB_NAME)
    with tempfile.TemporaryDirectory(prefix="sdv_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *COMMON_FLAGS, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
                   *extra_flags, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                             if "packed-fp32-ops" not in l)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
            if verbose and msgs.strip():
                print(msgs)
            return obj

        with ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
            objs = list(ex.map(compile_one, sources()))
        tmp_out = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
    print(build_probes(verbose="-v" in sys.argv))
