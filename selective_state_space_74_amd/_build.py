"""Build libssm.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")
# The micro-benchmarks that bench.py times (the scan's arithmetic ceiling, the
# matrix instructions' issue rate; not part of the libssm.so boundary).
MICRO_SRCS = sorted(glob.glob(os.path.join(PKG, "micro", "*.hip")))
MICRO_LIB = os.path.join(PKG, "libssm_micro.so")
ARCH = "gfx950"

# Packed fp32 (v_pk_*_f32) is kept out of the generated code.
HIPCC_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", INCLUDE, "-I", CSRC]


# Per-source extra flags.  The SSD kernel keeps its matrix-product
# accumulators in the ordinary VGPR file (the VGPR form of the MFMA
# instructions) instead of the accumulation registers, which saves the
# copies between the two files.
SOURCE_FLAGS = {"ssd_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def flags_for(src: str) -> list:
    return HIPCC_FLAGS + SOURCE_FLAGS.get(os.path.basename(src), [])


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; harmless
    noise = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libssm.so (always recompiles), and the
    micro-benchmarks into libssm_micro.so.  The library sources compile in
    parallel into a temporary directory, then link."""
    tmp = LIB + ".tmp"
    jobs = max(1, min(len(sources()), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="ssm_build_") as d:
        objs = [os.path.join(d, os.path.basename(src) + ".o") for src in sources()]
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run([hipcc(), *flags_for(so[0]), "-c", "-o", so[1], so[0]], verbose),
                        zip(sources(), objs)))
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs], verbose)
        mtmp = MICRO_LIB + ".tmp"
        _run([hipcc(), *HIPCC_FLAGS, "-shared", "-o", mtmp, *MICRO_SRCS], verbose)
    os.replace(tmp, LIB)
    os.replace(mtmp, MICRO_LIB)
    return LIB


def assembly(out_path: str, src: str | None = None) -> str:
    """Device assembly of one source (for inspecting the generated ISA)."""
    src = src or os.path.join(CSRC, "scan_fwd.hip")
    cmd = [hipcc(), *flags_for(src), "--cuda-device-only", "-S", "-o", out_path, src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
