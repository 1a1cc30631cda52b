"""Build the HIP library in-tree: gemv_decode_projections_amd/lib/libgdproj.so (gfx950).

Each translation unit compiles in parallel with hipcc, then hipcc links the
shared library. Packed FP32 VALU instructions are disabled for all device
code (the backend would otherwise form them from plain float code).
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(LIBDIR, "libgdproj.so")

SOURCES = [
    "proj_api.hip",
    "bench.hip",
    "skinny_bf16_nt1.hip",
    "skinny_bf16_nt2.hip",
    "skinny_f32.hip",
    "skinny_z.hip",
    "skinny_sk.hip",
    "tiled_variants.hip",
    "rowdot_variants.hip",
    "wide_variants.hip",
    "wide_dma_variants.hip",
]

ARCH = os.environ.get("GDP_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source extra flags. Tiled kernels keep MFMA accumulators in VGPRs: with
# AGPR accumulators the register allocator rotates them across the unrolled
# k-steps and copies them back every loop trip (measured slower for the
# skinny kernels, so only here).
EXTRA = {
    "tiled_variants.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "wide_variants.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "wide_dma_variants.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU-only feature flag; that warning is harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
