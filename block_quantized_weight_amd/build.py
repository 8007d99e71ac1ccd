"""Builds libqgemv.so (the HIP library behind the C ABI in include/qgemv.h) in-tree.

Each translation unit under csrc/ is compiled by hipcc for gfx950 in parallel
and linked into block_quantized_weight_amd/libqgemv.so.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemv.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 VALU ops are disabled for all device code.  Matrix-core results
# stay in ordinary VGPRs (no copies out of accumulation registers before the
# per-block scale is applied): measured faster for every co-batch shape.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, obj):
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return err


def build(verbose=True):
    """Compile every HIP source and link libqgemv.so (always rebuilds)."""
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="qgemv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
            for src, msg in zip(srcs, ex.map(_compile, srcs, objs)):
                if verbose and msg.strip():
                    print(f"[build] {os.path.basename(src)}:\n{msg}", file=sys.stderr)
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        os.replace(out_tmp, LIB)
    if verbose:
        print(f"[build] {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
