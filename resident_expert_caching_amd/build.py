"""Compile ``libmoe_spark.so`` (HIP kernels + C ABI host runtime) for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libmoe_spark.so")
SOURCES = [os.path.join(HERE, "csrc", s) for s in ("kernels.hip", "q4_decode.hip", "qb_decode.hip", "prefill.hip", "runtime.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    """Always compiles (the result is written atomically next to this file)."""
    out = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # matrix-core results in ordinary VGPRs: the prefill GEMMs scale every
           # block's MFMA result in fp32, which would otherwise copy it out of AGPRs
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wno-unused-command-line-argument", "-Wno-pass-failed",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", out] + SOURCES + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(out, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
