"""Build the gfx950 HIP library in-tree: quantized_linear_attention_amd/libstq.so."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", "stq.hip"), os.path.join(PKG, "csrc", "alloc.cpp")]
DEPS = SRC + [os.path.join(PKG, "csrc", "stq_device.h"), os.path.join(ROOT, "include", "stq.h")]
LIB = os.path.join(PKG, "libstq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every floating-point contraction in the kernels is an explicit fma
    "-ffp-contract=off",
    # no packed fp32 VALU ops (v_pk_{add,mul,fma}_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(force=True, verbose=False):
    """Compile libstq.so (always when force=True)."""
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in DEPS):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SRC + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=False))
