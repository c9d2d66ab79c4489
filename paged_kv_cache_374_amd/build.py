"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_374_amd.build
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedkv.so")

# Packed-FP32 vector ops are disabled for all device code (hipcc would otherwise
# form them from ordinary float code).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-mllvm", "-amdgpu-mfma-vgpr-form=1",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + \
        sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(out: str = LIB, extra=()) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
           *sources(), "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # the host pass does not know the device-only feature
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
