"""Build ``libmoe_w4a16.so`` for gfx950 with hipcc (in-tree).

Every HIP source is compiled with packed-FP32 instruction selection turned
off (``-packed-fp32-ops``): the kernels are written in scalar FP32 and must
not be turned into v_pk_{add,mul,fma}_f32.  Kernel-argument preloading is
on (``-amdgpu-kernarg-preload-count=16``): a kernel's leading scalar and
pointer arguments arrive in SGPRs with the wave, so the decode kernels'
first loads need no scalar load of the kernarg segment (firmware without
the feature runs the compiler's fallback loads instead).
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_w4a16.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-mllvm", "-amdgpu-kernarg-preload-count=16",
              "-Wall", "-Wno-unused-function"]
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = common + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(item):
    src, p = item
    _, err = p.communicate()
    lines = [l for l in (err or "").splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
