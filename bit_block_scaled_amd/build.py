"""Build libbbs.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbbs.so")
SOURCES = ["abi.hip", "quantize.hip", "gemm.hip", "gemm_nvfp4.hip", "gemm_mxfp8.hip",
           "codec.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # every FP32 step of the quantizers is one IEEE operation
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build() -> str:
    """Compile every HIP source and link libbbs.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def build_probe() -> str:
    """Compile the instruction probes used by tests/test_gpu_isa.py."""
    src = os.path.join(os.path.dirname(HERE), "tests", "hip", "probe.hip")
    out = os.path.join(os.path.dirname(src), "libprobe.so")
    subprocess.check_call([HIPCC, *FLAGS, "-shared", src, "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
