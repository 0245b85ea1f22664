"""Build libbfp8moe.so (HIP, gfx950) in-tree with hipcc.

    python -m block_fp8_mixture_route_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbfp8moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE semantics the bit-exact kernels rely on
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the leading kernel arguments arrive in SGPRs with the dispatch (no
    # scalar load of the argument segment before the first address is known;
    # the compiler keeps a loading prologue for firmware that does not preload)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
# argument checks, planning and launch set-up of the C ABI); the device code
# is built as always.  The library then needs clang's shared ASan runtime
# preloaded into the process (tests/run_sanitized.py does this).
SAN_LIB = os.path.join(PKG, "libbfp8moe_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libasan"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    from . import gen_exp_table

    gen_exp_table.write()  # csrc/exp_neg_table.h, included by device.h
    srcs = sources()
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
