"""Host-side sanitizer runs (CPU only, no GPU needed).

1. The library with AddressSanitizer + UndefinedBehaviorSanitizer on its host
   code (block_fp8_mixture_route_amd/build.py, sanitize=True): the C-ABI
   argument checks, layer planning and launch set-up, exercised by
   tests/test_abi.py (every host-side rejection, the stage and workspace
   queries) under clang's shared ASan runtime.
2. The CPU oracle built with gcc's -fsanitize=address,undefined, exercised by
   every oracle pin (tests/test_oracle_*.py) under gcc's libasan.

Each runs pytest in a child process with the runtime preloaded and the
sanitized build selected through BFP8MOE_LIB / BFP8MOE_ORACLE_LIB; a
sanitizer report aborts the child (no recovery), so a green run means none
fired.  Leak detection is off (the Python interpreter itself is not
instrumented).

    python tests/run_sanitized.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's shared ASan runtime was not found under /opt/rocm/lib/llvm")
    return hits[-1]


def gcc_asan_runtime() -> str:
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def run(label: str, env_extra: dict, args: list) -> int:
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               **env_extra)
    print(f"== {label}: {' '.join(args)}", flush=True)
    rc = subprocess.call([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *args],
                         cwd=ROOT, env=env)
    print(f"== {label}: exit {rc}", flush=True)
    return rc


# A child that hands the sanitized oracle a destination one row too short:
# ASan must stop it (proof that the runtime is live in these runs).
_PLANTED = """
import numpy as np
from oracle import oracle as O
x = np.zeros((2, 128), np.uint16)
q = np.zeros((1, 128), np.uint8)
s = np.zeros(2, np.float32)
O.lib().oracle_quant_fp8(O._p(x), 2, 128, 0, O._p(q), O._p(s))
"""


def planted_overflow_is_caught(olib: str) -> bool:
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", LD_PRELOAD=gcc_asan_runtime(), BFP8MOE_ORACLE_LIB=olib)
    r = subprocess.run([sys.executable, "-c", _PLANTED], cwd=ROOT, env=env, capture_output=True, text=True)
    caught = r.returncode != 0 and "AddressSanitizer" in r.stderr
    print(f"== planted out-of-bounds write in the sanitized oracle: {'caught' if caught else 'NOT caught'}",
          flush=True)
    return caught


def main() -> int:
    from block_fp8_mixture_route_amd import build as hip_build
    from oracle import oracle as O

    lib = hip_build.build(sanitize=True)
    olib = O.build(force=True, sanitize=True)
    if not planted_overflow_is_caught(olib):
        return 1
    rc1 = run("library host code (clang ASan + UBSan)", {"LD_PRELOAD": clang_asan_runtime(), "BFP8MOE_LIB": lib},
              ["tests/test_abi.py"])
    rc2 = run("oracle (gcc ASan + UBSan)", {"LD_PRELOAD": gcc_asan_runtime(), "BFP8MOE_ORACLE_LIB": olib},
              sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))))
    return 0 if rc1 == 0 and rc2 == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
