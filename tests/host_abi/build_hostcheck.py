"""Build the sanitizer host-check library of the C ABI (no device code).

    python tests/host_abi/build_hostcheck.py OUT.so

Compiles the ABI's host sources (wq_api.hip, wq_plan.cpp) as plain C++ with
g++ together with stub launchers, instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer.  A process that loads it needs the ASan runtime
preloaded (``LD_PRELOAD=$(g++ -print-file-name=libasan.so)``).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "weight_only_bit_dequant_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def build(out):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM_INCLUDE,
           "-x", "c++", os.path.join(CSRC, "wq_api.hip"), os.path.join(CSRC, "wq_plan.cpp"),
           os.path.join(HERE, "stub_launchers.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("host-check build failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-6000:]))
    return out


if __name__ == "__main__":
    print(build(sys.argv[1]))
