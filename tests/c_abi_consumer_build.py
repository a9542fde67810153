"""Build tests/_bin/c_abi_consumer (tests/c_abi_consumer.c): gcc, the HIP
runtime's C API and libditnorm.so, found at run time next to the repository's
package directory (rpath $ORIGIN), so the built tree runs wherever it is copied.

    python tests/c_abi_consumer_build.py [OUT]
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_consumer.c")
OUT = os.path.join(HERE, "_bin", "c_abi_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out=OUT):
    os.makedirs(os.path.dirname(out), exist_ok=True)
    pkg = os.path.join(ROOT, "dit_adaln_row_amd")
    rel = os.path.relpath(pkg, os.path.dirname(out))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
           # the HIP runtime headers ask a non-hipcc compiler to name the platform
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", out,
           "-L", pkg, "-lditnorm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/" + rel, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
