"""Build the plain C caller of the library (c_check.c) against the in-tree libqknorm.so and
liboracle.so, with gcc and the HIP runtime's C API; the binary finds both libraries next to
the sources through its run path."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "layerwise_qk_norm_amd")
    orc = os.path.join(ROOT, "oracle")
    rpath = ":".join(["$ORIGIN/../../layerwise_qk_norm_amd", "$ORIGIN/../../oracle",
                      os.path.join(ROCM, "lib")])
    tmp = EXE + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                           os.path.join(HERE, "c_check.c"), "-L", pkg, "-lqknorm", "-L", orc,
                           "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                           f"-Wl,-rpath,{rpath}", "-o", tmp])
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
