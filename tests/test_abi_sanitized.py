"""The C-ABI layer's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (validation, aliasing checks, dispatch) is compiled with the host compiler together with
host-only stand-ins for the kernel launchers (tests/sanitize/launch_stub.cpp, which answer
hipErrorNoDevice as the real launchers do without a GPU), and tests/test_abi_cpu.py is run
against that library in a child process with the sanitizer runtime preloaded. Any sanitizer
report fails the test. No device code is built or run.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layerwise_qk_norm_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _gpu_present() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


def build_sanitized(out_dir: str) -> str:
    """Compile api.cpp and the launcher stand-ins with g++ and the sanitizers; return the .so."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    # the two spellings hipcc's device-side headers would define: the alignment attribute and
    # the symbol of a device variable as the host names it
    common = ["g++", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
              "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(X)=X",
              "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), *SAN]
    objs = []
    for src, name in ((os.path.join(CSRC, "api.cpp"), "api.o"),
                      (os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"), "stub.o")):
        obj = os.path.join(out_dir, name)
        subprocess.run([*common, "-c", src, "-o", obj], check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "libqknorm_sanitized.so")
    subprocess.run(["g++", "-shared", *SAN, *objs, "-o", lib, "-Wl,--no-undefined"], check=True,
                   capture_output=True, text=True)
    return lib


def runtime(name: str) -> str:
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.skipif(_gpu_present(), reason="the fake-pointer validation tests run on CPU only")
@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_validation_under_sanitizers(tmp_path):
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan:
        pytest.skip("libasan not found")
    lib = build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env["QKN_LIBRARY"] = lib
    env["LD_PRELOAD"] = " ".join(p for p in (asan, ubsan) if p)
    # the interpreter itself is not instrumented and keeps memory until exit: no leak report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    # every ABI test except the one that looks for the gfx950 code object, which a host-only
    # build does not carry
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-k", "not gfx950_code_object",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    summary = out.strip().splitlines()[-1]
    assert " passed" in summary and "skipped" not in summary and "failed" not in summary, summary
