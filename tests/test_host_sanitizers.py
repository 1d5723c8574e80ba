"""Host sanitizer builds (AddressSanitizer and UndefinedBehaviorSanitizer), CPU only.

- oracle/ham_oracle.c with tests/sanitize/oracle_main.c (gcc): ham_oracle_forward in
  every configuration it takes and its error returns; leaks are checked as well.
- The host side of the C ABI, attention_sequence_mixing_amd/csrc/ham_api.cpp (g++,
  host-only against the HIP headers) with tests/sanitize/api_main.cpp, linked with the
  ordinary objects of the HIP sources: the workspace-size functions over a sweep of
  shapes (byte counts past 2^32 included) and every entry point's argument checks.  No
  call reaches a device.

Any sanitizer report aborts the program (halt_on_error), so a zero exit status means
none was raised and every expected return code held.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "attention_sequence_mixing_amd")
CSRC = os.path.join(PKG, "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-4000:]}"
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11"] + FLAGS + [os.path.join(ROOT, "oracle", "ham_oracle.c"),
                                        os.path.join(SAN, "oracle_main.c"), "-lm", "-o", exe])
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert "0 failure(s)" in out, out


def _device_objects():
    """The ordinary objects of the HIP sources, built again if any is missing or older
    than a source or header."""
    from attention_sequence_mixing_amd import build
    srcs = glob.glob(os.path.join(CSRC, "*.hip"))
    headers = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    newest = max(os.path.getmtime(f) for f in srcs + headers)
    objs = [os.path.join(build.BUILD, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest for o in objs):
        build.build()
    return objs


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="g++ or the HIP runtime is not installed")
def test_c_abi_host_side_under_asan_ubsan(tmp_path):
    objs = _device_objects()
    api = str(tmp_path / "ham_api_san.o")
    drv = str(tmp_path / "api_main.o")
    exe = str(tmp_path / "api_san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")] + inc + FLAGS +
         ["-c", os.path.join(CSRC, "ham_api.cpp"), "-o", api])
    _run(["g++", "-std=c++17"] + inc + FLAGS + ["-c", os.path.join(SAN, "api_main.cpp"), "-o", drv])
    _run(["g++", "-fsanitize=address,undefined", drv, api] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # the HIP runtime keeps allocations to the end of the process: no leak check here
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert "0 failure(s)" in out, out
