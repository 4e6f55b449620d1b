"""Sanitizer builds on the CPU: the C oracle, and the host side of libsgc
(layouts, helpers, workspace queries, every argument check the compute
calls make before queuing GPU work), compiled with
-fsanitize=address,undefined and driven by the programs in tests/sanitize/.
No GPU is used: the library's validation returns before any HIP call.  The
device code of the library is compiled as usual; the sanitizers apply to
host code only.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "compressed_sgd_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
          os.path.join(ROOT, "oracle", "sgc_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle driver ok" in r.stdout


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs the ROCm toolchain")
def test_library_host_code_under_sanitizers(tmp_path):
    # host-only sanitizer flags: each -fsanitize= goes after -Xarch_host
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
             "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")) + ["abi_driver.cpp"]

    def compile_one(f):
        src = os.path.join(SAN if f.endswith(".cpp") else CSRC, f)
        obj = str(tmp_path / (f.rsplit(".", 1)[0] + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime is not instrumented and keeps allocations past exit
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = _run([exe], env=env)
    assert "abi driver ok" in r.stdout
