"""The library from C: a C99 consumer of include/grz.h, built with gcc against
the regular library and with clang + AddressSanitizer against a build whose
host code is instrumented (-Xarch_host -fsanitize=address), and the header from
C++.  Host logic only:
plan helpers on pseudo-random plans and argument errors reported before any
launch (tests/native/host_checks.c)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "host_checks.c")
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "gradient_reduce_zero_amd")
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_consumer_against_the_library(tmp_path):
    exe = tmp_path / "host_checks"
    _run(["gcc", "-std=c99", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{INC}", f"-I{ROCM}/include",
          SRC, f"-L{PKG}", "-lgrz", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)])
    assert "host checks passed" in _run([str(exe)]).stdout


def _asan_runtime():
    for root, _, files in os.walk(f"{ROCM}/lib/llvm/lib/clang"):
        if "libclang_rt.asan-x86_64.so" in files:
            return root
    return None


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc") or _asan_runtime() is None,
                    reason="hipcc or the clang ASan runtime missing")
def test_host_code_under_address_sanitizer(tmp_path):
    from gradient_reduce_zero_amd.build import FLAGS, SRC as HIP_SRC
    lib = tmp_path / "libgrz.so"
    flags = [f for f in FLAGS if f not in ("-O3",)] + ["-O1", "-g"]
    _run([f"{ROCM}/bin/hipcc", *flags, "-Xarch_host", "-fsanitize=address", "-shared-libsan",
          f"-I{INC}", HIP_SRC, "-o", str(lib)])
    exe = tmp_path / "host_checks_asan"
    rt = _asan_runtime()
    _run([f"{ROCM}/llvm/bin/clang", "-g", "-O1", "-fsanitize=address", "-shared-libsan",
          "-D__HIP_PLATFORM_AMD__", f"-I{INC}", f"-I{ROCM}/include", SRC, f"-L{tmp_path}",
          "-lgrz", f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib", f"-Wl,-rpath,{rt}",
          "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    assert "host checks passed" in _run([str(exe)], env=env).stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no C++ compiler")
def test_header_compiles_as_cpp(tmp_path):
    # A C++ consumer sees the same declarations through the header's extern "C"
    # guard (syntax and linkage only, nothing runs).
    src = tmp_path / "use.cpp"
    src.write_text('#include "grz.h"\n'
                   'static_assert(sizeof(grz_bucket) == 16, "bucket layout");\n'
                   'static_assert(sizeof(grz_adamw_args) == 28, "args layout");\n'
                   'int (*const reduce)(const void* const*, int, int, const grz_bucket*, int, int,'
                   ' int, void*, double*, hipStream_t) = dp_reduce_scatter_mean;\n'
                   'int main() { return reduce == nullptr; }\n')
    _run(["g++", "-std=c++17", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", f"-I{INC}",
          f"-I{ROCM}/include", str(src)])
