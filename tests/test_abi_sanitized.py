"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled with the host pass instrumented by
``-fsanitize=address,undefined`` (UB fatal; the gfx950 device code is built
as usual, uninstrumented) into a separate shared library,
and the no-GPU ABI tests (``test_abi_cpu.py``: argument validation, workspace
checks, error strings, size queries with extreme arguments) run against it
in a child process with the sanitizer runtime preloaded.  A memory error or
undefined behaviour anywhere on the host path (the validation, the size
arithmetic, the error-message handling, the launchers up to the HIP call)
ends that run with a sanitizer report.  No kernel runs: without a device the
launches the valid calls reach return a HIP error.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

from w8a8_quantized_verification_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitized")
LIB = os.path.join(OUT, "libw8a8_sanitized.so")
# each -fsanitize applies to the host pass only (there is no device pass here)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    r = subprocess.run([B.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("the ASan runtime of the HIP toolchain is not installed")
    return path


def build_sanitized() -> str:
    os.makedirs(OUT, exist_ok=True)
    flags = [f for f in B.FLAGS if f != "-O3" and not f.startswith("-I")]
    flags += ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer", *SAN,
              f"-I{os.path.join(ROOT, 'include')}"]

    def comp(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([B.hipcc(), *flags, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"compile of {src} failed:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                        *SAN, *objs, "-o", LIB],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-3000:]}"
    return LIB


def instrumented_symbols(lib: str) -> set:
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return {line.split()[-1] for line in r.stdout.splitlines() if line.strip()}


def test_abi_validation_under_asan_and_ubsan():
    rt = asan_runtime()
    lib = build_sanitized()
    # the library really is instrumented (it calls into both runtimes)
    syms = instrumented_symbols(lib)
    assert any(n.startswith("__asan_report_") for n in syms), "no ASan checks in the build"
    assert any(n.startswith("__ubsan_handle_") for n in syms), "no UBSan checks in the build"
    env = dict(os.environ)
    env.update({
        "W8A8_LIBRARY": lib,
        "LD_PRELOAD": rt,
        # the interpreter and torch are not instrumented: no leak report at
        # exit, no complaint about their allocator pairs or link order
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:alloc_dealloc_mismatch=0:"
                        "halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import w8a8_quantized_verification_amd._lib as L; "
             "assert L.LIB_PATH == %r; L.lib(); print('loaded', L.LIB_PATH)" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, (r.stdout + r.stderr)[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out
