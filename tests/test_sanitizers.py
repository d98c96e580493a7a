"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

Two subprocesses, each with its sanitizer runtime preloaded (a process holds one ASan
runtime, so the oracle and the library run apart):

* the fp64 oracle (``oracle/liboracle_san.so``, gcc, ASan + UBSan on the whole
  library) under the oracle's pin tests;
* the library's host side (``libhypic_san.so``: the ABI translation unit, with the
  argument validation and dispatch, built with host-only ASan + UBSan and linked with
  the kernels' ordinary objects) under the host tests, which call every entry point
  with valid and invalid arguments and never reach the GPU.

UBSan aborts on its first report, and ASan reports end the process with an error; a
run passes only if the tests pass and neither sanitizer printed a report.  The
sanitized libraries come from ``__graft_entry__.build()``; without them the test is
skipped (it builds nothing itself).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SAN = os.path.join(ROOT, "oracle", "liboracle_san.so")
HYPIC_SAN = os.path.join(ROOT, "hybrid_prefill_amd", "libhypic_san.so")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehaviorSanitizer")


def _gcc_runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(preload, env_extra, test_file, probe):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = ":".join(preload)
    # the Python interpreter and torch are not instrumented: leaks at exit are theirs
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["CUDA_VISIBLE_DEVICES"] = ""          # host paths only
    env["HIP_VISIBLE_DEVICES"] = ""
    # the process runs under ASan and loads the sanitized copy, not the default build
    check = ("import ctypes; ctypes.CDLL(None).__asan_init; " + probe)
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "SANITIZED-COPY-LOADED" in r.stdout, r.stdout + r.stderr
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", test_file)]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_oracle_under_asan_ubsan():
    """The oracle's pin tests against the ASan + UBSan build of the oracle."""
    if not os.path.exists(ORACLE_SAN):
        pytest.skip("oracle/liboracle_san.so not built (run __graft_entry__.build())")
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    probe = ("import oracle; oracle._load(); "
             f"print('SANITIZED-COPY-LOADED' if oracle._LIB_PATH == {ORACLE_SAN!r} else oracle._LIB_PATH)")
    rc, out = _run([asan, ubsan], {"HYPIC_ORACLE_LIB": ORACLE_SAN}, "test_oracle_pins.py", probe)
    tail = "\n".join(out.strip().splitlines()[-25:])
    assert rc == 0, tail
    assert not any(r in out for r in REPORTS), tail
    assert " passed" in out, tail


def test_library_host_side_under_asan_ubsan():
    """The host tests (argument validation, shape checks, exported symbols) against the
    library whose ABI translation unit carries ASan + UBSan."""
    if not os.path.exists(HYPIC_SAN):
        pytest.skip("libhypic_san.so not built (run __graft_entry__.build())")
    asan = _clang_asan_runtime()
    if not asan:
        pytest.skip("clang's ASan runtime is not installed")
    probe = ("import hybrid_prefill_amd as hp; hp.lib(); "
             f"print('SANITIZED-COPY-LOADED' if hp.LIB_PATH == {HYPIC_SAN!r} else hp.LIB_PATH)")
    rc, out = _run([asan], {"HYPIC_LIB": HYPIC_SAN}, "test_abi_host.py", probe)
    tail = "\n".join(out.strip().splitlines()[-25:])
    assert rc == 0, tail
    assert not any(r in out for r in REPORTS), tail
    assert " passed" in out, tail
