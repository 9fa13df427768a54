"""CPU sanitizer runs over the native host code (no GPU).

* The fp64 oracle (oracle/gdn_oracle.c) built with ASan+UBSan under its whole pin
  suite, and its POSIX thread pool built with TSan (a standalone C driver, since a
  TSan-preloaded Python interpreter does not run reliably).
* The library's host-side argument validation (gdn_api.hip, host pass only) built with
  ASan+UBSan under the host ABI tests.
* A liveness check: each sanitizer configuration used here must report a planted
  error in a tiny throwaway C program, so a clean run above means something.

Each run is a child process, with the sanitizer runtime preloaded or linked in.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "oracle_threads.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(name + " not installed")
    return p


def _run(cmd, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def _cc(tmp_path, name, sources, san):
    exe = str(tmp_path / name)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-pthread", "-fno-omit-frame-pointer",
                           "-fsanitize=" + san, "-fno-sanitize-recover=all", "-o", exe] + sources + ["-lm"])
    return exe


def test_oracle_pin_suite_under_asan_ubsan():
    rt = _gcc_runtime("libasan.so")
    env = dict(ASAN_ENV, LD_PRELOAD=rt, GDN_ORACLE_SANITIZE="address,undefined")
    p = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_oracle_pins.py", "tests/test_oracle_golden.py",
              "tests/test_oracle_adaptive_pins.py"], env)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "passed" in p.stdout
    lib = os.path.join(ROOT, "oracle", "liboracle_address_undefined.so")
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms      # really instrumented


@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_oracle_thread_pool_driver(tmp_path, san):
    _gcc_runtime("libtsan.so" if san == "thread" else "libasan.so")
    exe = _cc(tmp_path, "oracle_threads", [DRIVER, ORACLE_SRC], san)
    p = _run([exe], dict(ASAN_ENV, TSAN_OPTIONS="halt_on_error=1"), timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "oracle thread check: ok" in p.stdout
    assert "WARNING: ThreadSanitizer" not in p.stderr and "ERROR: AddressSanitizer" not in p.stderr


def test_host_validation_under_asan_ubsan():
    try:
        from gated_deltanet_state_gdn_amd import build as gbuild
        gbuild.hipcc()
        rt = gbuild.clang_asan_runtime()
    except Exception as e:   # no ROCm toolchain on this host
        pytest.skip(str(e))
    lib = gbuild.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms
    env = dict(ASAN_ENV, LD_PRELOAD=rt, GDN_LIB_PATH=lib)
    p = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
              "tests/test_abi_host.py"], env)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "passed" in p.stdout and "skipped" not in p.stdout


PLANTED = {
    "thread": """
        #include <pthread.h>
        static int shared;
        static void *w(void *a) { (void)a; for (int i = 0; i < 100000; ++i) shared++; return 0; }
        int main(void) { pthread_t t[2]; for (int i = 0; i < 2; ++i) pthread_create(&t[i], 0, w, 0);
                         for (int i = 0; i < 2; ++i) pthread_join(t[i], 0); return shared == -1; }
    """,
    "address,undefined": """
        #include <stdlib.h>
        int main(int argc, char **argv) { (void)argv; int *p = malloc(4 * sizeof(int));
                                          int x = p[argc + 3]; free(p); return x == 12345; }
    """,
    "undefined": """
        #include <limits.h>
        int main(int argc, char **argv) { (void)argv; int x = INT_MAX - 1 + argc; return (x + 1) == 0; }
    """,
}


@pytest.mark.parametrize("san", sorted(PLANTED))
def test_sanitizers_report_planted_errors(tmp_path, san):
    _gcc_runtime("libtsan.so" if san == "thread" else "libasan.so" if "address" in san else "libubsan.so")
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent(PLANTED[san]))
    exe = _cc(tmp_path, "planted", [str(src)], san)
    p = _run([exe], dict(ASAN_ENV, TSAN_OPTIONS="halt_on_error=1"), timeout=120)
    assert p.returncode != 0
    assert any(s in p.stderr for s in ("ThreadSanitizer", "AddressSanitizer", "runtime error")), p.stderr
