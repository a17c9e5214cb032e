"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle (oracle/lora_oracle.c) and the host-only calls of the library
(csrc/batch_former.cpp, csrc/status.cpp) are rebuilt with
-fsanitize=address,undefined and the CPU tests that exercise them run again in
a child process with the ASan runtime preloaded and LORA_SANITIZE=1, which
makes both loaders take the sanitizer builds.  Any report fails the run
(-fno-sanitize-recover, halt_on_error), and so does a leak: LeakSanitizer
keeps each allocation's direct caller only, so tests/lsan_suppressions.txt
can set aside the interpreter's own allocations without hiding ours.  A
planted heap overflow and a planted leak in a throwaway library show that
the sanitizers are live in that child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the CPU tests that call the oracle's C code or the native batch former
SUITES = ["tests/test_oracle_pins.py", "tests/test_stacked_oracle.py", "tests/test_fused_oracle.py",
          "tests/test_batch_former.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN = _runtime("libasan.so")
pytestmark = pytest.mark.skipif(ASAN is None, reason="no gcc AddressSanitizer runtime on this host")


def _env():
    env = dict(os.environ)
    env.update(LD_PRELOAD=ASAN, LORA_SANITIZE="1", PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=1:malloc_context_size=2:halt_on_error=1:exitcode=86",
               LSAN_OPTIONS=f"suppressions={os.path.join(ROOT, 'tests', 'lsan_suppressions.txt')}:"
                            "print_suppressions=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def sanitized_builds():
    import oracle
    from adapter_gemv_amd import build as hip_build
    return oracle.build(force=True, sanitize=True), hip_build.build_host_sanitized()


@pytest.mark.parametrize("call,report", [("oob(4)", "heap-buffer-overflow"), ("leak(1000)", "LeakSanitizer")])
def test_planted_mistake_is_reported(tmp_path, call, report):
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int oob(int i) { int *a = malloc(4 * sizeof(int)); int v = a[i]; free(a); return v; }\n"
                   "int leak(int n) { int *a = malloc(n * sizeof(int)); a[0] = n; return a[0]; }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-fsanitize=address,undefined", "-g", str(src), "-o", str(lib)],
                   check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).{call}"
    r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]


def test_cpu_suites_clean_under_asan_and_ubsan(sanitized_builds):
    oracle_lib, host_lib = sanitized_builds
    probe = ("import oracle, adapter_gemv_amd as lg; print(oracle.library_path()); "
             "print(lg.host_lib()._name); print(lg.status_string(2))")
    r = subprocess.run([sys.executable, "-c", probe], env=_env(), cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = r.stdout.split("\n")
    assert lines[0] == oracle_lib and lines[1] == host_lib and lines[2].startswith("LORA_ERR_SHAPE"), r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *SUITES],
                       env=_env(), cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
