"""The ABI host tests (argument checks, plan builders, workspace queries,
status strings: everything that runs on the host side of libhydra) once more
against a build whose host code is instrumented by AddressSanitizer and
UndefinedBehaviorSanitizer (build.py --sanitize), in a child process that
preloads clang's sanitizer runtime. Any out-of-bounds access, use after
free or undefined behaviour on those paths aborts the child."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _env(lib, rt):
    return dict(os.environ, LD_PRELOAD=rt, HYDRA_LIB=lib,
                ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_abi_host_suite_under_address_and_undefined_behaviour_sanitizers():
    from speculative_decoding_hydra_amd import build as B

    lib = B.build(sanitize=True)
    rt = B.sanitizer_runtime()
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout and "__ubsan_handle" in nm.stdout, "host code is not instrumented"
    probe = ("import speculative_decoding_hydra_amd._lib as L; L.lib(); "
             "m = open('/proc/self/maps').read(); print('libhydra_san.so' in m, 'libclang_rt.asan' in m)")
    r = subprocess.run([sys.executable, "-c", probe], env=_env(lib, rt), cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.split() == ["True", "True"], r.stdout + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], env=_env(lib, rt), cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
