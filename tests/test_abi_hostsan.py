"""The C ABI's argument checks (tests/test_abi_cpu.py) run again against a
build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer:
every rejected call, workspace query and error text path, with any
out-of-bounds access, use after free or undefined behaviour on the host
aborting the run. No GPU is used (every call is rejected before a launch)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_argument_checks_under_host_sanitizers():
    sys.path.insert(0, os.path.join(ROOT, "compressed_sparse_kv_compress_amd"))
    try:
        import build_sanitized
    finally:
        sys.path.pop(0)
    lib = build_sanitized.build()
    env = dict(os.environ,
               CSKV_LIBRARY=lib,
               LD_PRELOAD=build_sanitized.runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
    # the binding did load the instrumented build, and the build is instrumented
    probe = subprocess.run([sys.executable, "-c",
                            "import compressed_sparse_kv_compress_amd._lib as L; print(L.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip().endswith("libcskv_hostsan.so"), probe.stdout + probe.stderr
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_" in syms and "__ubsan_handle_" in syms
