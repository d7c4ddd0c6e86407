"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libtsp.so with tsp_api.hip's host side instrumented (argument checks, workspace
layout, launch order; the gfx950 kernels are built as usual) and runs the CPU ABI tests
against it in a child process that preloads the ASan runtime. A sanitizer report ends that
process with a non-zero status. No kernel is launched.
"""

import os
import subprocess
import sys

import pytest

from long_context_transformer_amd import build, tsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(tsp.LIB_PATH),
                                reason="libtsp.so not built (python -m long_context_transformer_amd.build)")


def test_abi_tests_pass_under_host_sanitizers():
    try:
        lib = build.build_sanitized()
        runtime = build.asan_runtime()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"sanitized build unavailable: {e}")
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], check=True, text=True,
                               stdout=subprocess.PIPE).stdout
    assert "__asan_" in undefined and "__ubsan_" in undefined, "library is not instrumented"
    env = dict(os.environ, TSP_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really loads the instrumented build
    probe = subprocess.run([sys.executable, "-c",
                            "from long_context_transformer_amd import tsp; tsp.load(); "
                            "print(sum('_build_san/libtsp.so' in l for l in open('/proc/self/maps')))"],
                           cwd=ROOT, env=env, text=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                           timeout=300)
    assert probe.returncode == 0 and int(probe.stdout.split()[-1]) > 0, probe.stdout + probe.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, text=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                         timeout=600)
    tail = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, tail
    assert " passed" in res.stdout and "skipped" not in res.stdout, tail
