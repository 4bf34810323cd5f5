"""The ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer.

The host half of the library (argument, configuration and CSR checks, the
workspace planner's overflow guards) is built once more with ASan and UBSan
(device code unchanged) and the host ABI tests run against that build in a
child process with the sanitizer runtime preloaded; any report aborts the run.
No test here touches a GPU.
"""

import os
import subprocess
import sys

import pytest

from lm_head_logprobs_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_lib():
    path = os.path.join(B.ASAN_BUILD, "librlloss_asan.so")
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
    srcs.append(os.path.join(ROOT, "include", "rlloss.h"))
    if not os.path.exists(path) or os.path.getmtime(path) < max(map(os.path.getmtime, srcs)):
        B.build_asan()
    return path


def test_abi_host_checks_clean_under_asan_and_ubsan(tmp_path):
    try:
        lib, rt = _asan_lib(), B.asan_runtime()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = dict(os.environ)
    env.update(RL_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:5000])
