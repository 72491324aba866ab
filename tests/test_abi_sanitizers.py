"""The C ABI's host validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library is built once more with its host code instrumented (device code
as usual, every -fsanitize= applied to the host pass only), and the ABI tests
of tests/test_abi.py run against that build in a child process with the ASan
runtime preloaded: every entry point's argument checks, on NULL, misaligned,
undersized and out-of-range arguments, must run without a sanitizer report.
(No GPU is touched: every call there fails validation before any launch.)
"""

import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang ASan runtime in this toolchain")
def test_abi_validation_under_host_sanitizers(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "_isd_build", os.path.join(ROOT, "introspective_strided_decoding_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    out = os.path.join(ROOT, "_build", "host_sanitizers", "libisd.so")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    build.build(out=out, extra=build.HOST_SANITIZERS,
                link_extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                            "-shared-libasan"])
    rt = _asan_runtime()
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env.update(ISD_LIBRARY=out, LD_PRELOAD=rt,
               LD_LIBRARY_PATH=os.path.dirname(rt) + os.pathsep + env.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=0:log_path={log}")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(p).read() for p in glob.glob(log + "*"))
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:] + reports[-3000:]
    assert "passed" in res.stdout
    assert reports == "", reports[-5000:]
