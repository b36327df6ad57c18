"""The library's host layer built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through the host ABI tests (argument validation, workspace sizing, error paths),
with no GPU. Only host code is instrumented (each -fsanitize= sits behind -Xarch_host);
device code is compiled as usual. Any sanitizer report fails the test."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_abi_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's ASan runtime is not installed")
    from kv_cache_compaction_amd import build as b

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
               "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(b.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libamc_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *SAN, "-Xarch_host",
                        "-shared-libasan", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    code = ("import sys; sys.path.insert(0, %r); import kv_cache_compaction_amd as amc; "
            "amc.LIB_PATH = %r; import pytest; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r, '-k', 'not binding']))"
            % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
