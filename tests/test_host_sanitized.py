"""The host ABI tests (tests/test_abi_host.py: packing, work lists, the
stall-free scheduler, the rotary table, sizes and every error path) run again
against a build of the library whose host code is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged), with
the sanitizer runtime preloaded into the child interpreter.  Any out-of-bounds
access, use after free or undefined behaviour in the host C++ aborts the child
with a report.  CPU only: no device code runs."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_abi_tests_pass_under_address_and_ub_sanitizers():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc / clang ASan runtime in this environment")
    sys.path.insert(0, ROOT)
    from chunked_prefill_hybrid_layer_amd import build as B
    tmp = tempfile.mkdtemp(prefix="hb_san_")
    lib = B.build(sanitize=True, out=os.path.join(tmp, "libhb_san.so"))
    log = os.path.join(tmp, "asan")
    env = dict(os.environ, LD_PRELOAD=rt, HB_LIB_PATH=lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = sorted(glob.glob(log + "*"))
    detail = "".join(open(p).read()[:4000] for p in reports)
    assert r.returncode == 0 and not reports, f"rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}\n{detail}"
    assert " passed" in r.stdout
