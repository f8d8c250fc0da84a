"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of libdsa.so is built with the sanitizers on its host side only (the
device code is compiled as usual and never runs here), and the CPU tests of
the C ABI -- argument validation of every entry point, workspace sizes and
the workspace layouts over a grid of shapes -- run against it in a child
process with the sanitizer runtime preloaded.  Out-of-bounds host accesses,
signed overflow in the size arithmetic and the like then fail the run
instead of passing unnoticed.  A small deliberate overflow, built beside it,
shows that the harness reports such errors.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_attention_long_03_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# host-side sanitizers only (each flag behind -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    try:
        hipcc = BLD.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("sanitizer runtime not available")
    out = tmp_path_factory.mktemp("san")
    srcs = sorted(f for f in os.listdir(BLD.CSRC) if f.endswith(".hip"))

    def compile_one(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        cmd = [hipcc, *BLD._flags(), *BLD.EXTRA.get(src, []), *SAN, "-c", os.path.join(BLD.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}: {r.stderr[-2000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(out / "libdsa_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={BLD.ARCH}", "-shared", "-fPIC", *SAN, "-shared-libsan", *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib, rt, out


def _env(rt):
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_sanitized_library_is_instrumented(sanitized):
    lib, _, _ = sanitized
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_harness_reports_a_heap_overflow(sanitized):
    """A deliberate one-past-the-end write in a separate tiny library."""
    _, rt, out = sanitized
    src = out / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int overflow(int n) { int* p = (int*)malloc(n * sizeof(int)); p[n] = 1; int v = p[0]; free(p); "
                   "return v; }\n")
    so = str(out / "liboverflow.so")
    r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-shared", "-fPIC", "-fsanitize=address", "-shared-libsan",
                        str(src), "-o", so], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    code = f"import ctypes; ctypes.CDLL({so!r}).overflow(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(rt), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_abi_host_paths_clean_under_sanitizers(sanitized):
    lib, rt, _ = sanitized
    code = ("import sys\n"
            f"sys.path.insert(0, {ROOT!r})\n"
            "from sparse_attention_long_03_amd import binding as B\n"
            f"B.LIB_PATH = {lib!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
            f"                      {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r},\n"
            f"                      {os.path.join(ROOT, 'tests', 'test_workspace_layout_cpu.py')!r}]))\n")
    r = subprocess.run([sys.executable, "-c", code], env=_env(rt), capture_output=True, text=True, timeout=600,
                       cwd=ROOT)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert r.returncode == 0 and " passed" in r.stdout, report
