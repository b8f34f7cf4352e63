"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.

abi.cpp (descriptor validation, workspace layout, the allocation-free entry
point's checks, tracing) and recompute.cpp (the 128-bit planner arithmetic)
are compiled with host-only sanitizers -- every -fsanitize flag is placed
after -Xarch_host, so no GPU code is instrumented -- and linked with the
regular kernel objects into a separate library.  The CPU ABI and planner
tests then run against that library in a child process with the ASan runtime
preloaded; any sanitizer report aborts the child and fails this test.
"""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_recompute_attention_attn_amd")
HOST_SOURCES = ("abi.cpp", "recompute.cpp")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.fixture(scope="module")
def sanitized_lib():
    from selective_recompute_attention_attn_amd import build as b
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    kernel_objs = [os.path.join(b.BUILD_DIR, s + ".o") for s in b.SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        b.build()
    out = tempfile.mkdtemp(prefix="srat_san_")
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out, src + ".o")
        cmd = [b.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}",
               f"-I{os.path.join(ROOT, 'include')}", *SAN_FLAGS, "-x", "hip", "-c",
               os.path.join(PKG, "csrc", src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        objs.append(obj)
    lib = os.path.join(out, "libsrat.so")
    subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *objs, *kernel_objs, "-o", lib,
                    "-Xarch_host", "-shared-libsan", *SAN_FLAGS[:4]], check=True, capture_output=True)
    return lib, rt


def test_sanitized_library_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", lib], check=True, capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_and_planner_tests_pass_under_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    runner = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from selective_recompute_attention_attn_amd import ops\n"
        f"ops.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        f"    {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r},\n"
        f"    {os.path.join(ROOT, 'tests', 'test_recompute_plan.py')!r}]))\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", runner], env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert " passed" in res.stdout, report
