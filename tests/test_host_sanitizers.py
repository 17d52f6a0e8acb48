"""The host side of the library (argument validation, workspace planning, the
ring bookkeeping, byte counts, the C ABI's error paths) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU.

The HIP sources are compiled again with the sanitizers on their host code only
(the device code is unchanged: GPU sanitizers are not used), linked into a
separate library, and the host-only ABI and ring tests run against it in a
child process with the sanitizer runtime preloaded.  Any report fails the
test: AddressSanitizer aborts on its first error, UndefinedBehaviorSanitizer
is set to halt on its first."""

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_kv_cache_chunk_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ["api", "append", "absorb", "attend", "attend_wide", "attend_mha", "upproj", "cache_ring"]
# host-only sanitizer flags: each -fsanitize= goes to the host compilation
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not os.path.exists(HIPCC) or _asan_runtime() is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    out = tmp_path_factory.mktemp("sanitized")

    def compile_one(src):
        obj = str(out / f"{src}.o")
        cmd = [HIPCC, "-c", os.path.join(CSRC, src + ".hip"), "-o", obj, "--offload-arch=gfx950", "-O1", "-g",
               "-std=c++17", "-fPIC", "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}",
               f"-I{CSRC}"] + HOST_SANITIZE
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = str(out / "libmla_hip_sanitized.so")
    r = subprocess.run([HIPCC, "-shared", "-o", lib] + objs + ["--offload-arch=gfx950", "-fPIC"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def test_library_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms


def test_host_tests_clean_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), MLA_HIP_LIB=sanitized_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_ring.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    which = subprocess.run([sys.executable, "-c", "from latent_kv_cache_chunk_amd import mla; print(mla.LIB_PATH)"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert which.stdout.strip() == sanitized_lib, which.stdout + which.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert " passed" in log
