"""Host-side AddressSanitizer runs (CPU only): the C oracle built with ASan and
UBSan under its pins, and the host code of the HIP library (argument checks,
size limits, workspace queries) built with ASan under the C-ABI tests.

Each run is a child process with the sanitizer runtime preloaded and the
instrumented build named through VLA_ORACLE_LIB / VLA_LIB; a sanitizer report
aborts the child, so the test fails.  Device code is built without the
sanitizer (only the host side of each hipcc compile is instrumented).  A
planted heap overflow in a throwaway C file checks that the set-up reports
errors at all.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow

ENV_ASAN = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's ASan runtime is not installed")
    return p


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("the ROCm clang ASan runtime is not installed")
    return hits[-1]


def _child(cmd, preload, extra_env, timeout=600):
    env = dict(os.environ, **ENV_ASAN, **extra_env, LD_PRELOAD=preload)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def _gcc_asan_lib(src, out):
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", src, "-o", out, "-lm"], check=True)
    return out


def test_planted_overflow_is_reported(tmp_path):
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int *p = malloc(n * sizeof(int)); int s = p[n];"
                   " free(p); return s; }\n")
    lib = _gcc_asan_lib(str(src), str(tmp_path / "liboverflow.so"))
    r = _child([sys.executable, "-c",
                f"import ctypes; ctypes.CDLL({lib!r}).planted(4)"],
               _gcc_asan_runtime(), {})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = _gcc_asan_lib(os.path.join(ROOT, "oracle", "vla_oracle.c"),
                        str(tmp_path / "liboracle_asan.so"))
    r = _child([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                "tests/test_oracle_pins.py", "tests/test_oracle_grad_pins.py",
                "tests/test_oracle_baseline_pins.py"],
               _gcc_asan_runtime(), {"VLA_ORACLE_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def _build_host_asan_library(out_dir):
    sys.path.insert(0, ROOT)
    from long_context_sequence_amd import build as b
    host_only = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([b._hipcc(), *b.COMMON, *b.DEVICE_FLAGS, *host_only, "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib = os.path.join(out_dir, "libvla_asan.so")
    # a host link (the device code is already embedded in each object)
    subprocess.run([os.path.join(rocm, "llvm", "bin", "clang++"), "-shared", "-fPIC",
                    "-fsanitize=address", *objs, f"-L{rocm}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{rocm}/lib", "-o", lib], check=True)
    return lib


def test_abi_checks_under_asan(tmp_path):
    preload = _clang_asan_runtime()
    lib = _build_host_asan_library(str(tmp_path))
    r = _child([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                "tests/test_abi_cpu.py"], preload, {"VLA_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
