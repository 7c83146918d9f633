"""The CPU oracle and the library's host code (argument checks, launch
planning, metadata validators, workspace sizing) rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer, and run under the CPU tests
that exercise them, in a child process with the sanitizer runtime
preloaded.  Any report (out-of-bounds access, use after free, undefined
behaviour) aborts the child and fails the test.  No GPU is used: the host
tests only call entry points that return before any launch."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run_child(setup, test_files, tmp_path):
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
            f"{setup}\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', *{test_files!r}]))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), env=_env(), capture_output=True,
                         text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


pytestmark = pytest.mark.skipif(_runtime() is None or not os.path.exists(CLANG),
                                reason="the clang sanitizer runtime is not installed")


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """pa_oracle.c built with ASan + UBSan (single-threaded: the OpenMP
    pragmas compile away) under every oracle pin."""
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([CLANG, "-std=c11", "-fPIC", "-shared", *SAN, "-o", lib,
                    os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"], check=True)
    setup = f"import oracle.oracle as O; O._LIB = {lib!r}"
    files = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_oracle_blocks_pins.py",
                                                        "test_oracle_f16_pins.py", "test_oracle_int8_pins.py")]
    out = _run_child(setup, files, tmp_path)
    assert " passed" in out


def test_host_api_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """pa_api.cpp's host code built with ASan + UBSan (host side only; the
    kernels' objects are the normal build's) under the C-ABI host tests."""
    build = os.path.join(ROOT, "paged_kv_attention_mapping_amd", "_build")
    objs = [os.path.join(build, f) for f in ("pa_store.hip.o", "pa_decode.hip.o", "pa_prefill.hip.o")]
    if not all(os.path.exists(o) for o in objs):
        from paged_kv_attention_mapping_amd import build as pa_build
        pa_build.build()
    host = []
    for flag in SAN:
        host += ["-Xarch_host", flag]
    api_o = str(tmp_path / "pa_api_san.o")
    lib = str(tmp_path / "libpa_san.so")
    subprocess.run([HIPCC, "-std=c++17", "-fPIC", "--offload-arch=gfx950", *host,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "paged_kv_attention_mapping_amd", "csrc"),
                    "-c", os.path.join(ROOT, "paged_kv_attention_mapping_amd", "csrc", "pa_api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined",
                    "-o", lib, api_o, *objs], check=True, capture_output=True)
    setup = f"import paged_kv_attention_mapping_amd._lib as L; L.LIB_PATH = {lib!r}"
    files = [os.path.join(ROOT, "tests", f) for f in ("test_abi_host.py", "test_zz_no_alloc.py")]
    out = _run_child(setup, files, tmp_path)
    assert " passed" in out
