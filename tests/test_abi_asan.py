"""The host side of the C ABI under AddressSanitizer and UBSan (CPU only).

Rebuilds the library's API translation unit (argument checks, sizes,
layouts, header parsing, the composition of each entry point) with
host-side AddressSanitizer, links it with the library's kernel objects, and
runs tests/abi_asan_driver.c against it: host-only calls on good, truncated
and corrupted input, and every device entry point with arguments that fail
validation (nothing is launched, so no GPU is needed). The run must be clean.
Device code is built as usual: sanitizers apply to host code only.
"""

import glob
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "kv_cache_compression_layer_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_abi_host_code_runs_clean_under_sanitizers(tmp_path):
    objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.hip.o")) if "cg_api" not in o)
    if not objs:
        pytest.skip("library objects not built")
    from kv_cache_compression_layer_amd import build as bld

    api_o = str(tmp_path / "cg_api_asan.o")
    flags = [f for f in bld.FLAGS if f != "-O3"]
    subprocess.run([HIPCC, *flags, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(PKG, "csrc", "cg_api.hip"),
                    "-o", api_o], check=True)
    lib = str(tmp_path / "libcg_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-o", lib, api_o, *objs], check=True)
    exe = str(tmp_path / "abi_asan")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(HERE, "abi_asan_driver.c"), lib, f"-Wl,-rpath,{tmp_path}",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    # Leak checking is off: the HIP runtime keeps allocations until exit.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "ok" in r.stdout
