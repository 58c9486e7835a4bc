"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU): api.cpp is rebuilt with the host
sanitizers, linked with the library's other objects from the last build, and
the ABI checks of test_abi_cpu.py run against that library in a child process
with the sanitizer runtime preloaded; any report ends the child with an error.
"""
import glob
import os
import subprocess
import sys

import pytest
import torch

import importlib.util as _iu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = _iu.spec_from_file_location(
    "_cabf_build", os.path.join(ROOT, "content_adaptive_block_fractal_amd", "build.py"))
build = _iu.module_from_spec(_spec)
_spec.loader.exec_module(build)


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(torch.cuda.is_available(), reason="the ABI checks run host-only")
def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    runtime = _runtime()
    objs = [os.path.join(build.BUILD, s + ".o") for s in build.SOURCES if s != "api.cpp"]
    if runtime is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("sanitizer runtime or library objects missing (run the build first)")
    api_o = str(tmp_path / "api.o")
    lib = str(tmp_path / "libcabf_sanitized.so")
    # host code only: every -fsanitize= is preceded by -Xarch_host
    compile_cmd = [build._hipcc(), *build.FLAGS, "-O1", "-g",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined",
                   "-x", "hip", "-c", os.path.join(build.CSRC, "api.cpp"), "-o", api_o]
    subprocess.run(compile_cmd, check=True, capture_output=True)
    subprocess.run([build._hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-o", lib,
                    api_o, *objs], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=runtime, CABF_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
