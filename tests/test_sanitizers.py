"""CPU sanitizer runs: the oracle's pins under AddressSanitizer and
UndefinedBehaviorSanitizer (gcc), and the C ABI's host-side checks with the
library's host code built with the same sanitizers (clang's runtime; no GPU:
every call there is rejected or validated before any launch).  Each suite runs
in a child process with the sanitizer runtime preloaded; any report fails it."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC_ASAN = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
CLANG_ASAN = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


def _run_suite(files, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


@pytest.mark.skipif(not os.path.exists(GCC_ASAN), reason="gcc's libasan is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_asan.so"))
    out = _run_suite(["tests/test_oracle_pins.py", "tests/test_oracle_combine.py",
                      "tests/test_oracle_routing_variants.py", "tests/test_oracle_backward.py"],
                     {"LD_PRELOAD": GCC_ASAN, "MOE_ORACLE_LIB_PATH": lib})
    assert " passed" in out


@pytest.mark.skipif(not CLANG_ASAN, reason="clang's ASan runtime is not installed")
def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from mixture_experts_layer_45_amd import build as moe_build
    if not os.path.exists(os.path.join(moe_build.BUILD, "gemm.o")):
        pytest.skip("build() has not been run (no objects under _build/)")
    lib = moe_build.build_host_sanitized(str(tmp_path / "libmoe_asan.so"))
    out = _run_suite(["tests/test_abi_host.py"], {"LD_PRELOAD": CLANG_ASAN[-1], "MOE_LIB_PATH": lib})
    assert " passed" in out
