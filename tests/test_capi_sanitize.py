"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library sources with the sanitizers on the host side only (device
code is compiled as usual and never runs here) and links them with
tests/capi_sanitize_driver.cpp.  The driver calls every entry point with
arguments that validation must reject, and the size queries over a grid of
shapes up to the largest the checks admit; no call passes validation, so
nothing is launched and no GPU is needed.  Any sanitizer report, or a status
other than the expected one, fails the test.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_importance_scoring_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "capi_sanitize_driver.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
# host-only instrumentation: every sanitizer flag of a hipcc line goes through -Xarch_host
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def _compile(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", *HOST_SANITIZE.split(), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stderr[-4000:]}"
    return obj


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not present")
def test_c_abi_host_code_is_sanitizer_clean(tmp_path):
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(min(8, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, str(tmp_path)), sources))
    exe = os.path.join(str(tmp_path), "capi_sanitize")
    link = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", DRIVER,
            *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the HIP runtime keeps allocations until exit
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"sanitized driver failed (status {r.returncode}):\n{out[-6000:]}"
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert "ok: 0 mismatches" in r.stdout
    shutil.rmtree(str(tmp_path), ignore_errors=True)
