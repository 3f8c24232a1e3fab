"""The C ABI's argument validation under host AddressSanitizer and UndefinedBehaviorSanitizer:
the library sources are built with the sanitizers on their host code only (device code is
unchanged) together with tests/abi_sanitize.cpp, which calls every entry point with invalid
arguments; every call must return its documented status and the sanitizers must stay silent.
Runs on the CPU (no GPU is used: each call fails before any device work)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_rank_linear_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asan")
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".cpp", ".hip"))
            and f != "bench_stream.hip"]
    exe = str(out / "abi_sanitize")
    # sanitizers on the host compilation only: each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *san]
    objs = []
    for src in srcs + [os.path.join(ROOT, "tests", "abi_sanitize.cpp")]:
        obj = str(out / (os.path.basename(src) + ".o"))
        lang = "c++" if src.endswith("abi_sanitize.cpp") else "hip"
        r = subprocess.run([hipcc, *flags, "-x", lang, "-c", src, "-o", obj], capture_output=True, text=True,
                           timeout=900)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *san, *objs, "-o", exe], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_abi_validation_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "ok: 0 failures" in r.stdout
