"""The library's host code (argument checks, planning, workspace layout,
schedule parameters) built with AddressSanitizer and UndefinedBehaviorSanitizer
for the host side only, linked with checking stand-ins of the kernel
launchers (tests/host_sanitize/stub_launch.cpp) and run through a sweep of
every entry point (tests/host_sanitize/driver.cpp).  Needs no GPU: the
stand-ins never touch device memory, and device code is built without
sanitizers."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_gemm_int4_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
ROCM = "/opt/rocm"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    return hipcc, clang


def test_host_code_under_asan_ubsan(tmp_path):
    hipcc, clang = _tools()
    srcs = [os.path.join(CSRC, "hm_api.cpp"), os.path.join(CSRC, "plan_host.cpp"),
            os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "driver.cpp")]
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + HOST_SAN

    def compile_one(pair):
        src, obj = pair
        r = subprocess.run([hipcc, "-c", src, "-o", obj] + flags, capture_output=True, text=True)
        return src, r

    with cf.ThreadPoolExecutor(4) as ex:
        for src, r in ex.map(compile_one, zip(srcs, objs)):
            assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
    exe = str(tmp_path / "host_sweep")
    link = [clang, "-fsanitize=address,undefined", "-o", exe] + objs + [
        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # leaks inside the HIP runtime's own initialisation are not this code's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = env.get("HIP_VISIBLE_DEVICES", "")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "host sweep ok" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
