"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): pa_alloc.cpp and pa_host.cpp are built by the host compiler with
the sanitizers, linked with stand-ins for the device-side launches
(tests/sanitize/device_stubs.cpp) and driven by tests/sanitize/host_checks.cpp:
random allocator histories against a plain model, host-only pool lifecycles,
random split-K plans, and bad arguments to every host entry point.  A control
program with a deliberate out-of-bounds read shows the instrumentation is
live."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_walk_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-I", os.path.join(ROCM, "include")]


def _need_toolchain():
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    if not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("no HIP runtime library to link against")


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env.pop("LD_PRELOAD", None)        # the sanitizer runtime must come first
    return env


def _build(sources, exe):
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in sources:
        o = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        subprocess.run(["g++", *FLAGS, "-c", src, "-o", o], check=True, capture_output=True, text=True)
        objs.append(o)
    subprocess.run(["g++", "-fsanitize=address,undefined", *objs, "-L", os.path.join(ROCM, "lib"),
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-o", exe],
                   check=True, capture_output=True, text=True)


def test_sanitizers_are_live():
    _need_toolchain()
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(OUT, "oob.cpp")
    with open(src, "w") as f:
        f.write("#include <vector>\nint main(int c, char**) { std::vector<int> v(4); return v.data()[3 + c]; }\n")
    exe = os.path.join(OUT, "oob")
    subprocess.run(["g++", "-O0", "-fsanitize=address,undefined", src, "-o", exe], check=True,
                   capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=60)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr


def test_host_code_under_asan_ubsan():
    _need_toolchain()
    exe = os.path.join(OUT, "host_checks")
    _build([os.path.join(CSRC, "pa_alloc.cpp"), os.path.join(CSRC, "pa_host.cpp"),
            os.path.join(SAN, "device_stubs.cpp"), os.path.join(SAN, "host_checks.cpp")], exe)
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=300)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host checks passed" in r.stdout
