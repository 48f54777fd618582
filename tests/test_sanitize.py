"""The C-ABI host layer and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/ builds qmm_api.cpp (argument validation, overlap checks and
dispatch of every entry point) with its kernel launchers replaced by stubs
(host_stubs.cpp), together with the oracle, into one host program
(driver.cpp) compiled with -fsanitize=address,undefined and no recovery:
the program drives every entry point with well-formed and malformed
descriptors over fake device addresses and every oracle routine on small
seeded inputs.  Any sanitizer report aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _have_sanitizers(tmp):
    src = os.path.join(tmp, "probe.c")
    with open(src, "w") as f:
        f.write("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", *SAN, src, "-o", os.path.join(tmp, "probe")], capture_output=True, text=True)
    return r.returncode == 0


def test_host_layer_and_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc / g++ not available")
    tmp = str(tmp_path)
    if not _have_sanitizers(tmp):
        pytest.skip("the compiler has no address / undefined-behaviour sanitizer runtime")
    inc = ["-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, lang, extra in (
            (os.path.join(ROOT, "oracle", "qmm_oracle.c"), "gcc", ["-std=c11", "-ffp-contract=off"]),
            (os.path.join(ROOT, "quantized_matmul_ggml_amd", "csrc", "qmm_api.cpp"), "g++",
             ["-x", "c++", "-std=c++17", *inc]),
            (os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "g++", ["-std=c++17", *inc]),
            (os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), "g++", ["-std=c++17", *inc])):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        r = subprocess.run([lang, *SAN, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"compile {src}:\n{r.stderr[-3000:]}"
        objs.append(obj)
    exe = os.path.join(tmp, "sanitized")
    r = subprocess.run(["g++", *SAN, *objs, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
