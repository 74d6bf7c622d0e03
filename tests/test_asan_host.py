"""The argument-validation layer under AddressSanitizer, on the host.

Every source is compiled with AddressSanitizer instrumentation of the host pass only
(the device code is built as usual and never runs: there is no GPU here), linked into a
shared library, and the CPU ABI tests (argument errors, workspace arithmetic, status strings,
exports) are run against it in a child interpreter that preloads the sanitizer runtime.
A heap or stack overflow, use after free or similar in the checks that run before any
device work fails this test with the sanitizer's report."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_25_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if not os.path.exists(HIPCC) or _asan_runtime() is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    out = tmp_path_factory.mktemp("asan")
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(out / (os.path.basename(src)[:-4] + ".o"))
        objs.append(obj)
        # the sanitizer flags are scoped to the host compiler
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-shared-libasan", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, pr in procs:
        text, _ = pr.communicate()
        assert pr.returncode == 0, f"{src}:\n{text}"
    lib = str(out / "libgptq_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-shared-libasan", "-o", lib] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib


def test_argument_validation_under_asan(asan_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    # the interpreter itself is not instrumented and keeps its arenas to the end
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23"
    env["GPTQ_ABI_LIB"] = asan_lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not compiles"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in text
