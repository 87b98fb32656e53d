"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library compiled with the sanitizers on its host code only
(validation, plan choice, workspace and size queries; the gfx950 device code
is built as usual and never launched), linked with tests/abi_sanitize.cpp,
which walks every plan query over a grid of shapes (each plan kind forced in
turn) and every entry point's error paths; any sanitizer report aborts the
run.  No kernel is launched, so no GPU is needed."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_07_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
# host-code sanitizers only: each -fsanitize= applies to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr
    return res


@pytest.mark.timeout(900)
def test_host_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not installed")
    objs = []
    cmds = []
    for f in ("api", "gemm", "gemm_large", "layout", "moe", "quantize"):
        o = str(tmp_path / f"{f}.o")
        objs.append(o)
        cmds.append([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O2", "-g",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
                     "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, f + ".hip"), "-o", o])
    drv = str(tmp_path / "driver.o")
    cmds.append([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                 "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "abi_sanitize.cpp"),
                 "-o", drv])
    with ThreadPoolExecutor(6) as ex:
        list(ex.map(_run, cmds))
    exe = str(tmp_path / "abi_sanitize")
    _run([CLANG, "-fsanitize=address,undefined", *objs, drv, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "all host checks passed" in run.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out
