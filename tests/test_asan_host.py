"""Host-only sanitizer runs (CPU; no GPU is touched).

* The oracle's C source, built with gcc under AddressSanitizer (leak checks on) and
  UndefinedBehaviorSanitizer, runs its forward, step, gradients and diagonal-plus-low-
  rank forward on small packed inputs (tests/asan/oracle_asan.c).
* The C boundary's host code (gated_delta_rule_20_amd/csrc/gdn_abi.hip), built with
  the sanitizers on its host pass only, is driven with arguments every entry point must
  reject, the workspace-size queries and out-of-range enum values
  (tests/asan/abi_asan.cpp; kernel launchers are stubs that no call reaches).
Both programs abort on the first sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ("address", "undefined")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-fopenmp", "-o", exe,
         os.path.join(ROOT, "tests", "asan", "oracle_asan.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"]
        + ["-fsanitize=" + s for s in SAN])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2")
    r = run([exe], env=env)
    assert "clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not available")
def test_boundary_host_code_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", "-fsanitize=" + s]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "gated_delta_rule_20_amd", "csrc")]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"] + host_san + inc
    abi_o, main_o, exe = (str(tmp_path / n) for n in ("abi.o", "main.o", "abi_asan"))
    run([hipcc] + common + ["-c", os.path.join(ROOT, "gated_delta_rule_20_amd", "csrc", "gdn_abi.hip"), "-o", abi_o])
    run([hipcc] + common + ["-c", os.path.join(ROOT, "tests", "asan", "abi_asan.cpp"), "-o", main_o])
    run([os.path.join(ROCM, "llvm", "bin", "clang++"), "-fsanitize=" + ",".join(SAN), abi_o, main_o,
         "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # the HIP runtime keeps allocations until exit: leak checks cover the oracle run only
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert "clean" in r.stdout
