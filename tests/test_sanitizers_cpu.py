"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

* The fp64 oracle, built with gcc -fsanitize=address,undefined, runs every
  function on small inputs and edge cases (tests/sanitize_oracle_main.c).
* libdsa's sources are built with the host side under the same sanitizers
  (hipcc -Xarch_host -fsanitize=...; device code is compiled as usual and
  never runs here) and the C ABI's host path -- validation, workspace sizes,
  launch planning -- is fuzzed with edge-value sizes
  (tests/sanitize_abi_main.cpp).
Any sanitizer report aborts the driver with a non-zero status.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "sparse_attention_11_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-std=c11", *SAN, "-fno-omit-frame-pointer",
          os.path.join(HERE, "sanitize_oracle_main.c"), os.path.join(ROOT, "oracle", "dsa_oracle.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_path_under_asan_ubsan(tmp_path):
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              *host_san, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "sanitize_abi_main.cpp")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *common, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", *host_san, *objs, "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout
