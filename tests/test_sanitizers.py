"""Sanitizer builds of the host-side code, run on the CPU.

- The C oracle under AddressSanitizer + UndefinedBehaviorSanitizer, and under
  ThreadSanitizer (its worker pool), driven on every path by
  tests/sanitize/oracle_driver.c.
- The library's host-side argument checks (kda_api.hip) under ASan + UBSan:
  that file is rebuilt with host-only sanitizer flags, linked with the other
  objects of the regular build, and the C-ABI test file runs against it with
  the sanitizer runtime preloaded.  Device code is built as usual; no GPU call
  is made.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "kda_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} exited {r.returncode}:\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.parametrize("flags", [
    ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    ["-fsanitize=thread"],
], ids=["asan_ubsan", "tsan"])
def test_oracle_under_sanitizers(tmp_path, flags):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", *flags, ORACLE_C, DRIVER_C, "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "oracle driver: ok" in r.stdout


def test_host_checks_under_asan_ubsan(tmp_path):
    objs = {n: os.path.join(ROOT, "_build", n + ".hip.o")
            for n in ("kda_chunk", "kda_decode", "kda_onchip", "kda_verify")}
    missing = [o for o in objs.values() if not os.path.exists(o)]
    if missing or not ASAN_RT or not os.path.exists(HIPCC):
        pytest.skip(f"needs the regular build's objects ({missing}), hipcc and clang's ASan runtime")
    api_o, lib = str(tmp_path / "kda_api.o"), str(tmp_path / "libkda_asan.so")
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gated_delta_rule_65_amd", "csrc"),
          *host, "-c", os.path.join(ROOT, "gated_delta_rule_65_amd", "csrc", "kda_api.hip"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o, *objs.values(),
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-shared-libsan", "-o", lib])
    env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], KDA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = _run(["python", "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-x", "-q",
              "-p", "no:cacheprovider"], env=env, cwd=ROOT, timeout=900)
    assert " passed" in r.stdout
