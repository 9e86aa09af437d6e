"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/lora_oracle.c) is rebuilt with gcc's sanitizers and the
  oracle pins (tests/test_oracle_pins.py) run against that build in a
  subprocess (the sanitizer runtimes preloaded into it).
* The library's host code (argument checks, size queries, launch planning) is
  rebuilt with hipcc, sanitizers on the host side only, and linked with a small
  C harness (tests/sanitize/abi_checks.c) that calls every entry point with
  invalid arguments and asks the size queries for extreme sizes; nothing is
  enqueued, so no GPU is needed.

Any sanitizer report makes the run exit nonzero (halt on the first error).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from expand_token_adapter_amd import build as hip_build  # noqa: E402  (build recipe only; nothing is loaded)

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_runtime("libasan.so") is None, reason="no gcc sanitizers")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liblora_oracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
                    "-o", str(lib), os.path.join(ROOT, "oracle", "lora_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, **SAN_ENV)
    env["LORA_ORACLE_LIB"] = str(lib)
    env["LD_PRELOAD"] = f"{_gcc_runtime('libasan.so')}:{_gcc_runtime('libubsan.so')}"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/llvm/bin/clang++"), reason="no ROCm clang")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    hipcc = hip_build.hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", hip_build.INCLUDE, "-I", hip_build.CSRC]
    flags = [f for f in hip_build.HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    objs, cmds = [], []
    for src in hip_build.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        cmds.append([hipcc] + flags + san + inc + ["-c", os.path.join(hip_build.CSRC, src), "-o", obj])

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-3000:]

    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(run, cmds))
    clang = "/opt/rocm/llvm/bin/clang"
    harness = str(tmp_path / "abi_checks.o")
    run([clang, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", hip_build.INCLUDE, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_checks.c"), "-o", harness])
    exe = str(tmp_path / "abi_checks")
    run([clang + "++", "-fsanitize=address,undefined", harness] + objs +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    res = subprocess.run([exe], env=dict(os.environ, **SAN_ENV), capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "abi checks: ok" in res.stdout
