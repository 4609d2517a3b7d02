"""CPU sanitizer leg: the oracle's C and the host code of the C ABI, built with
AddressSanitizer and UndefinedBehaviorSanitizer (every report fatal), each exercised by its own
host tests in a child process that preloads the matching sanitizer runtime.

* oracle/hta_oracle.c and oracle/step_oracle.c: gcc, then the oracle's pin tests (closed forms,
  brute force, the pages' worked values, planted-mistake checks) with HTA_ORACLE_LIBRARY
  pointing at the sanitized build.
* include/hta.h's entry points: hta_api.hip (descriptor checks, planning, workspace carve-up,
  argument checks of every entry point) compiled with the sanitizers on its host side only,
  linked with the library's other objects, then the ABI host tests with HTA_LIBRARY pointing
  at that build.  No GPU is touched: every call these tests make is refused or answered
  before a launch.

A canary (an out-of-bounds read built with the same flags) first shows that each runtime
really reports.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]
# hipcc: the sanitizers apply to the host side only (each flag behind -Xarch_host)
HIP_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HIP_SAN_LINK = ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                "-fsanitize=undefined"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _gcc_runtime() -> str:
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def _clang_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    return hits[-1]


def _env(preload: str, **extra) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1", **extra)
    return env


def _run(cmd, env, timeout=900):
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def _canary(compiler: list, runtime: str):
    """An out-of-bounds read built with the same flags must be reported."""
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(OUT, "canary.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\n"
                "int canary(int i) { int* p = malloc(4 * sizeof(int)); int v = p[i];"
                " free(p); return v; }\n")
    lib = os.path.join(OUT, f"libcanary_{os.path.basename(compiler[0])}.so")
    subprocess.check_call([*compiler, "-shared", "-fPIC", src, "-o", lib])
    r = _run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).canary(4)"],
             _env(runtime))
    # (ASan's heap-buffer-overflow, or UBSan's object-size check when it fires first)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr
                                  or "insufficient space" in r.stderr), r.stderr[-2000:]


def _pytest_child(files, env):
    r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p",
              "no:cacheprovider", *files], env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    for rep in REPORTS:
        assert rep not in out, out[-6000:]
    return out


def test_oracle_under_address_and_undefined_sanitizers():
    _canary(["gcc", *GCC_SAN], _gcc_runtime())
    lib = os.path.join(OUT, "libhta_oracle_san.so")
    subprocess.check_call(["gcc", *GCC_SAN, "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                           os.path.join(ROOT, "oracle", "hta_oracle.c"),
                           os.path.join(ROOT, "oracle", "step_oracle.c"), "-o", lib, "-lm"])
    env = _env(_gcc_runtime(), HTA_ORACLE_LIBRARY=lib)
    probe = _run([sys.executable, "-c", "import oracle; print(oracle.lib()._name)"], env)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    _pytest_child(["tests/test_oracle_pins.py", "tests/test_step_oracle_pins.py",
                   "tests/test_chunk_mass_pins.py", "tests/test_oracle_mutants.py"], env)


def test_host_abi_under_address_and_undefined_sanitizers():
    from tree_verification_attention_amd import build as hip_build

    _canary([hip_build.HIPCC, "-x", "c", *HIP_SAN, "-O1", "-g"], _clang_runtime())
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "tree_verification_attention_amd", "csrc")
    objs = []
    for src in sorted(glob.glob(os.path.join(csrc, "*.hip"))):
        name = os.path.basename(src)
        san = name == "hta_api.hip"
        prebuilt = os.path.join(hip_build.BUILD, name + ".o")
        if not san and os.path.exists(prebuilt) and \
                os.path.getmtime(prebuilt) >= os.path.getmtime(src):
            objs.append(prebuilt)  # device code and launch wrappers, as built
            continue
        obj = os.path.join(OUT, name + ".o")
        extra = [*HIP_SAN, "-g"] if san else []
        subprocess.check_call([hip_build.HIPCC, *hip_build.HIP_FLAGS, *extra, "-c", src,
                               "-o", obj], stderr=subprocess.DEVNULL)
        objs.append(obj)
    lib = os.path.join(OUT, "libhta_san.so")
    subprocess.check_call([hip_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                           *HIP_SAN_LINK, *objs, "-o", lib])
    env = _env(_clang_runtime(), HTA_LIBRARY=lib)
    probe = _run([sys.executable, "-c",
                  "import tree_verification_attention_amd as h; print(h.load()._name)"], env)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    _pytest_child(["tests/test_abi_host.py"], env)
