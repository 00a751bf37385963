"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The fp64 oracle, built by gcc with -fsanitize=address,undefined, runs its
  pin suite (tests/test_oracle_pins.py).
* The library's host side (kvd_api.hip: argument checks, status strings, the
  paths that return before any launch), compiled with host-only sanitizers
  and linked with the regular kernel objects, runs the ABI host tests
  (tests/test_abi_host.py).

Each runs in a subprocess that preloads its compiler's sanitizer runtime; any
report aborts that process.  A copy of the oracle with one read planted past
the end of a row checks that the harness does catch such a read.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def gcc_oracle(src, out):
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"],
                   check=True)
    return out


def gcc_asan_runtime():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def run_sanitized(args, preload, extra_env, cwd):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    return subprocess.run([sys.executable, *args], env=env, cwd=cwd, capture_output=True,
                          text=True, timeout=900)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = gcc_oracle(ORACLE_SRC, str(tmp_path / "liboracle_san.so"))
    r = run_sanitized(["-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                       os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                      gcc_asan_runtime(), {"KVD_ORACLE_LIB": lib}, str(tmp_path))
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_a_planted_read_past_the_row_is_caught(tmp_path):
    """The rank count of a copy of the oracle reads one score past its row."""
    src = open(ORACLE_SRC).read()
    loop = "      for (i64 m = 0; m < nb; ++m)\n        if (s[m] > s[n] || (s[m] == s[n] && m < n)) ++rank;"
    assert src.count(loop) == 1
    bad = tmp_path / "oracle_bad.c"
    bad.write_text(src.replace(loop, loop.replace("m < nb; ++m", "m <= nb; ++m")))
    lib = gcc_oracle(str(bad), str(tmp_path / "liboracle_bad.so"))
    code = ("import numpy as np, oracle\n"
            "gs = np.arange(64, dtype=np.float64).reshape(1, 1, 64)\n"
            "oracle.topk(gs, np.array([1024], np.int32), 16, 8)\n")
    r = run_sanitized(["-c", code], gcc_asan_runtime(),
                      {"KVD_ORACLE_LIB": lib, "PYTHONPATH": ROOT}, str(tmp_path))
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-3000:]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not installed")
def test_host_api_under_asan_and_ubsan(tmp_path):
    from kv_cache_decode_amd import build as b
    runtime = _clang_asan_runtime()
    assert runtime, "clang's AddressSanitizer runtime not found under /opt/rocm/lib/llvm"
    objs = [os.path.join(b.BUILD_DIR, os.path.splitext(s)[0] + ".o")
            for s in b.SOURCES if s != "kvd_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    api = str(tmp_path / "kvd_api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    subprocess.run([b.hipcc(), *b.COMMON, "-O1", *host_san, "-c",
                    os.path.join(b.CSRC, "kvd_api.hip"), "-o", api], check=True,
                   capture_output=True)
    lib = str(tmp_path / "libkvdecode_san.so")
    subprocess.run([b.hipcc(), "-shared", "-fPIC", f"--offload-arch={b.ARCH}",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-shared-libsan", "-o", lib, *objs, api], check=True, capture_output=True)
    r = run_sanitized(["-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                       os.path.join(ROOT, "tests", "test_abi_host.py")],
                      runtime, {"KVD_LIBRARY_PATH": lib}, str(tmp_path))
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
