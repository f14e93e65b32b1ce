"""Host sanitizers on the CPU: AddressSanitizer and UndefinedBehaviorSanitizer over

* the oracle's C code (gcc build of oracle/starkv_oracle.c), under the oracle pin tests;
* the host code of the C ABI layer (api.cpp: argument validation, split planning, workspace
  layout), under the ABI validation tests, which reject or answer every call before anything is
  enqueued (no GPU is used).

Each runs in a subprocess with the sanitizer runtime preloaded and the library chosen through
STARKV_ORACLE_LIB / STARKV_LIBRARY; the subprocess first proves that the sanitized library is
the one mapped into it. Any sanitizer report fails the test (halt on the first error)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "sanitize")
OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _env(extra):
    env = dict(os.environ)
    env.update(OPTS)
    env.update(extra)
    return env


def _check_loaded(env, module, path):
    code = (f"import {module} as m; m.lib(); "
            f"assert {path!r} in open('/proc/self/maps').read(), 'sanitized library not mapped'")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]


def _run_tests(env, tests):
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:"):
        assert marker not in out, out[-4000:]
    return out


def _symbols(path):
    return subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout


def test_oracle_under_asan_and_ubsan():
    import oracle
    os.makedirs(SAN, exist_ok=True)
    lib = oracle.build_sanitized(os.path.join(SAN, "liboracle_asan.so"))
    assert "__asan_report" in _symbols(lib) and "__ubsan_handle" in _symbols(lib)
    pre = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                          check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in pre):
        pytest.skip("gcc sanitizer runtimes not found")
    env = _env({"LD_PRELOAD": " ".join(pre), "STARKV_ORACLE_LIB": lib})
    _check_loaded(env, "oracle", lib)
    out = _run_tests(env, ["tests/test_oracle_pins.py"])
    assert " passed" in out


def test_abi_layer_under_asan_and_ubsan():
    from rank_kv_cache_amd import build
    runtime = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtime:
        pytest.skip("clang AddressSanitizer runtime not found")
    os.makedirs(SAN, exist_ok=True)
    try:
        lib = build.build_host_sanitized(os.path.join(SAN, "libstarkv_asan.so"))
    except FileNotFoundError as e:
        pytest.skip(f"kernel objects of the regular build are missing: {e}")
    syms = _symbols(lib)
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = _env({"LD_PRELOAD": runtime[-1], "STARKV_LIBRARY": lib})
    _check_loaded(env, "rank_kv_cache_amd", lib)
    out = _run_tests(env, ["tests/test_abi.py"])
    assert " passed" in out
