"""CPU tests under AddressSanitizer and UndefinedBehaviorSanitizer.

Host code of the library (argument checks, tile capacities, the bucket planner) is built with ASan and
UBSan (device code untouched) and the ABI and planner tests run against that build in a child process
that preloads clang's ASan runtime; the oracle is built with gcc's ASan and UBSan and every pin runs
against it under gcc's runtime.  Any sanitizer report ends the child with a non-zero status.
"""
import os
import subprocess
import sys

import oracle
from sparse_moe_layer_03_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _instrumented(lib):
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    return "__asan_report" in syms and "__ubsan_handle" in syms


def test_host_code_under_asan_ubsan(tmp_path):
    lib = build.build(out=str(tmp_path / "libmoe355_san.so"), sanitize=True)
    assert _instrumented(lib)
    env = dict(os.environ, MOE355_LIB=lib, LD_PRELOAD=build.asan_runtime(), **ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_cpu.py", "tests/test_bucket_plan.py"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert " passed" in r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    assert _instrumented(lib)
    env = dict(os.environ, LD_PRELOAD=_gcc_asan(), **ENV)
    r = subprocess.run([sys.executable, "-m", "tests.run_pins", lib], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_planted_overflow_is_reported(tmp_path):
    """A copy of the oracle that reads one element past the router matrix must fail under ASan: the
    harness above would see such a mistake."""
    src = open(oracle._SRC).read()
    old = "float v = dot_bf16_f32(xt, w_router + (size_t)e * H, H);"
    assert src.count(old) == 1
    c = tmp_path / "overflow.c"
    c.write_text(src.replace(old, "float v = dot_bf16_f32(xt, w_router + (size_t)e * H, H + 1);"))
    lib = str(tmp_path / "liboverflow.so")
    cmd = [a for a in oracle.GCC_CMD if a not in (oracle._SRC, oracle.LIB_PATH, "-o", "-lm")]
    subprocess.run(cmd + oracle.SANITIZE_FLAGS + [str(c), "-o", lib, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=_gcc_asan(), **ENV)
    r = subprocess.run([sys.executable, "-m", "tests.run_pins", lib], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr
