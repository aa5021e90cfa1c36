"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each run over the tests that exercise it in a child process
with the sanitizer runtime preloaded (Python itself is not instrumented):
  - the C oracle built with gcc -fsanitize=address,undefined, running the
    oracle's pins (tests/test_oracle_pins.py);
  - libbqd.so with the sanitizers on its host code only (-Xarch_host: the
    gfx950 device code is built as usual), running the host tests of the C
    ABI (tests/test_abi_host.py): argument validation, the descriptor
    encoder of the persistent pass, the INT8-X host encoder and the int4
    pack helpers.
Leak checking is off (the interpreter keeps allocations to the end).  Any
sanitizer report ends the child with a non-zero status."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(compiler, name):
    try:
        path = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_tests(test_file, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def _instrumented(lib):
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    return "__asan_init" in syms or "__asan_version_mismatch_check" in syms


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    rt = _runtime("gcc", "libasan.so")
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                              "-fno-omit-frame-pointer", "-g"], out=str(tmp_path / "liboracle_san.so"))
    assert _instrumented(lib)
    out = _run_tests("test_oracle_pins.py", {"BQD_ORACLE_LIB": lib}, rt)
    assert " passed" in out


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from bit_quantized_decode_quantize_amd.csrc import build as lib_build
    rt = _runtime(os.path.join(os.path.dirname(os.path.realpath(lib_build.HIPCC)), "..", "llvm", "bin", "clang"),
                  "libclang_rt.asan-x86_64.so") or _runtime("/opt/rocm/llvm/bin/clang", "libclang_rt.asan-x86_64.so")
    if rt is None or not os.path.exists(lib_build.HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    host = []
    for flag in ("-g", "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", flag]
    lib = lib_build.build(host, out=str(tmp_path / "libbqd_san.so"))
    assert _instrumented(lib)
    out = _run_tests("test_abi_host.py", {"BQD_LIB": lib}, rt)
    assert " passed" in out
