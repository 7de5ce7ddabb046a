"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer).

- The oracle (plain C) is compiled with both sanitizers and all of its pins
  run against that build in a child process (the sanitizer runtime must be
  loaded first, so the child gets it through LD_PRELOAD).  A copy of the
  oracle with a planted out-of-bounds read must be stopped by the sanitizer,
  which shows the instrumentation is live.
- The C ABI's host code (argument validation, workspace sizing, error
  messages) is compiled with both sanitizers on the host side only and
  driven by ``abi_host_harness.cpp`` through every rejection path, with the
  int extremes as sizes.  Nothing in either run touches a GPU.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN_C = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-g"]


def _libasan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _run_pins(lib: str, timeout=900):
    env = dict(os.environ, LD_PRELOAD=_libasan(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "import oracle, oracle_pins\n"
            f"orc = oracle.Oracle({lib!r})\n"
            "for pin in oracle_pins.ALL_PINS:\n"
            "    pin(orc)\n"
            "print('PINS_OK', flush=True)\n")
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libtw_oracle_san.so")
    oracle.build(out=lib, extra=SAN_C)
    r = _run_pins(lib)
    assert r.returncode == 0 and "PINS_OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """The same build with the dot product reading one element past each
    row: the read past the last weight row leaves its allocation, and the
    sanitizer must stop the run (on the CPU)."""
    src = open(oracle.SOURCE).read()
    old = "for (int k = 0; k < K; ++k)\n        s += a[k] * b[k];"
    assert old in src
    bad = tmp_path / "tw_oracle_oob.c"
    bad.write_text(src.replace(old, "for (int k = 0; k <= K; ++k)\n        s += a[k] * b[k];"))
    lib = str(tmp_path / "libtw_oracle_oob.so")
    oracle.build(src=str(bad), out=lib, extra=SAN_C)
    r = _run_pins(lib)
    assert r.returncode != 0 and "PINS_OK" not in r.stdout
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def test_abi_host_validation_under_asan_ubsan(tmp_path):
    from activation_sparse_feed_gate_amd import build as b

    kernels = [os.path.join(b.BUILD_DIR, s + ".o") for s in b.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernels):
        b.build()
    # the sanitizers apply to host code only (-Xarch_host before each flag);
    # the kernel objects are the library's own, unchanged
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    flags = [x for x in b.FLAGS if x != "-fPIC"] + ["-g"]
    objs = []
    for src in (os.path.join(b.CSRC, "tw_api.cpp"), os.path.join(TESTS, "abi_host_harness.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([b.HIPCC, *flags, *san, "-x", "hip", "-c", src, "-o", obj], check=True,
                       capture_output=True)
        objs.append(obj)
    exe = str(tmp_path / "abi_host_harness")
    subprocess.run([b.HIPCC, "--offload-arch=gfx950", *san, *objs, *kernels, "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "HARNESS_OK" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr, r.stderr[-3000:]
