"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The library's host layer (api.cpp, variants.cpp) linked with the stand-in
  launchers of tests/host_model: every entry point's validation, and every
  schedule the GPU tests use replayed against the buffers each call was
  given -- the split plan built by the device's own plan code on 64 emulated
  lanes into an uninitialised workspace, each workgroup's segment walk, and
  every query row, cache row, partial and output address a kernel forms.
  The driver first checks that the model catches planted mistakes.
* The fp64 oracle, with every pin of tests/oracle_pins.py run against it.

Both are compiled with g++/gcc for the host only (no GPU code is built here).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODEL = os.path.join(ROOT, "tests", "host_model")
CSRC = os.path.join(ROOT, "head_latent_attention_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip("%s not available" % tool)


def _libasan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("libasan not available")
    return path


def test_host_layer_under_sanitizers(tmp_path):
    _need("g++")
    exe = str(tmp_path / "host_model")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "variants.cpp")] + [
        os.path.join(MODEL, f) for f in ("model.cpp", "lanes.cpp", "driver.cpp")]
    cmd = ["g++", "-std=c++20", "-O1", "-g", *SAN, "-I" + os.path.join(MODEL, "hip_shim"), "-I" + CSRC,
           "-I" + os.path.join(ROOT, "include"), *srcs, "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.count("self-check caught") == 4, r.stdout
    assert " 0 failures" in r.stdout, r.stdout


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    asan = _libasan()
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", *SAN, os.path.join(ROOT, "oracle", "mla_oracle.c"), "-o", lib, "-lm"],
                   check=True, capture_output=True, text=True)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, oracle_pins\n"
            "o = oracle.Oracle(%r)\n"
            "for pin in oracle_pins.ALL_PINS: pin(o)\n"
            "print('pins', len(oracle_pins.ALL_PINS))\n") % (ROOT, os.path.join(ROOT, "tests"), lib)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", LD_PRELOAD=asan, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle_pins
    assert "pins %d" % len(oracle_pins.ALL_PINS) in r.stdout, r.stdout
