"""The oracle's pins, run again against an AddressSanitizer + UndefinedBehaviorSanitizer build.

The oracle is plain C that indexes flat arrays by hand (grouped, padded transposes, gathered
rows, windows of larger matrices); an out-of-bounds read there would silently feed a wrong value
to every parity test that trusts it. This test builds the same source with ASan and UBSan (no
recovery: the first finding aborts), loads it in a fresh interpreter whose LD_PRELOAD puts the ASan
runtime first, and runs the oracle pin and ablation suites through it. A second case hands the
checking build a buffer one byte short and requires the sanitizer to stop the process, so a build
in which the sanitizers were not active cannot pass.
"""
import os
import subprocess
import sys

import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path_factory.mktemp("orc_san") / "libpmn_oracle_san.so")
    O.build(out=lib, sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{asan}:{ubsan}", PMN_ORACLE_LIB=lib, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    return env


def test_oracle_pins_and_ablations_clean_under_asan_ubsan(sanitized):
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(HERE, "test_oracle_pins.py"), os.path.join(HERE, "test_ablations.py")]
    p = subprocess.run(cmd, cwd=ROOT, env=sanitized, capture_output=True, text=True, timeout=900)
    out = p.stdout + p.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in p.stdout


def test_sanitizer_build_catches_a_short_buffer(sanitized):
    """A planted mistake on the CPU: the codes buffer of a 1 x 32 quantization is one byte short."""
    prog = (
        "import ctypes as C, numpy as np, oracle as O\n"
        "L = O.lib()\n"
        "x = np.ones(32, np.uint16) * 0x3F80\n"
        "codes = np.zeros(15, np.uint8); scales = np.zeros(2, np.uint8); outer = np.zeros(1, np.float32)\n"
        "p = lambda a: a.ctypes.data_as(C.c_void_p)\n"
        "L.orc_nvfp4_quantize(p(x), 1, 32, 1, 1, None, p(codes), p(scales), p(outer), None)\n"
        "print('NOT CAUGHT')\n")
    p = subprocess.run([sys.executable, "-c", prog], cwd=ROOT, env=sanitized, capture_output=True, text=True,
                       timeout=300)
    assert "NOT CAUGHT" not in p.stdout
    assert p.returncode == 86 and "heap-buffer-overflow" in p.stderr, p.stderr[-2000:]
