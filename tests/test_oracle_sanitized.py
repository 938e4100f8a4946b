"""The CPU oracle under sanitizers (CPU only).

- AddressSanitizer + UndefinedBehaviorSanitizer: oracle/sanitize_driver.c
  runs every oracle entry point over small seeded cases with buffers of
  exactly the contracted size (empty and CSR bags, every storage type and
  code, strided operands, rejected arguments), compiled together with
  oracle.c into one instrumented executable.
- UndefinedBehaviorSanitizer: the oracle library built with it and loaded in
  a fresh Python process runs every pin of tests/oracle_pins.py.

Either run fails on the first error a sanitizer reports.
"""
import os
import subprocess
import sys

from oracle import build as oracle_build

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
PINS = ("pin_pair_map", "pin_emb_bag", "pin_emb_bag_ext", "pin_emb_bag_fp8", "pin_interact",
        "pin_linear", "pin_forward")


def _assert_clean(proc, what):
    text = proc.stdout + proc.stderr
    assert proc.returncode == 0, f"{what} exited with {proc.returncode}:\n{text[-4000:]}"
    for marker in ("runtime error", "AddressSanitizer", "LeakSanitizer"):
        assert marker not in text, f"{what}: sanitizer report\n{text[-4000:]}"


def test_oracle_entry_points_under_asan_and_ubsan(tmp_path):
    exe = oracle_build.build_driver(str(tmp_path / "oracle_sanitized"))
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    _assert_clean(proc, "sanitize_driver")
    assert "0 failed" in proc.stdout, proc.stdout


def test_oracle_pins_under_ubsan(tmp_path):
    lib = oracle_build.build(out=str(tmp_path / "liboracle_ubsan.so"),
                             extra_flags=oracle_build.UBSAN_FLAGS)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, oracle_pins\n"
            "lib = oracle.load(%r)\n"
            "for name in %r:\n"
            "    getattr(oracle_pins, name)(lib)\n"
            "print('pins ok')\n") % (ROOT, TESTS, lib, PINS)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600, cwd=ROOT)
    _assert_clean(proc, "pins under UBSan")
    assert "pins ok" in proc.stdout
