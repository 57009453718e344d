"""The oracle's CPU pins under AddressSanitizer and UndefinedBehaviorSanitizer
(oracle/sanitize.py builds the sanitized library and runs the pins in a fresh
interpreter with the ASan runtime preloaded; any report fails the run)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_clean_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "oracle", "sanitize.py")],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
