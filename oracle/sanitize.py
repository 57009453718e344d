"""Run the oracle's CPU pins (tests/test_oracle_pins.py) against an
AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle.

    python oracle/sanitize.py

The same C source is compiled with -fsanitize=address,undefined (host code
only, gcc), the ASan runtime is preloaded into a fresh Python, and the pins
run with that library selected through ORACLE_LIB. Any sanitizer report
aborts the run (halt_on_error), so a zero exit status means a clean run.
Leak detection is off: the Python interpreter itself is not leak-clean.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "adacluster_oracle.c")
LIB = os.path.join(HERE, "liboracle_adacluster_asan.so")


def main() -> int:
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-o", LIB, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(ORACLE_LIB=LIB, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=ROOT)
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
