"""Compile the C oracle into oracle/liboracle.so.

Test infrastructure: the oracle is built with plain gcc, with contraction of
multiply-adds disabled and no fast-math, so that it keeps IEEE semantics.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


# Sanitized builds (tests only): UndefinedBehaviorSanitizer for the library
# loaded into the Python pins, AddressSanitizer + UndefinedBehaviorSanitizer
# for the standalone driver executable.
UBSAN_FLAGS = ("-fsanitize=undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-g")
ASAN_UBSAN_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-g")
DRIVER = os.path.join(HERE, "sanitize_driver.c")


def build_driver(out: str, extra_flags=ASAN_UBSAN_FLAGS) -> str:
    """Compile the oracle with sanitize_driver.c into the executable `out`."""
    flags = [f for f in CFLAGS if f not in ("-fPIC", "-shared")]
    cmd = ["gcc", *flags, *extra_flags, "-o", out, DRIVER, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile `src` into the shared library `out` and return its path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
