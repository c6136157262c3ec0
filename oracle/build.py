"""Build the CPU oracle into oracle/liboracle.so with gcc.

Test infrastructure only: the tests, the smoke check and the CPU-baseline leg
of the benchmark load the result; the HIP product path never does.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

# IEEE single precision with no contraction of a*b+c into fma and no
# reassociation: every rounding is the one the source spells out.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(sanitize: bool = False, out: str = None) -> str:
    out = out or (os.path.join(HERE, "liboracle_san.so") if sanitize else LIB)
    cmd = ["gcc", *CFLAGS]
    if sanitize:
        cmd += ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    cmd += [os.path.join(HERE, "qsa_oracle.c"), "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv))
