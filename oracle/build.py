"""Builds the fp64 CPU oracle (test infrastructure) with gcc.

``build()`` compiles ``fa_oracle.c`` into ``oracle/libfa_oracle.so``; ``build_mutant(n, dir)``
compiles the same source with ``-DORACLE_MUTANT=n`` (one planted mistake) for the tests
that check that the pins catch mistakes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fa_oracle.c")
LIB = os.path.join(HERE, "libfa_oracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def _compile(out, defines=()):
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build():
    return _compile(LIB)


def build_mutant(n, out_dir):
    return _compile(os.path.join(out_dir, f"libfa_oracle_m{n}.so"), [f"ORACLE_MUTANT={n}"])


if __name__ == "__main__":
    print(build())
