"""Build the CPU oracle (test infrastructure) with gcc.

``build()`` writes ``liboracle.so`` next to this file; ``build_mutant(n, dir)``
writes a variant carrying planted mistake ``n`` (see ORACLE_MUTANT in
moe_oracle.c), used only to show that the oracle's pins detect it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def _gcc(out, extra=()):
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *FLAGS, *extra, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force=True):
    if force or not os.path.exists(LIB):
        _gcc(LIB)
    return LIB


def build_mutant(n, out_dir):
    return _gcc(os.path.join(out_dir, "liboracle_mutant%d.so" % n), ["-DORACLE_MUTANT=%d" % n])


if __name__ == "__main__":
    print(build())
