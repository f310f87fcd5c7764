"""Build the CPU oracle (TEST INFRASTRUCTURE ONLY) into oracle/liboracle.so.

Plain gcc, -O2, no fast-math, no floating-point contraction: every add and
multiply of the oracle rounds on its own, in the order the C source states.
OpenMP runs its per-sample loops on host threads (same bits for any count).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cfc_oracle.c")
BODY = os.path.join(HERE, "cfc_oracle_body.h")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so; with force=False, skip when it is newer than its sources."""
    if not force and os.path.exists(LIB):
        newest_src = max(os.path.getmtime(SRC), os.path.getmtime(BODY))
        if os.path.getmtime(LIB) >= newest_src:
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
