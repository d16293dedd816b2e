"""Compile the CPU oracle (plain C) into oracle/liboracle.so.

Test infrastructure only: the library never links or loads the oracle.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
# NEOX_ORACLE_SO points the tests at another build of the same source (e.g. one with
# host sanitizers); build_oracle(force=False) then uses it as it is.
SO = os.environ.get("NEOX_ORACLE_SO", os.path.join(HERE, "liboracle.so"))

# No fast-math and no FP contraction: every arithmetic line of the oracle is one IEEE
# operation in the precision it names.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build_oracle(force: bool = True) -> str:
    if not force and os.path.exists(SO):
        return SO
    src = os.path.join(HERE, "oracle.c")
    tmp = SO + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build_oracle())
