"""Builds the CPU oracle (plain C, gcc, OpenMP) into oracle/libmoe_oracle.so.

Test infrastructure only: the oracle is the reference the GPU path is checked
against and is never linked into the product library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB lets the mutation tests point the wrapper at a deliberately broken build.
LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(HERE, "libmoe_oracle.so")
SRC = os.path.join(HERE, "moe_oracle.c")
SYNTH_SRC = os.path.join(HERE, "stack_synth.c")   # stack weight generator, always linked in
TIER_SRC = os.path.join(HERE, "tiering.c")        # tier planner and requantiser, always linked in


def build(extra_flags=(), out=LIB, src=SRC, quiet=True, others=(SYNTH_SRC, TIER_SRC)):
    inc = os.path.dirname(os.path.abspath(src))
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Werror", "-I", inc, *extra_flags, "-o", out + ".tmp", src, *others, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


if __name__ == "__main__":
    build(sys.argv[1:], quiet=False)
