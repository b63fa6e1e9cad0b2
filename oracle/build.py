"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is compiled as plain C11 with no fast-math and no FMA contraction,
so its arithmetic is the literal fp64 evaluation of the source.
"""
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "dcn_oracle.c"
LIB = HERE / "libdcn_oracle.so"


def build(verbose: bool = False) -> pathlib.Path:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", str(LIB), str(SRC), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
