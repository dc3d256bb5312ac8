"""Build the fp64 attention oracle (forward and gradient; test infrastructure)
with the host C compiler.

The oracle is plain C compiled without -ffast-math so that every operation is
an IEEE fp64 operation in the order the source states.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "attn_oracle.c"), os.path.join(HERE, "attn_oracle_bwd.c")]
LIB = os.path.join(HERE, "liboracle_attn.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           *SRCS, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
