"""Compile the C oracle (``ssm_oracle.c``) into ``libssm_oracle.so`` with gcc.

Test infrastructure only (see ``oracle/__init__.py``).  The flags keep the
arithmetic the plain definition: no -ffast-math, no floating-point
contraction into fused multiply-adds.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "libssm_oracle.so")


def build(verbose: bool = False, out: str = LIB, src: str = SRC) -> str:
    """Build the oracle library from ``src`` (another source only in the mutation tests)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math",
        "-o", out + ".tmp", src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
