"""Build the CPU oracle: gcc -> oracle/libpa_oracle.so.

TEST INFRASTRUCTURE ONLY (see pa_oracle.c).  Plain gcc, no HIP."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "libpa_oracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile ``src`` (default oracle/pa_oracle.c) into the shared library ``out``."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
