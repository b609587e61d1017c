"""Build the C++ oracle (moe_oracle.cpp) into oracle/libmoe_oracle.so with g++.

    python -m oracle.build

Test infrastructure: the oracle is a plain float64 CPU definition of the layer; g++ with OpenMP,
no GPU headers.  Products are not contracted into fused multiply-adds, so each product is
rounded before it is added, as written.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
LIB = os.path.join(HERE, "libmoe_oracle.so")
CMD = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
       "-o", LIB + ".tmp", SRC]


def build(verbose: bool = True) -> str:
    r = subprocess.run(CMD, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on {SRC}:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
