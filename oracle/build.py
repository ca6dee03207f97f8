"""Compile the C++ oracle (oracle/clsa_oracle.cpp) into oracle/libclsa_oracle.so.

Test infrastructure: the library is loaded only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  Plain g++, IEEE fp64 (no fast-math).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "clsa_oracle.cpp")
LIB = os.path.join(HERE, "libclsa_oracle.so")


def build() -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", "-o", LIB + ".tmp", SRC]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
