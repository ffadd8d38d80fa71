"""Builds the C part of the oracle (test infrastructure only): liboracle_copy.so."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(_HERE, "copy_ref.c")
    out = os.path.join(_HERE, "liboracle_copy.so")
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", src, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
