"""Builds the oracle's C code into oracle/libkvc_oracle.so (test infrastructure only)."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "kvc_oracle.c")
    out = os.path.join(_HERE, "libkvc_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
