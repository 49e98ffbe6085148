"""Build the scalar C reference encoder (oracle/libencref.so) with gcc.

Test infrastructure: building the checker is not using it.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    src = os.path.join(_HERE, "encode_ref.c")
    out = os.path.join(_HERE, "libencref.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
           src, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
