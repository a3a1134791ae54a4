"""Builds oracle/liboracle.so (test infrastructure) with the host C compiler, -O2, no fast-math."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_HERE, "liboracle.so")


def build():
    src = os.path.join(_HERE, "moe_oracle.c")
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out
