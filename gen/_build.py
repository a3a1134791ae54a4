"""Builds gen/libmoegen.so from gen/gen.c with the host C compiler."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_HERE, "libmoegen.so")


def build():
    src = os.path.join(_HERE, "gen.c")
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out
