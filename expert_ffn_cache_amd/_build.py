"""Builds expert_ffn_cache_amd/libmoecache.so from csrc/*.hip with hipcc for gfx950."""
import glob
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_BUILD = os.path.join(_ROOT, "_build", "moecache")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(_ROOT, "include"), "-I", os.path.join(_HERE, "csrc"),
]


def lib_path():
    return os.path.join(_HERE, "libmoecache.so")


def sources():
    return sorted(glob.glob(os.path.join(_HERE, "csrc", "*.hip")))


def build(verbose=False):
    os.makedirs(_BUILD, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(_BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the gfx950 feature flag; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if text.strip():
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    out = lib_path()
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out
