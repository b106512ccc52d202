"""Build libpagedattn.so for gfx950 with hipcc, in-tree (next to this file).

    python -m paged_kv_varlen_flash_amd.build
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedattn.so")
SOURCES = ["pagedattn.hip", "plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))


def build(verbose: bool = False, out: str = LIB, host_flags=()) -> str:
    """Compile every source into libpagedattn.so (at `out`); returns its path.
    host_flags: extra flags for the host half of every source only (each is
    passed after -Xarch_host, so the device code is unchanged)."""
    objdir = os.path.join(HERE, "_build") if out == LIB else os.path.dirname(out)
    os.makedirs(objdir, exist_ok=True)
    xhost = [f for flag in host_flags for f in ("-Xarch_host", flag)]
    common = xhost + [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              # packed fp32 VALU ops stay off: hipcc would otherwise form them
              # from plain float code (the host pass warns it does not know the
              # feature; that warning is harmless)
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        _run([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + common, verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + xhost + objs,
         verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
