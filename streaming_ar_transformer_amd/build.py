"""Build the sdec HIP library in-tree: ``streaming_ar_transformer_amd/libsdec.so`` for gfx950.

Each source is compiled to an object of its own (in parallel), then the objects are linked."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsdec.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("kernels.hip", "rvq.hip", "conv.hip", "sdec.cpp")]
ARCH = os.environ.get("SDEC_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def compile_command(src: str, obj: str):
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-c",
            # packed fp32 instructions stay off: only scalar/float2 code is generated.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            "-x", "hip", src, "-o", obj]


def link_command(objs, out: str):
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
