"""Build the gfx950 C-ABI library ``libttt_amd.so`` in-tree with hipcc.

The library holds the HIP kernels (csrc/*.hip) and the host entry points of
include/ttt.h (csrc/ttt_api.cpp).  It is always built for gfx950 only.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libttt_amd.so")
SOURCES = ["ttt_api.cpp", "ttt_validate.cpp", "ttt_linear.hip", "ttt_mlp.hip", "ttt_decode.hip", "ttt_decode_compact.hip", "ttt_backward.hip",
           "ttt_mlp_decode.hip",
           "ttt_mlp_decode_compact.hip", "ttt_mlp_backward.hip", "ttt_input.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are disabled on purpose: the kernels are
# written for unpacked fp32 arithmetic.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + lang + [
        "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        sys.stderr.write(msg + "\n")


def build() -> str:
    """Compile every source and link libttt_amd.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp]
                          + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
