"""Ahead-of-time build of the HIP library ``libmi355attn.so`` for gfx950.

Run ``python -m exact_attention_46_amd.build`` (or ``__graft_entry__.build()``).
The library is built in-tree, next to this file, so it travels with the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmi355attn.so")
SOURCES = ["abi.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"]
# Extra flags per source. The kernels never see a signalling NaN (their
# inputs to max() come from MFMA and FMA results), so the compiler need not
# quiet operands before each max; argument checking in abi.hip keeps full NaN
# semantics (it tests the scale with isfinite).
SOURCE_FLAGS = {
    "attn_fwd.hip": ["-fno-honor-nans"],
    "attn_decode.hip": ["-fno-honor-nans"],
}
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags():
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # Packed fp32 VALU instructions stay off: the compiler would otherwise
        # form them from plain float code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if out.strip() and verbose:
        print(out)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compiles every source (one object each) and links the shared library
    (always recompiles)."""
    tag = ".tmp%d" % os.getpid()
    objs = []
    try:
        for src in SOURCES:
            obj = os.path.join(HERE, src + tag + ".o")
            objs.append(obj)
            cmd = [hipcc()] + flags() + SOURCE_FLAGS.get(src, []) + [
                "-c", os.path.join(CSRC, src), "-o", obj]
            rc, out = _run(cmd, verbose)
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
        tmp = LIB + tag
        rc, out = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp],
                       verbose)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("link failed:\n" + out)
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
