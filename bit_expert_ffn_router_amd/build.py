"""Build the HIP libraries in-tree for gfx950.

    python bit_expert_ffn_router_amd/build.py

(Run it by path: importing the package loads the library it builds.)

Produces bit_expert_ffn_router_amd/libmoe.so (the layer) and
synth/libmoe_synth.so (the device side of the seeded input generator).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

LIBS = {
    os.path.join(HERE, "libmoe.so"): [
        os.path.join(HERE, "csrc", f) for f in
        ("api.hip", "pack.hip", "route.hip", "router.hip", "decode.hip", "prefill.hip", "slots.hip",
         "host_ffn.hip", "noalloc.hip")
    ],
    os.path.join(ROOT, "synth", "libmoe_synth.so"): [
        os.path.join(ROOT, "synth", "csrc", "synth_fill.hip"),
    ],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> None:
    for out, srcs in LIBS.items():
        tmp = out + ".tmp"
        cmd = [hipcc()] + HIPCC_FLAGS + srcs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed for %s" % out)
        os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose=True)
