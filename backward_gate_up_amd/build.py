"""Build the HIP library in-tree: backward_gate_up_amd/libswiglu_mlp.so (gfx950)."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "swiglu_mlp.hip")
OUT = os.path.join(HERE, "libswiglu_mlp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # no packed-fp32 VALU instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    """Compile the library (always; takes ~15 s). Raises on failure."""
    tmp = OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
