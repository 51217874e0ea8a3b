"""Build the HIP library in-tree: backward_gate_up_amd/libswiglu_mlp.so (gfx950).

The kernels are instantiated in eighteen translation units (csrc/instantiate.hip
compiled once per dtype, entry point and weight layout) plus the C ABI
(csrc/swiglu_mlp.hip);
they compile in parallel and are linked into one shared library.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libswiglu_mlp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]

# (object name, source, defines)
UNITS = [("abi", "swiglu_mlp.hip", [])] + [
    (f"{dt}_{op}_{lay}", "instantiate.hip",
     [f"-DSWIGLU_INST_DTYPE={i}", f"-DSWIGLU_INST_OP={j}", f"-DSWIGLU_INST_LIN={k}"])
    for i, dt in enumerate(("bf16", "fp16", "fp32")) for j, op in enumerate(("fwd", "bwd", "infer"))
    for k, lay in enumerate(("kernel", "linear"))
]


def _filter(text):
    return [ln for ln in text.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln]


def build(verbose=False, jobs=None):
    """Compile every unit and link the library (always). Raises on failure."""
    jobs = jobs or max(1, min(len(UNITS), len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="swiglu_build_") as tmpdir:
        def compile_unit(u):
            name, src, defs = u
            obj = os.path.join(tmpdir, name + ".o")
            cmd = [HIPCC] + FLAGS + defs + ["-c", "-o", obj, os.path.join(CSRC, src)]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return name, cmd, r, obj

        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_unit, UNITS))
        objs = []
        for name, cmd, r, obj in results:
            msgs = _filter(r.stdout + r.stderr)
            if verbose:
                print(" ".join(cmd), flush=True)
                if msgs:
                    print("\n".join(msgs))
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {name}:\n" + "\n".join(msgs))
            objs.append(obj)
        tmp = OUT + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_filter(r.stdout + r.stderr)))
        os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
