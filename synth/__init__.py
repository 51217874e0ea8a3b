"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers; it holds none of the MLP's
arithmetic, and it imports neither the oracle nor the HIP package.

Recipe (the pages state no value distributions; these keep G and U at unit
variance): for a workload with seed s, a CPU ``torch.Generator`` seeded with s
draws, in this fixed order, X[T,D], Wg[D,H], Wu[D,H], Wd[H,D], dY[T,D] as
float32 standard normals, each scaled by its standard deviation
(1, 1/sqrt(D), 1/sqrt(D), 1/sqrt(H), 1) and then cast (round to nearest even)
to the storage dtype. In fp32 mode the float32 values are kept.

The workload shapes are the pages' own ("[RFC] Full-pipeline SwiGLU MLP ...",
section "Validation environment": training B=8, S up to 8192 at
(D,H) in {(1024,2816), (2048,5632), (4096,11008)}; inference B=1, S from 1
to 256).
"""

import math

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}

# name: (D, H, B, S, seed)
WORKLOADS = {
    "mlp_1024x2816_T128": (1024, 2816, 1, 128, 1000),
    "mlp_1024x2816_T16384": (1024, 2816, 8, 2048, 1001),
    "mlp_2048x5632_T32768": (2048, 5632, 8, 4096, 1002),
    "mlp_4096x11008_T65536": (4096, 11008, 8, 8192, 1003),
    "mlp_2048x5632_T4096_fp32": (2048, 5632, 8, 512, 1002),
}

INFER_S = (1, 2, 4, 8, 16, 32, 64, 128, 256)
INFER_DH = ((1024, 2816), (4096, 11008))


def make_inputs(T, D, H, seed, dtype="bf16", with_dy=True):
    """Draw X, Wg, Wu, Wd (and dY) on the CPU; returns a dict of CPU tensors."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    tdt = DTYPES[dtype]
    out = {}
    spec = [("X", (T, D), 1.0), ("Wg", (D, H), 1.0 / math.sqrt(D)),
            ("Wu", (D, H), 1.0 / math.sqrt(D)), ("Wd", (H, D), 1.0 / math.sqrt(H))]
    if with_dy:
        spec.append(("dY", (T, D), 1.0))
    for name, shape, std in spec:
        v = torch.randn(shape, generator=gen, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        out[name] = v.to(tdt) if tdt != torch.float32 else v
    return out


def workload_inputs(name, dtype="bf16", with_dy=True):
    D, H, B, S, seed = WORKLOADS[name]
    return make_inputs(B * S, D, H, seed, dtype=dtype, with_dy=with_dy)
