"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np


def rel_fro(got, want) -> float:
    """Relative Frobenius error ||got - want|| / ||want|| in float64."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    den = np.linalg.norm(w.ravel())
    num = np.linalg.norm((g - w).ravel())
    return float(num / den) if den > 0 else float(num)


def dev(x, dtype):
    """numpy float32 (storage-exact) -> device tensor of `dtype`."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


# Tolerances (relative Frobenius over the whole output tensor):
#  fp32 inputs, fp32 arithmetic                          -> 1e-5
#  bf16 inputs with fp32 outputs of the feature map      -> 1e-5: bf16 x bf16 products
#      are exact in fp32 and only the fp32 accumulation order differs
#  bf16 feature map stored as bf16                        -> 5e-3: one rounding to 8
#      significant bits (unit roundoff 2^-8) on top of the fp32 result
#  bf16 attention paths (phi, A and S rounded to bf16 as MFMA operands) -> 2e-2
#  feature-map backward (bf16 X, Theta)                   -> 5e-3: Y and s are exact
#      products summed in fp32; dY is rounded once to bf16 (unit roundoff 2^-9)
#      before the two fp32-accumulated products, so each output is a sum of
#      terms with one independent relative error of at most 2^-9 each
TOL_F32 = 1e-5
TOL_FEAT_BF16_IN = 1e-5
TOL_FEAT_BF16_OUT = 5e-3
TOL_BF16 = 2e-2
TOL_BWD_BF16 = 5e-3
