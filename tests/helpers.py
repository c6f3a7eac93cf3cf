"""Small helpers shared by the GPU parity tests."""
import sys

import numpy as np
import torch

# Tolerances on relative L2 error (the whole tensor, fp64): fp32 inputs, bf16 inputs.
TOL_F32 = 1e-5
TOL_BF16 = 2e-3


def rel_l2(x, ref) -> float:
    x = x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    ref = ref.detach().double().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def tol_for(dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def dev(d, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def say(*a):
    """Print and flush before a GPU step, so a failing case is named even if the run dies."""
    print(*a, flush=True)
    sys.stdout.flush()
