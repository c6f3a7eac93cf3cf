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


def _np64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().cpu()
    return np.asarray(x)


def stream_errors(x, ref, stream_dims: int):
    """Relative L2 error of each stream of `x` against `ref` (the leading `stream_dims` axes index
    the streams: (batch, head), (sequence, head), ...), computed one stream at a time in fp64.
    Returns (whole-tensor rel-L2, worst stream rel-L2, index of the worst stream, max |x - ref|)."""
    x, ref = _np64(x), _np64(ref)
    shape = tuple(ref.shape[:stream_dims])
    num = den = 0.0
    worst, worst_at, max_abs = -1.0, None, 0.0
    for idx in np.ndindex(*shape):
        a = x[idx]
        a = a.double().numpy() if isinstance(a, torch.Tensor) else np.asarray(a, np.float64)
        r = ref[idx]
        r = r.double().numpy() if isinstance(r, torch.Tensor) else np.asarray(r, np.float64)
        d2 = float(np.sum((a - r) ** 2))
        r2 = float(np.sum(r * r))
        num += d2
        den += r2
        e = (d2 / r2) ** 0.5 if r2 > 0 else d2 ** 0.5
        if e > worst:
            worst, worst_at = e, idx
        if a.size:
            max_abs = max(max_abs, float(np.max(np.abs(a - r))))
    whole = (num / den) ** 0.5 if den > 0 else num ** 0.5
    return whole, worst, worst_at, max_abs


def check_streams(name, x, ref, stream_dims: int, tol_whole: float, tol_stream: float):
    """Print and assert the whole-tensor and worst-stream relative L2 errors of x against ref."""
    whole, worst, at, max_abs = stream_errors(x, ref, stream_dims)
    print(f"{name}: rel-L2 whole {whole:.3e}, worst stream {worst:.3e} at {at}, max-abs {max_abs:.3e}", flush=True)
    assert whole <= tol_whole, (name, whole)
    assert worst <= tol_stream, (name, worst, at)
    return whole, worst
