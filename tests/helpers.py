"""Shared test helpers: error metrics, device handling and case announcements."""
import sys

import numpy as np


def maxrel(x, ref):
    """Normwise max relative error: max|x - ref| / max|ref| over one tensor."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(x - ref).max() if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def announce(msg):
    """Name the GPU case on stdout before running it (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


TOL_FP32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(dtype):
    import torch

    return TOL_FP32 if dtype == torch.float32 else TOL_BF16


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False
