"""Shared test helpers: error metrics, device handling and case announcements."""
import json
import os
import sys

import numpy as np

# Elements whose reference magnitude is below this fraction of the tensor's
# largest one are left out of the elementwise error (their relative error is
# dominated by absolute rounding of the larger terms they are summed from).
ELEM_FLOOR = 1e-3


def elemrel(x, ref, floor=ELEM_FLOOR):
    """Elementwise relative error max_i |x_i - r_i| / |r_i| over |r_i| >= floor * max|r|."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    mag = np.abs(ref)
    keep = mag >= floor * mag.max()
    if not keep.any():
        return float(np.abs(x - ref).max())
    return float((np.abs(x - ref)[keep] / mag[keep]).max())


def maxrel(x, ref, name=None):
    """Normwise max relative error: max|x - ref| / max|ref| over one tensor.

    The elementwise error (elemrel) is computed beside it; both are printed and,
    when SSLP_PARITY_LOG names a file, appended to it as one JSON line with the
    running test's id, so every parity comparison leaves its achieved errors."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(x - ref).max() if ref.size else 0.0
    norm = float(num / den) if den > 0 else float(num)
    elem = elemrel(x, ref)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    label = name or "tensor"
    print(f"    [parity] {test} {label}: normwise {norm:.3e} elementwise {elem:.3e} "
          f"(n={ref.size})", flush=True)
    log = os.environ.get("SSLP_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps(dict(test=test, name=label, normwise=norm, elementwise=elem,
                                    n=int(ref.size), shape=list(ref.shape))) + "\n")
    return norm


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
