"""Helpers shared by the GPU parity tests: error metric and host/device moves."""
import sys

import numpy as np
import torch

# Tolerances on the scaled max error (max |x - r| / max |r| per (request, head)
# slice): 1e-4 when the state is FP32, 2e-2 when it is stored in BF16 and the
# oracle rounds to BF16 at the same points.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*a):
    """Name the case before a GPU step (flushed, so a lost box still shows it)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def scaled_err(x, r, lead: int) -> float:
    """max over the first `lead` axes of max|x - r| / max|r| over the rest."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        return 0.0
    n = int(np.prod(x.shape[:lead])) if lead else 1
    xs = x.reshape(n, -1)
    rs = r.reshape(n, -1)
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.max(np.abs(rs), axis=1)
    den = np.where(den > 0, den, 1.0)
    if np.any(np.isnan(xs) != np.isnan(rs)):
        return float("inf")
    num = np.nan_to_num(num, nan=0.0)
    return float(np.max(num / den))


def tol(*dtypes) -> float:
    """1e-4 when every tensor that feeds the compared value is FP32, else 2e-2."""
    return TOL_BF16 if any(d == torch.bfloat16 for d in dtypes) else TOL_F32


def seq_err(x, r, cu) -> float:
    """Scaled max error per (sequence, head) slice of a [N, H, d] prefill output:
    max over sequences s and heads h of max|x - r| / max|r| over the tokens of s."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    cu = np.asarray(cu, np.int64)
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b > a:
            worst = max(worst, scaled_err(x[a:b].transpose(1, 0, 2), r[a:b].transpose(1, 0, 2), 1))
    return worst
