"""Helpers shared by the GPU parity tests: error metrics, tolerances and
host/device moves.

Every error the metrics compute is also recorded: printed to stderr and, when
the environment names a file in GDN_MARGIN_LOG, appended to it as one JSON
line (test id, scaled max error, and the elementwise relative error over the
elements that are not near zero), so a run leaves the parity margins on
record."""
import json
import os
import sys

import numpy as np
import torch

# Tolerances on the scaled max error (max |x - r| / max |r| per (request, head)
# slice): 1e-4 when the state is FP32, 2e-2 when it is stored in BF16 and the
# oracle rounds to BF16 at the same points.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# elements whose reference magnitude is at least this fraction of their
# slice's largest take part in the elementwise relative-error report
NEAR_ZERO = 1e-2


def _record(kind: str, scaled: float, elementwise: float, slices: int) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    rec = dict(test=test, kind=kind, scaled=scaled, elementwise=elementwise, slices=slices)
    print(f"[margin] {test} {kind}: scaled {scaled:.3e}, elementwise {elementwise:.3e}",
          file=sys.stderr, flush=True)
    path = os.environ.get("GDN_MARGIN_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _slice_errors(xs: np.ndarray, rs: np.ndarray):
    """Per row: max|x - r| / max|r|, and max |x - r| / |r| over elements with
    |r| >= NEAR_ZERO * max|r| of the row."""
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.max(np.abs(rs), axis=1)
    den = np.where(den > 0, den, 1.0)
    num = np.nan_to_num(num, nan=0.0)
    keep = np.abs(rs) >= NEAR_ZERO * den[:, None]
    rel = np.where(keep, np.abs(xs - rs) / np.where(keep, np.abs(rs), 1.0), 0.0)
    rel = np.nan_to_num(rel, nan=0.0)
    return num / den, np.max(rel, axis=1)


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
    if np.any(np.isnan(xs) != np.isnan(rs)):
        return float("inf")
    scaled, elem = _slice_errors(xs, rs)
    _record("slices", float(np.max(scaled)), float(np.max(elem)), n)
    return float(np.max(scaled))


def tol(*dtypes) -> float:
    """1e-4 when every tensor that feeds the compared value is FP32, else 2e-2."""
    return TOL_BF16 if any(d == torch.bfloat16 for d in dtypes) else TOL_F32


def state_tol(state_dtype) -> float:
    """Tolerance on a stored state: 1e-4 for an FP32 state whatever the
    activation dtype (BF16 activations are exact inputs to both sides), 2e-2
    for a BF16-stored state.  Outputs o stored in BF16 take tol(BF16)."""
    return TOL_F32 if state_dtype == torch.float32 else TOL_BF16


def seq_err(x, r, cu) -> float:
    """Scaled max error per (sequence, head) slice of a [N, H, d] prefill output:
    max over sequences s and heads h of max|x - r| / max|r| over the tokens of s."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    cu = np.asarray(cu, np.int64)
    worst, worst_elem, n = 0.0, 0.0, 0
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b > a:
            xs = x[a:b].transpose(1, 0, 2).reshape(x.shape[1], -1)
            rs = r[a:b].transpose(1, 0, 2).reshape(r.shape[1], -1)
            if np.any(np.isnan(xs) != np.isnan(rs)):
                return float("inf")
            scaled, elem = _slice_errors(xs, rs)
            worst = max(worst, float(np.max(scaled)))
            worst_elem = max(worst_elem, float(np.max(elem)))
            n += xs.shape[0]
    _record("sequence-heads", worst, worst_elem, n)
    return worst
