"""Helpers shared by the GPU tests (marshalling only; no arithmetic of the method)."""
import numpy as np


def to_dev(a, torch, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def upload(q, bits, scales, x, torch):
    return (to_dev(q, torch), to_dev(bits, torch), to_dev(scales.view(np.int16), torch, torch.float16),
            to_dev(np.atleast_2d(x).view(np.int16), torch, torch.float16))


def within_bound(y_gpu, y_ref, bound, rel=1e-3):
    """Acceptance of the GEMV: |y - y_ref| <= rel * sum|w||x| per output.

    Outputs whose bound is non-finite (a non-finite weight met a nonzero x)
    must be non-finite; outputs with a zero bound must be exactly zero.
    Returns (ok, worst ratio of error to bound, index of the worst output).
    """
    y = np.asarray(y_gpu, dtype=np.float64)
    fin = np.isfinite(bound)
    ok = True
    if (~fin).any():
        ok &= bool(np.all(~np.isfinite(y[~fin])))
    zero = fin & (bound == 0)
    if zero.any():
        ok &= bool(np.all(y[zero] == 0))
    live = fin & (bound > 0)
    if not live.any():
        return ok, 0.0, None
    err = np.abs(y[live] - y_ref[live])
    ratio = np.where(np.isfinite(err), err / bound[live], np.inf)
    worst = int(np.argmax(ratio))
    ok &= bool(np.all(ratio <= rel))
    return ok, float(ratio[worst]), worst
