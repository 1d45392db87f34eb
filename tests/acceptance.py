"""Acceptance rule for comparing GPU outputs with the FP64 oracle.

Gate: every element finite; |err| <= 2e-2 + 2e-2*|ref| on at least 99.99% of the
elements, counted in integers; no element with |err| > 1e-1.

Also reported, for information: the pages' BF16 rule (page "Audit SGLang interfaces
and refresh validated kernel solutions", README BF16 tolerance sentence and
scripts/task_acceptance.py compare_output): |err| <= 0.005 + 0.016*|ref| with a
0.9999 matched fraction for the dense attention tasks.
"""
import numpy as np

ATOL = 2e-2
RTOL = 2e-2
RATIO_NUM, RATIO_DEN = 9999, 10000
CAP = 1e-1
PAGES_ATOL = 0.005
PAGES_RTOL = 0.016


def bf16_bits_to_f64(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def compare(actual, ref):
    """actual: GPU output (BF16 bits or float array); ref: oracle FP64, same shape."""
    a = bf16_bits_to_f64(actual) if np.asarray(actual).dtype == np.uint16 else np.asarray(
        actual, np.float64)
    r = np.asarray(ref, np.float64)
    assert a.shape == r.shape, (a.shape, r.shape)
    finite = bool(np.isfinite(a).all())
    err = np.abs(a - r)
    total = int(err.size)
    close = err <= ATOL + RTOL * np.abs(r)
    matched = int(close.sum())
    pages_close = err <= PAGES_ATOL + PAGES_RTOL * np.abs(r)
    pages_matched = int(pages_close.sum())
    max_err = float(np.nanmax(err)) if total else 0.0
    ok = (finite and matched * RATIO_DEN >= RATIO_NUM * total and (max_err <= CAP)
          and not np.isnan(err).any())
    return {
        "ok": bool(ok),
        "finite": finite,
        "elements": total,
        "matched": matched,
        "max_abs_err": max_err,
        "mean_abs_err": float(err.mean()) if total else 0.0,
        "pages_rule_matched": pages_matched,
        "pages_rule_ok": bool(finite and pages_matched * RATIO_DEN >= RATIO_NUM * total),
    }


def assert_accepted(actual, ref, what=""):
    res = compare(actual, ref)
    assert res["ok"], f"{what}: {res}"
    return res
