"""Acceptance check of an attention result against the FP64 oracle.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): used by tests, smoke() and the bench's
CPU leg only.

Tolerances are the stated acceptance bar for the BF16 output and the FP32 log-sum-exp:
relative L2 <= 5e-3 and max-abs <= 2e-2 over every checked output element, and
|LSE - LSE_ref| <= 1e-3 absolute. Expected error of a correct kernel is about 2e-3
relative L2 (BF16 output rounding alone is ~1.7e-3 on N(0,1) data); page "[sglang]
SANA-Video 2.0 anchor attention ... FP32 upcast", section on accuracy, reports a
layer-level relative L2 of 2.2e-3 for BF16 inputs against the FP32 path.
"""
from __future__ import annotations

import numpy as np

REL_L2_TOL = 5e-3
MAX_ABS_TOL = 2e-2
LSE_TOL = 1e-3


def compare(o, o_ref, lse=None, lse_ref=None) -> dict:
    """Error metrics of o (any float dtype, same shape as o_ref) and optionally lse."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    diff = o - o_ref
    nref = float(np.linalg.norm(o_ref.ravel()))
    out = {
        "rel_l2": float(np.linalg.norm(diff.ravel())) / nref if nref > 0 else float(np.linalg.norm(diff.ravel())),
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "finite": bool(np.all(np.isfinite(o))),
        "n_elems": int(o.size),
    }
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        assert lse.shape == lse_ref.shape, (lse.shape, lse_ref.shape)
        out["lse_max_abs"] = float(np.max(np.abs(lse - lse_ref))) if lse.size else 0.0
        out["finite"] = out["finite"] and bool(np.all(np.isfinite(lse)))
    out["ok"] = bool(out["finite"] and out["rel_l2"] <= REL_L2_TOL and out["max_abs"] <= MAX_ABS_TOL
                     and out.get("lse_max_abs", 0.0) <= LSE_TOL)
    return out


def bf16_round_f64(y) -> np.ndarray:
    """The bfloat16 number nearest to each float64 value (ties to even), as float64.

    bfloat16 keeps 8 significant bits: with y = m * 2^e and 0.5 <= |m| < 1, the nearest
    bfloat16 is rint(m * 2^8) * 2^(e - 8) (numpy's rint breaks ties to even)."""
    m, e = np.frexp(np.asarray(y, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_spacing(y) -> np.ndarray:
    """Distance between consecutive bfloat16 numbers around |y| (normal range)."""
    _, e = np.frexp(np.asarray(y, dtype=np.float64))
    return np.ldexp(1.0, e - 8)


def bf16_faithful(got, exact, abs_floor: float = 2.0 ** -18) -> dict:
    """A BF16 result against exact values. 'ok' when every element is within one bfloat16
    spacing of the exact value, or within abs_floor of it (values that come out of a
    cancellation in FP32 carry an absolute error of a few FP32 ulps of the operands, which
    is far more than a bfloat16 spacing of the tiny result). 'rne_frac' is the fraction of
    elements equal to the nearest-even rounding of the exact value."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    assert got.shape == exact.shape, (got.shape, exact.shape)
    err = np.abs(got - exact)
    lim = np.maximum(bf16_spacing(exact), abs_floor)
    return {
        "max_err_over_limit": float(np.max(err / lim)) if err.size else 0.0,
        "rne_frac": float(np.mean(got == bf16_round_f64(exact))) if err.size else 1.0,
        "finite": bool(np.all(np.isfinite(got))),
        "n_elems": int(got.size),
        "ok": bool(np.all(np.isfinite(got)) and np.all(err <= lim)),
    }
