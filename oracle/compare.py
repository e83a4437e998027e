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
