"""Stored FP64 expectations in tests/golden/attention_cases.json (written by
tests/golden/make_golden.py from the oracle).

CPU: the oracle still reproduces every stored value (a change to its arithmetic that moves
them fails here), and the stored values of the length-1 segment equal what the definition
gives by hand (o = v_0, lse = s q.k), so the fixture itself is pinned to the mathematics.
GPU: the dense and packed kernels match the stored rows within the parity tolerances, with
no oracle run at test time.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import bf16_bits_to_f64, compare, scale_as_used
from tests.golden.make_golden import OUT, expected, inputs

CASES = json.load(open(OUT))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces_stored_values(case):
    o, lse = expected(case["kind"], case["args"], case["scale"], case["rows"])
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=1e-12, atol=1e-15)


def test_stored_length_one_segment_is_closed_form():
    case = next(c for c in CASES if c["kind"] == "varlen" and c["args"]["seqlens"][0] == 1)
    q, k, v, cu = inputs("varlen", case["args"])
    T = int(cu[-1])
    s = scale_as_used(case["scale"])
    seen = 0
    for i, r in enumerate(case["rows"]):
        h, t = divmod(r, T)
        if t != 0:
            continue
        qv, kv, vv = (bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        assert case["o"][i] == list(vv)                       # exactly the one value row
        assert math.isclose(case["lse"][i], s * math.fsum(qv * kv), rel_tol=1e-14, abs_tol=1e-14)
        seen += 1
    assert seen == case["args"]["H"]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_kernel_matches_stored_values(case):
    import torch

    import video_diffusion_dit_amd as vd
    from tests.gpu_util import dev, dev_i32, f64_of

    print(f"[golden] {case['name']}", flush=True)
    q, k, v, cu = inputs(case["kind"], case["args"])
    rows = np.asarray(case["rows"])
    if case["kind"] == "dense":
        o, lse = vd.attn_fwd(dev(q), dev(k), dev(v), scale=case["scale"], return_lse=True)
        torch.cuda.synchronize()
        og = f64_of(o).reshape(-1, q.shape[-1])[rows]
        lg = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    else:
        o, lse = vd.attn_fwd_varlen(dev(q), dev(k), dev(v), dev_i32(cu), scale=case["scale"], return_lse=True)
        torch.cuda.synchronize()
        T = int(cu[-1])
        og = f64_of(o)[rows % T, rows // T]
        lg = lse.cpu().numpy().astype(np.float64)[rows // T, rows % T]
    m = compare(og, np.array(case["o"]), lg, np.array(case["lse"]))
    print(f"[golden] {case['name']}: {m}", flush=True)
    assert m["ok"], m
