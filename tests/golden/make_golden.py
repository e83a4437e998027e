"""Writes attention_cases.json: FP64 oracle outputs of a few small seeded attention problems,
kept as a regression fixture (a later change to the oracle that moves them fails
tests/test_golden.py) and as stored expectations the GPU kernels are checked against
without running the oracle at test time.

Calls only ``oracle/`` (the arithmetic) and the seeded input generators of ``workloads``
(which hold none of the method's arithmetic). Run from the repository root:

    python tests/golden/make_golden.py

What the stored values are: softmax attention with natural-log LSE, as defined on page
"[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on sglang PR #49219),
section "code analysis" item 1 (non-causal SDPA, no mask, no dropout, on equal-shape BF16
Q/K/V) and page "PR #33702 report", breakdown item 2 (packed varlen attention confined to
each sequence). The pages print no worked example, so no stored value is a page value.
"""
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import attention_dense, attention_varlen  # noqa: E402
from workloads import random_dense, random_varlen  # noqa: E402

OUT = os.path.join(HERE, "attention_cases.json")
SCALE = 1.0 / math.sqrt(128.0)

# (name, kind, generator arguments, scale, checked rows). V stays N(0, 1) in every case: the
# outputs then stay below 4 in magnitude, where BF16 output rounding alone is under 2e-2. Dense rows are flat indices
# (b*H + h)*N + n; packed rows are h*T + t. Each case spans several 64-key tiles and ends in
# a ragged tail; the packed case has a length-1 and a 127-token segment.
CASES = [
    ("dense_ragged_N300", "dense", {"B": 1, "H": 2, "N": 300, "seed": 41, "std": 1.0}, SCALE,
     [0, 63, 255, 256, 299, 300, 431, 599]),
    ("dense_large_logits_N130", "dense", {"B": 1, "H": 1, "N": 130, "seed": 45, "std": 4.0, "v_std": 1.0}, SCALE,
     [0, 1, 64, 127, 128, 129]),
    ("varlen_1_127_200", "varlen", {"seqlens": [1, 127, 200], "H": 2, "seed": 43, "std": 1.0}, SCALE,
     [0, 1, 127, 128, 327, 328, 329, 455, 655]),
]


def inputs(kind, args):
    if kind == "dense":
        q, k, v = random_dense(args["B"], args["H"], args["N"], seed=args["seed"], std=args["std"])
        if "v_std" in args:   # V of its own spread (N(0,1) keeps |o| where BF16 output rounding < 2e-2)
            v = random_dense(args["B"], args["H"], args["N"], seed=args["seed"] + 500, std=args["v_std"])[2]
        return q, k, v, None
    return random_varlen(args["seqlens"], args["H"], seed=args["seed"], std=args["std"])


def expected(kind, args, scale, rows):
    q, k, v, cu = inputs(kind, args)
    rows = np.asarray(rows, dtype=np.int64)
    if kind == "dense":
        o, lse = attention_dense(q, k, v, scale, rows=rows)
    else:
        T = int(cu[-1])
        o_full, lse_full = attention_varlen(q, k, v, cu, scale)
        h, t = rows // T, rows % T
        o, lse = o_full[t, h], lse_full[h, t]
    return o, lse


def main():
    doc = {"about": __doc__.strip().splitlines()[0], "definition": (
        "o_i = sum_j softmax_j(s q_i.k_j) v_j, lse_i = ln sum_j exp(s q_i.k_j), FP64 from the BF16 "
        "inputs; page 'SANA-Video 2.0 anchor attention ... FP32 upcast' (blog on sglang PR #49219), "
        "code analysis item 1; page 'PR #33702 report', breakdown item 2 (varlen)"),
        "cases": []}
    for name, kind, args, scale, rows in CASES:
        o, lse = expected(kind, args, scale, rows)
        doc["cases"].append({"name": name, "kind": kind, "args": args, "scale": scale, "rows": rows,
                             "o": [[float("%.17g" % x) for x in r] for r in o],
                             "lse": [float("%.17g" % x) for x in lse]})
    with open(OUT, "w") as f:   # one output row per line
        f.write("{\n")
        f.write('"about": %s,\n"definition": %s,\n"cases": [\n' % (json.dumps(doc["about"]), json.dumps(doc["definition"])))
        for ci, c in enumerate(doc["cases"]):
            head = {k: c[k] for k in ("name", "kind", "args", "scale", "rows", "lse")}
            f.write(json.dumps(head)[:-1] + ',\n "o": [\n')
            f.write(",\n".join("  " + json.dumps(r, separators=(",", ":")) for r in c["o"]))
            f.write("\n ]}" + ("," if ci + 1 < len(doc["cases"]) else "") + "\n")
        f.write("]}\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
