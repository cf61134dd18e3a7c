"""Writes the stored expected values under tests/golden/ from the oracle alone.

    python tests/golden/make_golden.py

tiny_dense_rows.json: for the tiny workload (one 1024-token fp32 prefill, 4 heads of dim 32,
top-64, seed 0) the oracle's selection and scores on a fixed set of rows, plus a digest of the
generated inputs so that a change of the generator is noticed. It is a regression pin of the
oracle and a ready-made expected value for the GPU parity test of the same rows.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

ROWS = [0, 1, 2, 31, 63, 64, 65, 127, 300, 511, 777, 1000, 1023]


def digest(p):
    h = hashlib.sha256()
    for a in (p.q, p.k, p.w, p.q_pos, p.k_len):
        h.update(a.tobytes())
    return h.hexdigest()


def main():
    p = W.make_tiny(0)
    inp = oracle.Inputs(p)
    rows = {}
    for t in ROWS:
        r = oracle.dense_row(inp, 0, t, 64)
        rows[str(t)] = dict(ids=[int(i) for i in r["ids"]],
                            scores=[float(s) for s in r["scores"]])
    out = dict(workload="tiny", k=64, seed=0, input_sha256=digest(p), rows=rows,
               note="oracle output (float64 scores, selection order = descending score, "
                    "lower index first on ties); written by tests/golden/make_golden.py")
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                           "tiny_dense_rows.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
