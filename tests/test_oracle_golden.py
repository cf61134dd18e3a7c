"""Regression pin: the oracle and the input generator still reproduce the stored tiny-workload
rows written by tests/golden/make_golden.py."""
import hashlib
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_dense_rows.json")


def test_tiny_golden_rows():
    g = json.load(open(GOLDEN))
    p = W.make_tiny(g["seed"])
    h = hashlib.sha256()
    for a in (p.q, p.k, p.w, p.q_pos, p.k_len):
        h.update(a.tobytes())
    assert h.hexdigest() == g["input_sha256"]
    inp = oracle.Inputs(p)
    for t, row in g["rows"].items():
        r = oracle.dense_row(inp, 0, int(t), g["k"])
        assert r["ids"].tolist() == row["ids"]
        assert np.array_equal(r["scores"], np.array(row["scores"]))
