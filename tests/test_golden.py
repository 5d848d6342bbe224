"""Stored fixtures under tests/golden/ (written by tests/golden/make_golden.py, which calls
only the input generators and the oracle): the SHA-256 of every input tensor of the five
stated workloads, and the oracle's r and row sums of h1 and y for the 256^3 forward.
A change of the seeded inputs or of the oracle's forward arithmetic fails here."""
import hashlib
import os

import numpy as np

import oracle as O
import workloads as W

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_rows(name):
    with open(os.path.join(HERE, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_input_hashes_of_the_five_workloads():
    stored = {(w, k): (shape, h) for w, k, shape, h in read_rows("input_sha256.txt")}
    assert {w for w, _ in stored} == set(W.WORKLOADS)
    for name, fn in W.WORKLOADS.items():
        wl = fn()
        for k, a in wl.tensors.items():
            shape, h = stored[(name, k)]
            assert "x".join(map(str, a.shape)) == shape, (name, k)
            assert hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest() == h, (name, k)


def test_tiny_forward_oracle_values():
    rows = np.array([[float(v) for v in r] for r in read_rows("tiny_fwd_oracle.txt")])
    assert rows.shape == (256, 4) and np.array_equal(rows[:, 0], np.arange(256))
    wl = W.tiny_fwd(0)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    # fp64 results of a BLAS may differ in the last bits between builds; nothing else may
    np.testing.assert_allclose(ref["r"], rows[:, 1], rtol=1e-12, atol=0)
    np.testing.assert_allclose(ref["h1"].sum(axis=1), rows[:, 2], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(ref["y"].sum(axis=1), rows[:, 3], rtol=1e-10, atol=1e-10)
