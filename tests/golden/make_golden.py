"""Writes the stored fixtures of tests/golden/ (run from the repository root:
`python tests/golden/make_golden.py`). It calls only the seeded input generators and
the oracle, never the HIP path.

- input_sha256.txt: the SHA-256 of every input tensor of the five stated workloads, as
  generated (bf16 bit patterns, C order), so that a change of the generators or of
  numpy's PCG64 stream shows up as a failed test rather than as silently different data.
- tiny_fwd_oracle.txt: the oracle's r and the row sums of h1 and y for the 256 x 256 x
  256 forward (seed 0), printed with 17 significant digits. The pages print no worked
  example, so these are the oracle's own values: they pin the oracle against unnoticed
  changes of its arithmetic, while the pins of tests/test_oracle.py tie it to closed
  forms and library routines.
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def input_hashes():
    lines = []
    for name, fn in W.WORKLOADS.items():
        wl = fn()
        for k in sorted(wl.tensors):
            a = np.ascontiguousarray(wl.tensors[k])
            lines.append(f"{name} {k} {'x'.join(map(str, a.shape))} {hashlib.sha256(a.tobytes()).hexdigest()}")
    return lines


def tiny_oracle():
    wl = W.tiny_fwd(0)
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    return ref["r"], ref["h1"].sum(axis=1), ref["y"].sum(axis=1)


def main():
    with open(os.path.join(HERE, "input_sha256.txt"), "w") as f:
        f.write("# workload tensor shape sha256 -- written by tests/golden/make_golden.py\n")
        f.write("\n".join(input_hashes()) + "\n")
    r, h1s, ys = tiny_oracle()
    with open(os.path.join(HERE, "tiny_fwd_oracle.txt"), "w") as f:
        f.write("# row r h1_rowsum y_rowsum -- fp64 oracle, 256x256x256 forward, seed 0, eps 1e-6;\n")
        f.write("# written by tests/golden/make_golden.py (the pages print no worked example)\n")
        for m in range(r.shape[0]):
            f.write(f"{m} {r[m]:.17g} {h1s[m]:.17g} {ys[m]:.17g}\n")


if __name__ == "__main__":
    main()
