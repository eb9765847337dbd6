"""Writes tests/golden/tiny_oracle.txt from the oracle alone.

The pages print no worked example (no input or output values), so the only
stored values here are the oracle's own results on the tiny case (2 sequences
of lengths 5 and 13, 64 channels; one decode token per sequence through the
gated delta rule with 2+2 heads of dim 16).  They guard against an
unintended change to the oracle's arithmetic: any such change must be made
on purpose and this file regenerated in the same commit.

Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")


def tiny_results():
    d = synth.tiny(0)
    chunks = oracle.build_conv_chunks(d["qsl"])
    y, cs = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                         d["qsl"], d["state_indices"], d["has_init"])
    yu, cs2 = oracle.causal_conv1d_update(d["x_dec"], d["weight"], d["bias"], cs,
                                          d["state_indices"])
    o, st = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    d["state_indices"], None, None, 1.0, True)
    return dict(chunks=chunks, conv_y=y, conv_state=cs, update_y=yu, update_state=cs2,
                gdn_o=o, gdn_state=st[d["state_indices"]])


def main():
    res = tiny_results()
    with open(OUT, "w") as f:
        f.write("# oracle results on the tiny case (seed 0); written by make_golden.py\n")
        for name, a in res.items():
            a = np.asarray(a)
            f.write("%s %s %s\n" % (name, a.dtype.str, " ".join(map(str, a.shape))))
            flat = a.ravel()
            if a.dtype.kind == "f":
                f.write(" ".join(v.hex() for v in flat.astype(float)) + "\n")
            else:
                f.write(" ".join(str(int(v)) for v in flat) + "\n")


if __name__ == "__main__":
    main()
