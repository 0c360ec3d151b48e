"""Write the stored oracle values for the tiny d=16 workload.

Calls only ``oracle`` and ``gdn_inputs``.  Run from the repository root:
    python tests/golden/make_golden.py
The fixture lets later changes to the oracle be caught as a change of value.
The workload is the tiny step recurrence (N=1, one head, d_k=d_v=16, T=64,
fp32, S0=0, a=exp(-softplus(x)), norm weight 1), the values the oracle
computes for it: outputs o [64, 16], the final state S [16, 16] and the
RMSNormGated output y [64, 16] (eps=1e-6, scale=1).
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import gdn_inputs  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "tiny_d16_oracle.txt")


def compute():
    x = gdn_inputs.workload(0)
    orc = oracle.load()
    o, S = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, scale=1.0)
    y = orc.rmsnorm_gated(o, x.z, x.w, eps=1e-6)
    return o[:, 0, :], S[0, 0], y[:, 0, :]


def main():
    o, S, y = compute()
    with open(OUT, "w") as f:
        f.write("# oracle values for the tiny d=16 step-recurrence workload (seed 0)\n")
        f.write("# written by tests/golden/make_golden.py; sections o[64,16], S[16,16], y[64,16]\n")
        for name, arr in (("o", o), ("S", S), ("y", y)):
            f.write(f"{name} {arr.shape[0]} {arr.shape[1]}\n")
            for row in arr:
                f.write(" ".join(f"{x:.17g}" for x in row) + "\n")


if __name__ == "__main__":
    main()
