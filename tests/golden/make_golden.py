"""Writes the stored expected values under tests/golden/.

Only the CPU oracle (oracle/) and the seeded input generator are used.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssd_inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    for tv, name in ((False, "tiny_dt_zero.txt"), (True, "tiny_dt_varying.txt")):
        inp = ssd_inputs.tiny_case(tv)
        y, _ = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
        header = ("Real part of y for the Skills-page tiny recipe (B=2, T=16, H=2, D=N=4, seed 0, "
                  "dt %s), flattened (B,T,H,D) row-major. Written by make_golden.py from the oracle."
                  % ("~ N(0,1) drawn after C_t" if tv else "= 0"))
        np.savetxt(os.path.join(HERE, name), y.real.reshape(-1), fmt="%.17g", header=header)


if __name__ == "__main__":
    main()
