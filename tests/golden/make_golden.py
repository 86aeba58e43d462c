"""Write the oracle regression fixture ``oracle_tiny.json``.

The pages print no worked numeric example of the scan, so nothing here pins
the oracle to a printed value; the oracle is pinned by identities in
tests/test_oracle_pins.py.  This fixture only freezes the oracle's output on
one tiny seeded case so that a later change to its arithmetic shows up as a
diff.  It calls nothing but ``oracle`` and ``selscan_inputs``.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import selscan_inputs as si  # noqa: E402

CASE = dict(batch=1, L=12, dim=3, N=4, dtype=si.F32, gate=True, seed=424242, h0=True)


def main():
    inp = si.make_fwd_inputs(**CASE)
    y, h = oracle.fwd_inputs(inp, threads=1)
    out = {
        "about": "oracle regression fixture (not a pin: the pages print no worked example)",
        "case": CASE,
        "y": [float(v) for v in y.ravel()],
        "h_last": [float(v) for v in h.ravel()],
    }
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
