"""Write tests/golden/oracle_tiny.json: fixed small inputs and the fp64 oracle's
outputs for them.  The pages print no worked numeric example for this method,
so this fixture is a regression lock on the oracle itself (its values are
pinned independently by tests/test_oracle_pins.py); it calls only oracle/.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def inputs():
    # exact binary fractions, so the fixture is reproducible bit for bit
    t = np.arange(6, dtype=np.float64)
    i = np.arange(4, dtype=np.float64)
    j = np.arange(3, dtype=np.float64)
    q = ((t[:, None] + 1) * (i[None, :] - 1.5) / 8.0)[None, None]
    k = ((2 - t[:, None]) * (i[None, :] + 0.5) / 8.0)[None, None]
    v = ((t[:, None] - 2.5) + (j[None, :] - 1) / 4.0)[None, None]
    g = ((t[:, None] - i[None, :]) / 2.0)[None, None]
    th = ((i[None, :] - t[:, None] + 1.0) / 4.0)[None, None]
    S0 = ((i[:, None] - j[None, :]) / 16.0)[None, None]
    return q, k, v, g, th, S0


def main():
    q, k, v, g, th, S0 = inputs()
    o, ST = oracle.scan(q, k, v, g, th, S0)
    la, lb = oracle.gates(g, th)
    qs = np.concatenate([q[0, 0], q[0, 0, :2] * 3.0]).reshape(1, 1, 8, 4)
    ks = (np.arange(8 * 4, dtype=np.float64).reshape(1, 8, 4) % 5 - 2) / 4.0
    vs = np.concatenate([v[0, 0], v[0, 0, :2]]).reshape(1, 1, 8, 3)
    os_ = oracle.swska(qs, ks, vs, 3)
    rec = {"shapes": "B=1 H=1 T=6 dk=4 dv=3; SW-SKA T=8 w=3",
           "q": q.tolist(), "k": k.tolist(), "v": v.tolist(), "g": g.tolist(), "theta": th.tolist(),
           "S0": S0.tolist(), "o": o.tolist(), "S_T": ST.tolist(),
           "log_a": la.tolist(), "log_beta": lb.tolist(),
           "swska_q": qs.tolist(), "swska_k": ks.tolist(), "swska_v": vs.tolist(),
           "swska_window": 3, "swska_o": os_.tolist()}
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as fh:
        json.dump(rec, fh, indent=0)


if __name__ == "__main__":
    main()
