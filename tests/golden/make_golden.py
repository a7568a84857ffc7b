"""Writes tests/golden/tiny_fwd.json: a frozen sample of the float64 oracle's
output on the Tiny workload (B=1, L=64, D=32, N=16, fp32), used as a
regression guard on the oracle.  Calls only ``oracle`` and the seeded input
generator ``workloads``.  The pages print no numeric worked example for the
scan, so no fixture here carries values taken from them.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.as_float32(workloads.make_inputs(w))
    y, hf = oracle.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"],
                            inp["z"], inp["dt_bias"], None, softplus=True)
    idx = np.linspace(0, y.size - 1, 48).astype(int)
    out = {
        "workload": "tiny: B=1 L=64 D=32 N=16 fp32, seed 1, softplus on, no h0",
        "y_index": idx.tolist(),
        "y_values": [float(v) for v in y.reshape(-1)[idx]],
        "y_sum": float(np.sum(y)),
        "h_final_sumsq": float(np.sum(hf * hf)),
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fwd.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
