"""Writes ``tiny_oracle.json``: the tiny configuration's seeded inputs and the
oracle's fp64 output.  Calls only the oracle and the seeded input generator.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from broadcast_gemm_amd.inputs import CONFIGS, make_inputs  # noqa: E402


def main():
    cfg = CONFIGS[0]
    x = make_inputs(cfg)
    Y = oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c)
    doc = {
        "_about": "Tiny LCE configuration (fp32, B_u=2, B_c=8): seeded inputs and the CPU "
                  "oracle's fp64 output Y[b] = W_u.U[map[b]] + W_c.C[b]. Written by make_golden.py.",
        "config": cfg.name,
        "shapes": {"B_u": cfg.B_u, "B_c": cfg.B_c, "K_u": cfg.K_u, "K_c": cfg.K_c, "M": cfg.M, "D": cfg.D},
        "map": x.map.tolist(),
        "U": x.U.ravel().tolist(), "C": x.C.ravel().tolist(),
        "W_u": x.W_u.ravel().tolist(), "W_c": x.W_c.ravel().tolist(),
        "Y": [float.hex(float(v)) for v in Y.ravel()],
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as fh:
        json.dump(doc, fh, indent=0)


if __name__ == "__main__":
    main()
