"""Write oracle_tiny_regression.txt: sampled oracle outputs of a small seeded
GDN-2 problem.  Calls only the oracle and the seeded input generator."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from channel_wise_gated_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_regression.txt")


def compute():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=64, dk=16, dv=16)
    x = make_inputs(wl)
    o, sT = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                           gamma=x["gamma"], z=x["z"], S0=x["S0"])
    return o, sT


def main():
    o, sT = compute()
    lines = ["# oracle regression: gdn2 recipe at B1 H2 T64 d16, seed 2",
             "# kind index value"]
    for idx in [(0, 0, 0, 0), (0, 0, 31, 5), (0, 1, 63, 15), (0, 1, 17, 9)]:
        lines.append(f"o {','.join(map(str, idx))} {float(o[idx])!r}")
    for idx in [(0, 0, 0, 0), (0, 1, 15, 15), (0, 1, 3, 12)]:
        lines.append(f"S_T {','.join(map(str, idx))} {float(sT[idx])!r}")
    lines.append(f"o_norm - {float(np.linalg.norm(o))!r}")
    lines.append(f"S_T_norm - {float(np.linalg.norm(sT))!r}")
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
