"""Write tests/golden/oracle_single_seed0.txt from the fp64 oracle only.

Row layout: logits z[24], coefficients pre|post|H [24], layer_in[:8],
X'[:, :8] (4 x 8), for the single-token workload (T=1, n_hc=4, d=256, seed 0).
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from deepseek_v4_hyper_amd import workloads as wl  # noqa: E402


def main():
    case = wl.make_single(0)
    X = wl.state_to_f64(case.X, case.dtype)
    lo = wl.state_to_f64(case.layer_out, case.dtype)
    li, c, out = oracle.fused(X, case.W, case.bias, lo, case.eps, case.iters)
    _, _, z = oracle.pre(X, case.W, case.bias, case.eps, case.iters)
    vals = np.concatenate([z[0], c[0], li[0, :8], out[0, :, :8].ravel()])
    path = os.path.join(ROOT, "tests", "golden", "oracle_single_seed0.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle, single-token workload (T=1, n_hc=4, d=256, seed 0)\n")
        f.write("# z[24] | pre|post|H [24] | layer_in[:8] | X'[:, :8] (4x8); "
                "written by tests/golden/make_golden.py\n")
        for v in vals:
            f.write("%.17g\n" % v)


if __name__ == "__main__":
    main()
