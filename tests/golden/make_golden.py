"""Write tests/golden/small_cases.json from the oracle only.

The KeOps pages print no numeric outputs, so these fixtures are regression
values written by this script, which calls nothing but ``oracle/`` and the
seeded input generator.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from geometric_map_reduce_amd import workloads  # noqa: E402

CASES = [
    # name, M, N, D, E, K, sigma, seed
    ("tiny_d3", 7, 11, 3, 1, 4, 0.8, 100),
    ("ragged_d5_e2", 13, 29, 5, 2, 6, 1.3, 101),
    ("d32_e1", 9, 40, 32, 1, 5, 4.0, 102),
]


def main():
    out = {}
    for name, M, N, D, E, K, sigma, seed in CASES:
        rng = np.random.default_rng(seed)
        x, y, b = workloads.random_points(rng, M, N, D, E)
        g = rng.standard_normal((M, E)).astype(np.float32)
        s = float(np.float32(sigma))
        a, n = oracle.gauss_sum(x, y, b, s)
        l = oracle.gauss_lse(x, y, b, s)
        G, nu = oracle.gauss_grad_x(x, y, b, g, s)
        Gy, nuy = oracle.gauss_grad_y(x, y, b, g, s)
        Gb, nub = oracle.gauss_grad_b(x, y, g, s)
        kd, ki = oracle.kmin(x, y, K)
        out[name] = dict(M=M, N=N, D=D, E=E, K=K, sigma=s, seed=seed,
                         x=x.tolist(), y=y.tolist(), b=b.tolist(), g=g.tolist(),
                         sum=a.tolist(), sum_norm=n.tolist(), lse=l.tolist(),
                         grad_x=G.tolist(), grad_norm=nu.tolist(),
                         grad_y=Gy.tolist(), grad_y_norm=nuy.tolist(),
                         grad_b=Gb.tolist(), grad_b_norm=nub.tolist(),
                         kmin_d=kd.tolist(), kmin_idx=ki.tolist())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "small_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
