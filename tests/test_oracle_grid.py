"""oracle.noise_grid is the oracle's uniform -> E -> g on consecutive grid points
(its values are pinned by the decimal tests of test_oracle_noise.py)."""
import numpy as np

import oracle


def test_noise_grid_matches_pointwise():
    for fp64, bits in ((False, 23), (True, 52)):
        for k0 in (0, 5, 2**bits // 2 - 2, 2**bits - 3):
            E, g = oracle.noise_grid(fp64, k0, 3)
            for t in range(3):
                e1, g1 = oracle.noise_of_uniform((k0 + t + 0.5) / 2**bits)
                assert E[t] == e1 and g[t] == g1
