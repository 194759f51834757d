"""The uncertainty helper used by the GPU pipeline tests: perturbations of the maps within the
stated bound never flip a keep decision that it marks certain, and some do flip the others."""
import numpy as np

import oracle
import workloads as W
from capture_bounds import certain_patterns


def test_certain_patterns_survive_every_perturbation_within_the_bound():
    A = W.capture_maps(layers=1, heads=8, L=128, n_avg=4, layer_offset=21)
    ref = oracle.capture(A)
    flips_outside = 0
    for rel in (1e-2, 5e-2):
        cd, cv = certain_patterns(A, rel, 1e-9)
        assert cd.mean() > 0.9 and cv.mean() > 0.9
        rng = np.random.default_rng(1)
        for trial in range(12):
            f = 1 + (rng.uniform(-rel, rel, A.shape) if trial % 3 else rel * rng.choice([-1, 1], A.shape))
            c = oracle.capture((A.astype(np.float64) * f).astype(np.float32))
            dd = c["keep_diag"] != ref["keep_diag"]
            dv = c["keep_vert"] != ref["keep_vert"]
            assert not (dd & cd).any() and not (dv & cv).any()
            flips_outside += int(dd.sum() + dv.sum())
    assert flips_outside > 0   # the bound is not vacuous: uncertain patterns do flip
