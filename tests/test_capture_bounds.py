"""The uncertainty helper used by the GPU pipeline tests: perturbations of the maps within the
stated bound never flip a keep decision that it marks certain, and some do flip the others."""
import numpy as np

import oracle
import workloads as W
from capture_bounds import certain_patterns, certain_selection


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


def test_certain_selection_survives_every_perturbation_within_the_bound():
    rng = np.random.default_rng(8)
    n, S, rows = 6, 400, 8
    x = rng.pareto(1.2, size=(n, S))
    x *= 0.7 * rows / x.sum(axis=1, keepdims=True)    # 70 % of the sampled mass not covered yet
    x[:, ::17] = 0.0
    flips_outside = 0
    for rel, ab in ((1e-3, 1e-6), (2e-2, 1e-5)):
        for alpha in (0.5, 0.9, 0.97):
            sure = certain_selection(x, rel, ab, alpha, rows, band=3)
            ref = oracle.select_patterns(oracle.fixed_point(x), alpha, rows, band=3)
            assert sure.mean() > 0.8
            for trial in range(10):
                e = rng.uniform(-1, 1, x.shape) if trial % 2 else rng.choice([-1, 1], x.shape)
                xp = np.maximum(x + e * (rel * x + ab), 0.0)
                got = oracle.select_patterns(oracle.fixed_point(xp), alpha, rows, band=3)
                assert not ((got != ref) & sure).any()
                flips_outside += int((got != ref).sum())
    assert flips_outside > 0
