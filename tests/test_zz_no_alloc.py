"""GPU: the allocation-free sample-scores entry point (sa_sample_scores_noalloc, static scratch) against the
allocating one (sa_sample_scores, caller workspace) through the C ABI: the same kernels, so the row LSE and the
int64 scores are bit-identical.  Two calls in a row on one GPU, the second with a smaller input (the static
array keeps the first call's contents), then a request above the 16 MiB limit, which is rejected."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import note, sa, to_dev

pytestmark = pytest.mark.gpu


def _both(m, q, k, row0, n, band, skip=None):
    qd, kd = to_dev(q), to_dev(k)
    sk = None if skip is None else torch.from_numpy(skip).cuda()
    ref = m.sample_scores(qd, kd, row0, n, band=band, skip_cols=sk)
    got = m.sample_scores(qd, kd, row0, n, band=band, skip_cols=sk, no_alloc=True)
    torch.cuda.synchronize()
    for a, b, what in zip(ref, got, ("diag", "vert", "row_lse")):
        assert torch.equal(a, b), what
    return got


def test_noalloc_matches_allocating_entry_point_twice():
    m = sa()
    note("no-alloc sample scores: large call")
    q, k, _ = W.qkv(91, 2, 8, 2, 6000, 128, "bf16")
    skip = (np.random.default_rng(91).random((8, 6000)) < 0.05).astype(np.uint8)
    _both(m, q, k, 5800, 200, 32, skip)
    note("no-alloc sample scores: smaller call after it")
    q, k, _ = W.qkv(92, 1, 4, 4, 900, 64, "f32")
    _both(m, q, k, 800, 100, 8)


def test_noalloc_rejects_scratch_above_limit():
    m = sa()
    note("no-alloc sample scores: above the static limit")
    B, hq, S, d = 1, 64, 65536, 64
    q = torch.zeros((B, hq, S, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, S, d), dtype=torch.bfloat16, device="cuda")
    # 64 heads x 256 rows x 256 splits x 8 bytes = 32 MiB > 16 MiB
    assert m.lib.sa_sample_scores_workspace(B, hq, S - 256, 256) > 16 << 20
    with pytest.raises(m.SAError) as e:
        m.sample_scores(q, k, S - 256, 256, no_alloc=True)
    assert e.value.code == -4
