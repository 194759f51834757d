"""GPU parity: sa_attention_maps vs the fp64 oracle (float32 maps, max-abs 1e-5), and the
capture pipeline from Q/K: GPU maps -> GPU capture equals the oracle capture of the same
maps bit for bit (keep flags, hit counts, true mask)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from capture_bounds import certain_patterns
from gpu_util import assert_close_f32, note, sa, to_dev

pytestmark = pytest.mark.gpu


def _maps(q, k, what, scale=None):
    m = sa()
    B, hq, L, d = q.shape
    note("maps %s B=%d hq=%d hkv=%d L=%d d=%d dtype=%s" % (what, B, hq, k.shape[1], L, d, q.dtype))
    got = m.attention_maps(to_dev(q), to_dev(k), softmax_scale=scale)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    ref = oracle.attention_maps(q, k, scale=scale)
    assert_close_f32(g.astype(np.float64), ref, what)
    iu = np.triu_indices(L, 1)
    assert not g[:, iu[0], iu[1]].any(), "entries above the diagonal must be zero"
    return got, ref


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_maps_ragged_length_gqa(dtype, d):
    """L = 333: five row blocks with a ragged last one, rows not a multiple of 4; GQA 4:2."""
    q, k, _ = W.qkv(41, 2, 4, 2, 333, d, dtype)
    _maps(q, k, "ragged")


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 512])
def test_maps_sizes(L):
    q, k, _ = W.qkv(42, 3, 2, 1, L, 64, "bf16")
    got, _ = _maps(q, k, "L=%d" % L)
    assert (got[:, 0, 0] - 1).abs().max().item() < 1e-6   # row 0 attends to key 0 only


def test_maps_batch_over_one_chunk_and_custom_scale():
    """B = 37 takes three batch chunks (16 + 16 + 5) through the read-add-write path."""
    q, k, _ = W.qkv(43, 37, 2, 2, 200, 128, "f32")
    _maps(q, k, "B=37", scale=0.3)


def test_maps_rows_are_distributions():
    q, k = W.capture_qk(44, 4, 8, 2, 512, 64, "bf16")
    got, _ = _maps(q, k, "structured")
    rows = got.sum(dim=2)
    assert (rows - 1).abs().max().item() < 1e-5


def test_maps_full_capture_length_limit():
    """The longest capture window the library takes, L = 4096."""
    q, k, _ = W.qkv(45, 1, 2, 1, 4096, 128, "bf16")
    _maps(q, k, "L=4096")


@pytest.mark.parametrize("d", [64, 128])
def test_capture_from_qk_pipeline(d):
    """One layer at the capture length: 32 query heads / 8 kv heads, batch 16, L = 512.  The GPU
    pipeline (maps -> capture) against the oracle pipeline on the same Q/K.  The maps agree within
    |A_gpu - A| <= 1e-5 A + 1e-9 (checked); the keep flags must then agree on every pattern whose
    decision no map within that bound can change (tests/capture_bounds.py), and those must be
    nearly all of them.  The inputs carry sink columns 0..3 and diagonal 0, which both keep."""
    m = sa()
    q, k = W.capture_qk(46, 16, 32, 8, 512, d, "bf16")
    note("capture pipeline from Q/K d=%d" % d)
    maps = m.attention_maps(to_dev(q), to_dev(k))
    got = m.pattern_capture(maps)
    torch.cuda.synchronize()
    ref_maps = oracle.attention_maps(q, k)
    g = maps.cpu().numpy().astype(np.float64)
    assert (np.abs(g - ref_maps) <= 1e-5 * ref_maps + 1e-9).all()
    ref = oracle.capture(ref_maps.astype(np.float32))
    cd, cv = certain_patterns(ref_maps.astype(np.float32), 1e-5 + 1e-7, 1e-9)
    note("certain patterns: diag %.5f vert %.5f" % (cd.mean(), cv.mean()))
    assert cd.mean() > 0.99 and cv.mean() > 0.99
    gd, gv = got["keep_diag"].cpu().numpy(), got["keep_vert"].cpu().numpy()
    np.testing.assert_array_equal(gd[cd], ref["keep_diag"][cd])
    np.testing.assert_array_equal(gv[cv], ref["keep_vert"][cv])
    assert ref["keep_vert"][:, :4].all() and ref["keep_diag"][:, 0].all()
