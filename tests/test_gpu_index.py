"""GPU parity: sa_build_index vs the oracle index, bit for bit (every array)."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import note, sa

pytestmark = pytest.mark.gpu

KEYS = ("run_ptr", "run_lo", "run_hi", "seg_ptr", "seg_lo", "seg_hi", "bcol_ptr", "bcol_idx", "col_ptr", "col_idx",
        "pair_count", "dbits")


def _compare(desc, BM, what):
    note("index %s S=%d H=%d BM=%d" % (what, desc.S, desc.H, BM))
    m = sa()
    pat = m.DevicePatterns.from_host(desc)
    ix = m.build_index(pat, BM, validate=True)
    torch.cuda.synchronize()
    assert int(ix.status.item()) == 0
    got = ix.to_numpy()
    ref = oracle.build_index(desc, BM)
    for k in KEYS:
        np.testing.assert_array_equal(np.asarray(got[k]).astype(np.int64), np.asarray(ref[k]).astype(np.int64),
                                      err_msg="%s: %s" % (what, k))


@pytest.mark.parametrize("variant", ["base", "dense_causal", "all_ones", "diag0"])
@pytest.mark.parametrize("BM", [64, 128])
def test_index_tiny(variant, BM):
    _compare(W.tiny(variant), BM, "tiny-" + variant)


@pytest.mark.parametrize("S,BM", [(8192, 64), (8192, 128), (1000, 64), (777, 128)])
def test_index_llama1b_like(S, BM):
    _compare(W.llama1b_like(S=S), BM, "1b-like")


def test_index_capture_extension():
    maps = W.capture_maps(layers=1, heads=32, n_avg=16)
    c = oracle.capture(maps)
    diags, verts = oracle.extend(c["keep_diag"], c["keep_vert"], 16384)
    _compare(W.desc_from_lists(16384, diags, verts), 64, "capture-ext")


@pytest.mark.parametrize("S", [65536, 4000])
def test_index_llama8b_like(S):
    _compare(W.llama8b_like(S=S), 64, "8b-like")


@pytest.mark.parametrize("S,BM", [(131072, 128), (5000, 128), (5000, 64)])
def test_index_long_stripes(S, BM):
    _compare(W.long_stripes(S=S), BM, "stripes")


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 130])
def test_index_edge_lengths(S):
    rng = np.random.default_rng(S)
    diags = [np.arange(min(3, S)), np.zeros(0), np.array([S - 1]), np.arange(S)]
    verts = [np.zeros(0), rng.choice(S, size=min(S, 3), replace=False), np.array([0]), np.arange(S)]
    for BM in (64, 128):
        _compare(W.desc_from_lists(S, diags, verts), BM, "edge")


def test_index_mixed_all_kinds():
    rng = np.random.default_rng(21)
    S, H = 1500, 4
    diags = [np.unique(np.concatenate([np.arange(rng.integers(1, 200)), rng.choice(S, 6, replace=False)]))
             for _ in range(H)]
    verts = [rng.choice(S, 9, replace=False) for _ in range(H)]
    nbq = -(-S // 128)
    bm = (rng.random((H, nbq, nbq)) < 0.2).astype(np.uint8)
    stripes = [[np.sort(rng.choice(S, size=int(rng.integers(0, 60)), replace=False)) for _ in range(-(-S // 256))]
               for _ in range(H)]
    d = W.desc_from_lists(S, diags, verts, block_mask=bm, block_size=128, stripes=stripes, stripe_rows=256)
    for BM in (64, 128):
        _compare(d, BM, "mixed")


def test_index_rejects_invalid_descriptor():
    m = sa()
    d = W.desc_from_lists(100, [np.array([0, 1])], [np.array([3])])
    bad = m.DevicePatterns.from_host(d)
    bad.diag_off = torch.tensor([1, 0], dtype=torch.int32, device="cuda")   # not increasing
    with pytest.raises(m.SAError) as e:
        m.build_index(bad, 64, validate=True)
    assert e.value.code == -3


def test_index_capacity_overflow_is_reported():
    m = sa()
    d = W.llama1b_like(S=2000, H=2)
    pat = m.DevicePatterns.from_host(d)
    ix = m.build_index(pat, 64)
    torch.cuda.synchronize()
    small = ix.c_struct()
    small.capacity.n_cols = max(0, ix.sizes["n_cols"] - 5)
    sizes = m._Sizes()
    rc = m.lib.sa_build_index(C.byref(pat.c_struct()), C.byref(small), C.byref(sizes), 0,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == -4
    rc = m.lib.sa_build_index(C.byref(pat.c_struct()), C.byref(small), None, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(ix.status.item()) & 1
