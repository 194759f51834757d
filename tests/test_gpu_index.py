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
    """Both build modes (with and without descriptor validation) against the oracle index."""
    note("index %s S=%d H=%d BM=%d" % (what, desc.S, desc.H, BM))
    m = sa()
    pat = m.DevicePatterns.from_host(desc)
    ref = oracle.build_index(desc, BM)
    for validate in (True, False):
        ix = m.build_index(pat, BM, validate=validate)
        m.refill_index(pat, ix)   # a second build into the same arrays gives the same index
        torch.cuda.synchronize()
        assert int(ix.status.item()) == 0
        got = ix.to_numpy()
        for k in KEYS:
            np.testing.assert_array_equal(np.asarray(got[k]).astype(np.int64), np.asarray(ref[k]).astype(np.int64),
                                          err_msg="%s (validate=%s): %s" % (what, validate, k))


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


@pytest.mark.parametrize("BM", [64, 128])
def test_index_max_length(BM):
    """The longest accepted sequence, every pattern kind, offsets and columns up to S - 1."""
    _compare(W.max_length(), BM, "max-length")


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


@pytest.mark.parametrize("BM", [64, 128])
def test_index_block_only_heads(BM):
    """Heads whose rows hold only block-mask columns: block size 128 over 64-row blocks, a ragged last
    block, rows with no set block below the diagonal, and an all-zero head next to a dense one."""
    rng = np.random.default_rng(31)
    S, H, bs = 2000, 4, 128
    nbq = -(-S // bs)
    bm = np.tril(rng.random((H, nbq, nbq)) < 0.3).astype(np.uint8)
    bm[1] = 0
    bm[2] = np.tril(np.ones((nbq, nbq), np.uint8))
    bm[3, 5] = 0
    d = W.desc_from_lists(S, [np.zeros(0)] * H, [np.zeros(0)] * H, block_mask=bm, block_size=bs)
    _compare(d, BM, "blocks-only")


@pytest.mark.parametrize("BM", [64, 128])
def test_index_stripe_only_heads(BM):
    """Stripe lists longer than the row block: with 256-row stripes, the first row block of a stripe sees
    only the list's columns up to its own last row; empty lists and lists of a single column."""
    rng = np.random.default_rng(32)
    S, H, sr = 3000, 3, 256
    nst = -(-S // sr)
    stripes = []
    for h in range(H):
        per = []
        for t in range(nst):
            top = min(S, (t + 1) * sr) - 1
            k = int(rng.integers(0, 3)) if h == 1 else int(rng.integers(1, top + 2))
            per.append(np.sort(rng.choice(top + 1, size=min(k, top + 1), replace=False)))
        stripes.append(per)
    d = W.desc_from_lists(S, [np.zeros(0)] * H, [np.zeros(0)] * H, stripes=stripes, stripe_rows=sr)
    _compare(d, BM, "stripes-only")


@pytest.mark.parametrize("BM", [64, 128])
def test_index_diagonal_runs_merge(BM):
    """Diagonal runs whose column intervals merge or stay apart by one column, runs clipped at column 0,
    verticals inside and outside the band, and a head with more offsets than fit in LDS."""
    S = 5000
    diags = [np.concatenate([np.arange(0, 10), np.arange(10 + BM, 20 + BM), np.arange(21 + 2 * BM, 30 + 2 * BM),
                             [700, 701, 900]]),
             np.arange(0, S, 3),
             np.arange(S),
             np.array([4999])]
    verts = [np.array([0, 5, 100, 2500, 4999]), np.array([1, 2, 3]), np.arange(0, S, 7), np.zeros(0)]
    d = W.desc_from_lists(S, diags, verts)
    _compare(d, BM, "diag-runs")


@pytest.mark.parametrize("BM", [64, 128])
def test_index_many_diagonals(BM):
    """Heads with more diagonal offsets than one wave stages (the lists path with the offsets staged once per
    workgroup, up to four times as many) and with more than a workgroup stages (the bitmap path): a band plus
    scattered offsets, as runtime-captured masks have, with verticals."""
    S, rng = 16384, np.random.default_rng(61)
    diags = [np.concatenate([np.arange(1024), 1024 + np.sort(rng.choice(S - 1024, 1000, replace=False))]),
             np.sort(rng.choice(S, 3000, replace=False)),
             np.sort(rng.choice(S, 7000, replace=False)),
             np.arange(0, S, 2)]
    verts = [np.sort(rng.choice(S, n, replace=False)) for n in (12, 200, 64, 0)]
    d = W.desc_from_lists(S, diags, verts)
    _compare(d, BM, "many-diagonals")


def test_index_unsorted_stripe_list_stays_in_range():
    """An unsorted stripe list (an invalid descriptor) built without validation: every column the index
    holds is still a valid key column of its row block."""
    m = sa()
    S = 512
    stripes = [[np.array([300, 5, 100]), np.array([1, 2]), np.array([400, 3]), np.array([7])]]
    d = W.desc_from_lists(S, [np.zeros(0)], [np.zeros(0)], stripes=stripes, stripe_rows=128)
    pat = m.DevicePatterns.from_host(d)
    ix = m.build_index(pat, 128)
    torch.cuda.synchronize()
    got = ix.to_numpy()
    for rb in range(4):
        cols = got["col_idx"][got["col_ptr"][rb]:got["col_ptr"][rb + 1]]
        assert np.all((cols >= 0) & (cols <= min(S, 128 * rb + 128) - 1))


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
