"""GPU parity: runtime capture from sampled query rows (sa_sample_scores) and pattern selection
(sa_select_patterns) against the fp64 oracle, and the two-stage per-input pipeline end to end.

Scores are int64 fixed point (2^-32 of one row's mass); against the oracle's fp64 sums they agree
within 1e-5 relative plus 1e-7 absolute (fp32 scores, softmax and partial sums; rounding of each
partial sum to the fixed point).  The selection is exact integer arithmetic, so on the same integer scores it is bit-exact.
The pipeline's keep flags are compared on every pattern whose decision no score within that bound
can change (tests/capture_bounds.py)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from capture_bounds import certain_selection
from gpu_util import assert_close_bf16, note, sa, to_dev

pytestmark = pytest.mark.gpu

UNIT = 4294967296.0
REL, ABS = 1e-5, 1e-7


def _scores_close(got, ref, what):
    g = got.cpu().numpy().astype(np.float64) / UNIT
    err = np.abs(g - ref)
    bad = err > REL * ref + ABS
    assert not bad.any(), "%s: %d scores off, worst %.3g at %.3g" % (what, bad.sum(), err.max(), ref.flat[err.argmax()])


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("band,skip", [(0, False), (16, True)])
def test_sample_scores_vs_oracle(dtype, d, band, skip):
    """S = 700 (ragged), 100 sampled rows from 600 (four chunks, the last one partial), GQA 4:2, batch 2."""
    m = sa()
    B, hq, hkv, S, row0, n = 2, 4, 2, 700, 600, 100
    q, k, _ = W.qkv(81, B, hq, hkv, S, d, dtype)
    skip_cols = (np.random.default_rng(9).random((hq, S)) < 0.2).astype(np.uint8) if skip else None
    note("sample scores %s d=%d band=%d skip=%s" % (dtype, d, band, skip))
    dg, vt, lse = m.sample_scores(to_dev(q), to_dev(k), row0, n, band=band,
                                  skip_cols=None if skip_cols is None else torch.from_numpy(skip_cols).cuda())
    torch.cuda.synchronize()
    rd, rv, rl = oracle.sample_scores(q, k, row0, n, band=band, skip_cols=skip_cols)
    _scores_close(dg, rd, "diag")
    _scores_close(vt, rv, "vert")
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), rl, rtol=0, atol=1e-5)


def test_sample_scores_totals_accumulation_and_lse_reuse():
    m = sa()
    B, hq, hkv, S, d = 1, 2, 1, 1000, 128
    q, k, _ = W.qkv(82, B, hq, hkv, S, d, "bf16")
    qd, kd = to_dev(q), to_dev(k)
    note("sample scores totals / accumulation")
    d1, v1, l1 = m.sample_scores(qd, kd, 900, 100)
    d2, v2, _ = m.sample_scores(qd, kd, 300, 64)
    da, va, _ = m.sample_scores(qd, kd, 900, 100)
    m.sample_scores(qd, kd, 300, 64, scores=(da, va))              # accumulate a second block
    dr, vr, _ = m.sample_scores(qd, kd, 900, 100, row_lse=l1, lse_given=True)
    d_only, none_v, _ = m.sample_scores(qd, kd, 900, 100, families=(True, False))
    none_d, v_only, _ = m.sample_scores(qd, kd, 900, 100, families=(False, True))
    torch.cuda.synchronize()
    assert torch.equal(da, d1 + d2) and torch.equal(va, v1 + v2)  # integer sums: exact
    assert torch.equal(dr, d1) and torch.equal(vr, v1)            # the given LSE is the one computed
    assert none_v is None and none_d is None
    assert torch.equal(d_only, d1) and torch.equal(v_only, v1)    # one family alone: the same sums
    for t in (d1, v1):                                            # 100 rows of mass one each
        tot = t.sum(dim=1).double().cpu().numpy() / UNIT
        assert np.all(np.abs(tot - 100.0) < 1e-4), tot


def _rand_scores(rng, n, S, rows, uncovered):
    x = rng.pareto(1.1, size=(n, S))
    x[:, rng.random(S) < 0.1] = 0.0
    x *= uncovered * rows / x.sum(axis=1, keepdims=True)
    v = oracle.fixed_point(x)
    v[:, 5:40:7] = v[:, 5:6]          # ties
    return v


@pytest.mark.parametrize("alpha", [0.3, 0.8, 0.95, 0.999, 1.0])
@pytest.mark.parametrize("S", [1, 777, 131072])
def test_select_matches_oracle_bit_exact(alpha, S):
    m = sa()
    rng = np.random.default_rng(int(alpha * 1000) + S)
    rows = 64
    v = _rand_scores(rng, 5, S, rows, uncovered=0.6)
    note("select alpha=%g S=%d" % (alpha, S))
    for band in (0, 16):
        got = m.select_patterns(torch.from_numpy(v).cuda(), alpha, rows, band=band)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), oracle.select_patterns(v, alpha, rows, band=band))


def test_select_edge_cases():
    m = sa()
    rng = np.random.default_rng(4)
    rows = 8
    v = _rand_scores(rng, 3, 500, rows, uncovered=0.05)   # 95 % already covered
    for alpha in (0.9, 0.95, 0.96, 1.0):                   # need <= 0, about 0, > 0, and need > all scores
        got = m.select_patterns(torch.from_numpy(v).cuda(), alpha, rows)
        np.testing.assert_array_equal(got.cpu().numpy(), oracle.select_patterns(v, alpha, rows))
    z = np.zeros((2, 300), np.int64)
    got = m.select_patterns(torch.from_numpy(z).cuda(), 0.9, rows, band=5)
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.select_patterns(z, 0.9, rows, band=5))
    big = np.full((2, 4096), (1 << 40) + 12345, np.int64)   # all equal, many bits
    got = m.select_patterns(torch.from_numpy(big).cuda(), 0.5, 1 << 20)
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.select_patterns(big, 0.5, 1 << 20))


@pytest.mark.parametrize("alpha_cols,alpha", [(0.8, 0.9), (0.9, 0.97)])
def test_runtime_capture_pipeline(alpha_cols, alpha):
    """Two-stage per-input capture (columns to alpha_cols, then diagonals on what the columns leave, to
    alpha), then extension, index and attention, against the oracle on EVERY head:
      stage 1  GPU column scores and keep flags vs the oracle's (flags on every decision that no score
               within the error bound can flip);
      stage 2  run on the oracle's stage-1 flags on both sides, so that every head is scored on the same
               uncovered mass: GPU diagonal scores and flags vs the oracle's;
      GPU-only pipeline  its column flags may differ from the oracle's only on decisions the bound calls
               unsure; where they are equal its diagonal flags are compared as in stage 2;
      attention  the index and attention of the oracle's final mask on every head, every row of the first
               and the last row block and 24 seeded rows per head."""
    m = sa()
    B, hq, hkv, S, d, n, band = 1, 8, 2, 4096, 128, 64, 64
    q, k = W.runtime_qk(83, B, hq, hkv, S, d, "bf16")
    _, _, v = W.qkv(83, B, hq, hkv, S, d, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    row0 = S - n
    note("runtime capture pipeline alpha_cols=%g alpha=%g" % (alpha_cols, alpha))
    rkd, rkv, rv, rd = oracle.runtime_capture(q, k, row0, n, alpha_cols, alpha, band)
    assert (rkd.sum(1) > band).all() and (rkv.sum(1) > 0).all()    # both stages keep patterns

    # stage 1 on the GPU
    _, vs, lse = m.sample_scores(qd, kd, row0, n, band=band, families=(False, True))
    keep_v = m.select_patterns(vs, alpha_cols, B * n)
    # stage 2 on the oracle's column flags (both sides score the same uncovered mass on every head)
    ds_o, _, _ = m.sample_scores(qd, kd, row0, n, band=band, skip_cols=torch.from_numpy(rkv).cuda(), row_lse=lse,
                                 lse_given=True, families=(True, False))
    keep_d_o = m.select_patterns(ds_o, alpha, B * n, band=band)
    # the GPU-only pipeline: stage 2 on the GPU's own column flags
    ds, _, _ = m.sample_scores(qd, kd, row0, n, band=band, skip_cols=keep_v, row_lse=lse, lse_given=True,
                               families=(True, False))
    keep_d = m.select_patterns(ds, alpha, B * n, band=band)
    torch.cuda.synchronize()

    _scores_close(vs, rv, "stage-1 column scores")
    _scores_close(ds_o, rd, "stage-2 diagonal scores")
    gv, gd_o, gd = keep_v.cpu().numpy(), keep_d_o.cpu().numpy(), keep_d.cpu().numpy()
    sure_v = certain_selection(rv, REL, ABS, alpha_cols, B * n)
    sure_d = certain_selection(rd, REL, ABS, alpha, B * n, band=band)
    assert sure_v.mean() > 0.99 and sure_d.mean() > 0.95
    np.testing.assert_array_equal(gv[sure_v], rkv[sure_v])          # every head
    np.testing.assert_array_equal(gd_o[sure_d], rkd[sure_d])        # every head
    same_v = [h for h in range(hq) if np.array_equal(gv[h], rkv[h])]
    for h in same_v:
        np.testing.assert_array_equal(gd[h][sure_d[h]], rkd[h][sure_d[h]])
    note("unsure decisions: columns %d, diagonals %d; heads with equal column flags %s"
         % (int((~sure_v).sum()), int((~sure_d).sum()), same_v))

    # attention on the oracle's mask, every head
    desc = W.desc_from_lists(S, [np.nonzero(x)[0] for x in rkd], [np.nonzero(x)[0] for x in rkv])
    ix = m.build_index(m.DevicePatterns.from_host(desc), 64)
    o = m.sparse_attn_prefill(qd, kd, vd, ix)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ix.pair_count.cpu().numpy(), oracle.pair_count(desc))
    rng = np.random.default_rng(5)
    rows = np.array([(0, h, i) for h in range(hq)
                     for i in np.concatenate([np.arange(64), np.arange(S - 64, S), rng.choice(S, 24)])], np.int32)
    ref, _ = oracle.attention_rows(desc, q, k, v, rows)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    got = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
    assert_close_bf16(got, ref, "runtime pipeline attention")


def test_sample_scores_on_a_side_stream():
    """Scores made on another stream than the current one (the zeroed outputs are ordered before the
    accumulating kernel) equal those made on the current stream."""
    m = sa()
    B, hq, hkv, S, d = 1, 4, 2, 1500, 64
    q, k, _ = W.qkv(84, B, hq, hkv, S, d, "bf16")
    qd, kd = to_dev(q), to_dev(k)
    note("sample scores side stream")
    d1, v1, l1 = m.sample_scores(qd, kd, 1400, 100, band=8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda._sleep(20000000)          # the current stream is still busy when the side launch is queued
    d2, v2, l2 = m.sample_scores(qd, kd, 1400, 100, band=8, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(v1, v2) and torch.equal(l1, l2)
    with pytest.raises(ValueError):
        m.sample_scores(qd, kd, 1400, 100, row_lse=torch.zeros(1, hq, 99, device="cuda"), lse_given=True)
