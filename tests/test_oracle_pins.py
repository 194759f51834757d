"""Pins for the CPU oracle: it is checked against things other than itself.

* brute-force whole-matrix numpy twins (tests/brute.py) on tiny inputs,
* textbook causal attention (torch scaled_dot_product_attention, fp64, CPU),
* closed forms and special cases (diagonal 0 only -> O = V; V == 1 -> O = 1;
  one-hot V -> softmax rows that sum to one),
* hand-worked examples under tests/golden/ (each with its derivation),
* invariants of pattern capture (monotone threshold, hit-count totals) and the
  textbook Box-Cox formula (x^lambda - 1) / lambda,
* planted-pattern maps whose kept sets are known in advance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from brute import attention_brute, index_brute, mask_matrix
from golden.load import arr, load


def widen64(x):
    """float32 or bf16 bit patterns -> float64 values."""
    return W.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _rand_desc(rng, S, H, kinds):
    diags, verts = [], []
    for _ in range(H):
        d = set()
        if "diag" in kinds:
            w = int(rng.integers(1, max(2, S // 4)))
            d.update(range(w))
            d.update(int(x) for x in rng.choice(S, size=min(S, int(rng.integers(0, 5))), replace=False))
        diags.append(np.array(sorted(d), dtype=np.int32))
        v = set()
        if "vert" in kinds:
            v.update(int(x) for x in rng.choice(S, size=min(S, int(rng.integers(0, 7))), replace=False))
        verts.append(np.array(sorted(v), dtype=np.int32))
    bm = None
    if "block" in kinds:
        nbq = -(-S // 32)
        bm = (rng.random((H, nbq, nbq)) < 0.3).astype(np.uint8)
    stripes = None
    if "stripe" in kinds:
        nst = -(-S // 32)
        stripes = [[np.sort(rng.choice(S, size=int(rng.integers(0, S // 3 + 1)), replace=False)) for _ in range(nst)]
                   for _ in range(H)]
    return W.desc_from_lists(S, diags, verts, block_mask=bm, block_size=32, stripes=stripes, stripe_rows=32)


KINDS = [("diag",), ("vert",), ("block",), ("stripe",), ("diag", "vert"), ("diag", "vert", "block"),
         ("diag", "stripe"), ("diag", "vert", "block", "stripe")]


# ----------------------------------------------------------------------------- masks and counts
@pytest.mark.parametrize("kinds", KINDS)
@pytest.mark.parametrize("S", [1, 7, 37, 64])
def test_row_mask_matches_brute_force(kinds, S):
    rng = np.random.default_rng([S, len(kinds)])
    d = _rand_desc(rng, S, 2, kinds)
    for h in range(2):
        m = mask_matrix(d, h)
        for i in range(S):
            np.testing.assert_array_equal(oracle.row_mask(d, h, i).astype(bool), m[i, :i + 1])
        assert oracle.pair_count(d)[h] == m.sum()


def test_pair_count_matches_row_masks_mid_size():
    rng = np.random.default_rng(7)
    d = _rand_desc(rng, 300, 3, ("diag", "vert", "block", "stripe"))
    pc = oracle.pair_count(d)
    for h in range(3):
        assert pc[h] == sum(int(oracle.row_mask(d, h, i).sum()) for i in range(300))


# ----------------------------------------------------------------------------- index
def test_index_hand_worked_example():
    g = load("index_example.txt")
    d = W.desc_from_lists(int(arr(g, "S")[0]), [arr(g, "diag")], [arr(g, "vert")])
    ix = oracle.build_index(d, int(arr(g, "row_block")[0]))
    for key in ("run_ptr", "run_lo", "run_hi", "seg_ptr", "seg_lo", "seg_hi", "bcol_ptr", "bcol_idx", "col_ptr",
                "col_idx", "pair_count"):
        np.testing.assert_array_equal(np.atleast_1d(ix[key]), np.atleast_1d(arr(g, key)), err_msg=key)


@pytest.mark.parametrize("kinds", KINDS)
@pytest.mark.parametrize("S,BM", [(37, 16), (64, 16), (100, 32), (129, 32)])
def test_index_matches_enumeration(kinds, S, BM):
    rng = np.random.default_rng([S, BM, len(kinds), 1])
    d = _rand_desc(rng, S, 2, kinds)
    ix = oracle.build_index(d, BM)
    br = index_brute(d, BM)
    for key in br:
        np.testing.assert_array_equal(np.asarray(ix[key]).astype(np.int64), br[key].astype(np.int64), err_msg=key)


def _expand(d, ix, h):
    """Pairs the two kernel phases would compute, from the index alone (counts per pair)."""
    S, BM, nb = d.S, ix["row_block"], ix["n_row_blocks"]
    offs = set(int(x) for x in d.diags(h))
    cnt = np.zeros((S, S), dtype=np.int32)
    for rb in range(nb):
        b0, b1 = rb * BM, min(S, (rb + 1) * BM) - 1
        it = h * nb + rb
        bset = set(ix["bcol_idx"][ix["bcol_ptr"][it]:ix["bcol_ptr"][it + 1]].tolist())
        for s in range(ix["seg_ptr"][it], ix["seg_ptr"][it + 1]):
            for j in range(ix["seg_lo"][s], ix["seg_hi"][s] + 1):
                for i in range(max(j, b0), b1 + 1):
                    if (i - j) in offs or j in bset:
                        cnt[i, j] += 1
        for j in ix["col_idx"][ix["col_ptr"][it]:ix["col_ptr"][it + 1]]:
            for i in range(max(j, b0), b1 + 1):
                cnt[i, j] += 1
    return cnt


@pytest.mark.parametrize("kinds", [("diag", "vert"), ("diag", "vert", "block"), ("diag", "stripe"),
                                   ("diag", "vert", "block", "stripe")])
def test_index_phases_cover_each_retained_pair_once(kinds):
    rng = np.random.default_rng([11, len(kinds)])
    d = _rand_desc(rng, 150, 2, kinds)
    ix = oracle.build_index(d, 32)
    for h in range(2):
        cnt = _expand(d, ix, h)
        m = mask_matrix(d, h)
        assert cnt.max() <= 1
        np.testing.assert_array_equal(cnt.astype(bool), m)
        assert ix["pair_count"][h] == m.sum()


def test_index_rejects_row_block_across_block_rows():
    rng = np.random.default_rng(12)
    d = _rand_desc(rng, 100, 1, ("block",))
    with pytest.raises(ValueError):
        oracle.build_index(d, 64)


# ----------------------------------------------------------------------------- attention
def _f64(x):
    return W.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _all_rows(B, H, S):
    return np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S)], dtype=np.int32)


@pytest.mark.parametrize("kinds", KINDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_matches_brute_force(kinds, dtype):
    S, B, hq, hkv, dh = 48, 2, 4, 2, 16
    rng = np.random.default_rng([3, len(kinds)])
    d = _rand_desc(rng, S, hq, kinds)
    q, k, v = W.qkv(99, B, hq, hkv, S, dh, dtype, seed_extra=len(kinds))
    rows = _all_rows(B, hq, S)
    for mode in (0, 1):
        o, lse = oracle.attention_rows(d, q, k, v, rows, mode=mode)
        ob, lb = attention_brute(d, _f64(q), _f64(k), _f64(v))
        np.testing.assert_allclose(o, ob.reshape(-1, dh), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lb.reshape(-1), rtol=0, atol=1e-12)


def test_attention_custom_scale_and_gqa_mapping():
    S, B, hq, hkv, dh = 40, 1, 6, 3, 8
    rng = np.random.default_rng(5)
    d = _rand_desc(rng, S, hq, ("diag", "vert"))
    q, k, v = W.qkv(98, B, hq, hkv, S, dh, "f32")
    o, lse = oracle.attention_rows(d, q, k, v, _all_rows(B, hq, S), scale=0.37)
    ob, lb = attention_brute(d, _f64(q), _f64(k), _f64(v), scale=0.37)
    np.testing.assert_allclose(o, ob.reshape(-1, dh), atol=1e-12)
    np.testing.assert_allclose(lse, lb.reshape(-1), atol=1e-12)


@pytest.mark.parametrize("variant", ["dense_causal", "all_ones"])
def test_full_mask_is_textbook_causal_attention(variant):
    S, dh = 96, 32
    d = W.tiny(variant, S=S)
    q, k, v = W.qkv(97, 1, 1, 1, S, dh, "f32")
    o, lse = oracle.attention_rows(d, q, k, v, _all_rows(1, 1, S))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64)), is_causal=True)
    np.testing.assert_allclose(o, ref.numpy().reshape(-1, dh), atol=1e-12)
    s = (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T) / np.sqrt(dh)
    s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_diagonal_zero_only_returns_v_exactly(dtype):
    S, dh = 70, 16
    d = W.tiny("diag0", S=S)
    q, k, v = W.qkv(96, 1, 1, 1, S, dh, dtype)
    o, _ = oracle.attention_rows(d, q, k, v, _all_rows(1, 1, S))
    np.testing.assert_array_equal(o, _f64(v)[0, 0])


def test_constant_v_gives_ones_and_one_hot_v_gives_unit_rows():
    S, dh = 64, 64
    rng = np.random.default_rng(8)
    d = _rand_desc(rng, S, 1, ("diag", "vert", "block"))
    q, k, _ = W.qkv(95, 1, 1, 1, S, dh, "f32")
    ones = np.ones((1, 1, S, dh), np.float32)
    o, _ = oracle.attention_rows(d, q, k, ones, _all_rows(1, 1, S))
    nonempty = mask_matrix(d, 0).any(axis=1)
    np.testing.assert_allclose(o[nonempty], 1.0, atol=1e-14)
    eye = np.eye(S, dh, dtype=np.float32)[None, None]
    p, _ = oracle.attention_rows(d, q, k, eye, _all_rows(1, 1, S))
    np.testing.assert_allclose(p[nonempty].sum(axis=1), 1.0, atol=1e-14)
    m = mask_matrix(d, 0)
    assert np.all(p[~m[:, :dh]] == 0.0)


def test_empty_rows_give_zero_output_and_minus_inf_lse():
    S, dh = 20, 8
    d = W.desc_from_lists(S, [np.zeros(0)], [np.array([5])])
    q, k, v = W.qkv(94, 1, 1, 1, S, dh, "f32")
    o, lse = oracle.attention_rows(d, q, k, v, _all_rows(1, 1, S))
    assert np.all(o[:5] == 0) and np.all(np.isneginf(lse[:5]))
    np.testing.assert_array_equal(o[5:], np.repeat(v[0, 0, 5:6].astype(np.float64), S - 5, axis=0))


def test_band_and_column_encodings_agree():
    S, dh = 128, 16
    q, k, v = W.qkv(93, 1, 1, 1, S, dh, "bf16")
    a, la = oracle.attention_rows(W.tiny("dense_causal", S), q, k, v, _all_rows(1, 1, S))
    b, lb = oracle.attention_rows(W.tiny("all_ones", S), q, k, v, _all_rows(1, 1, S))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ----------------------------------------------------------------------------- capture
def test_capture_hand_worked_example():
    g = load("capture_example.txt")
    L = int(arr(g, "L")[0])
    maps = arr(g, "map_row", np.float32).reshape(1, L, L)
    for scope in (0, 1):
        c = oracle.capture(maps, norm_scope=scope, want_mask=True)
        np.testing.assert_array_equal(c["true_mask"][0], arr(g, "true_mask_row"))
        np.testing.assert_array_equal(c["diag_hits"][0], arr(g, "diag_hits"))
        np.testing.assert_array_equal(c["vert_hits"][0], arr(g, "vert_hits"))
        np.testing.assert_array_equal(c["keep_diag"][0], arr(g, "keep_diag"))
        np.testing.assert_array_equal(c["keep_vert"][0], arr(g, "keep_vert"))


def test_capture_true_mask_follows_textbook_boxcox():
    """M agrees with (x^lambda - 1)/lambda (numpy power), min-max per row, >= tau,
    except on cells within rounding distance of the threshold."""
    maps = W.capture_maps(layers=1, heads=3, L=128, n_avg=4)
    c = oracle.capture(maps, want_mask=True)
    lam, eps, tau = 0.5, 1e-8, 0.3
    for n in range(maps.shape[0]):
        for i in range(128):
            x = maps[n, i, :i + 1].astype(np.float64) + eps
            y = (np.power(x, lam) - 1.0) / lam
            if y.max() == y.min():
                t = np.ones_like(y)
            else:
                t = (y - y.min()) / (y.max() - y.min())
            sure = np.abs(t - tau) > 1e-12
            np.testing.assert_array_equal(c["true_mask"][n, i, :i + 1][sure], (t >= tau)[sure])
            assert not c["true_mask"][n, i, i + 1:].any()


def test_capture_invariants_monotone_rows_and_hit_totals():
    maps = W.capture_maps(layers=1, heads=2, L=64, n_avg=2)
    for scope in (0, 1):
        c = oracle.capture(maps, norm_scope=scope, want_mask=True)
        for n in range(maps.shape[0]):
            M = c["true_mask"][n]
            assert c["diag_hits"][n].sum() == M.sum() == c["vert_hits"][n].sum()
            for i in range(64):
                row, a = M[i, :i + 1].astype(bool), maps[n, i, :i + 1]
                if row.any() and (~row).any():
                    assert a[row].min() > a[~row].max()   # M is an up-set in A within a row
            L = 64
            r = np.arange(L)
            np.testing.assert_array_equal(c["keep_diag"][n], (c["diag_hits"][n] / (L - r) >= 0.8).astype(np.uint8))
            np.testing.assert_array_equal(c["keep_vert"][n], (c["vert_hits"][n] / (L - r) >= 0.8).astype(np.uint8))


@pytest.mark.parametrize("scope", [0, 1])
def test_capture_planted_patterns(scope):
    L = 48
    A = np.full((L, L), 1e-4, dtype=np.float64)
    for i in range(L):
        A[i, i] += 0.5
        if i >= 5:
            A[i, i - 5] += 0.3
        if i >= 2:
            A[i, 2] += 0.15
    A = np.tril(A).astype(np.float32)[None]
    c = oracle.capture(A, norm_scope=scope)
    assert sorted(np.nonzero(c["keep_diag"][0])[0].tolist()) == [0, 5]
    assert sorted(np.nonzero(c["keep_vert"][0])[0].tolist()) == [2, L - 1]


def test_capture_rejects_bad_lambda():
    with pytest.raises(ValueError):
        oracle.capture(np.ones((1, 4, 4), np.float32), lam=float("nan"))
    with pytest.raises(ValueError):
        oracle.capture(np.ones((1, 4, 4), np.float32), lam=0.0, eps=0.0)   # log 0
    with pytest.raises(ValueError):
        oracle.capture_scores(np.ones((1, 4, 4), np.float32), lam=-1.0, eps=0.0)


def _minmax_rows(y, scope):
    """Min-max scaling of the causal cells of y [L, L] (NaN above the diagonal): per row or per map."""
    L = y.shape[0]
    t = np.full_like(y, np.nan)
    if scope == 1:
        lo, hi = np.nanmin(y), np.nanmax(y)
    for i in range(L):
        r = y[i, :i + 1]
        if scope == 0:
            lo, hi = r.min(), r.max()
        t[i, :i + 1] = 1.0 if hi == lo else (r - lo) / (hi - lo)
    return t


@pytest.mark.parametrize("lam", [-0.5, 0.0, 0.25, 0.5, 1.0, 2.0])
@pytest.mark.parametrize("scope", [0, 1])
def test_capture_scores_follow_scipy_boxcox(lam, scope):
    """t = min-max of scipy.special.boxcox(A + eps, lambda) over the causal row (or map)."""
    from scipy.special import boxcox
    maps = W.capture_maps(layers=1, heads=2, L=96, n_avg=2, layer_offset=5)
    t = oracle.capture_scores(maps, lam=lam, eps=1e-8, norm_scope=scope)
    L = 96
    for n in range(2):
        y = np.where(np.tri(L, dtype=bool), boxcox(maps[n].astype(np.float64) + 1e-8, lam), np.nan)
        ref = _minmax_rows(y, scope)
        np.testing.assert_allclose(t[n], ref, rtol=0, atol=1e-11, equal_nan=True)


def test_capture_scores_linear_case_and_mask():
    """lambda = 1 makes y = A + eps - 1, so t is the min-max of A itself; M = (t >= tau) cell by cell."""
    maps = W.capture_maps(layers=1, heads=2, L=80, n_avg=3, layer_offset=9)
    L = 80
    t = oracle.capture_scores(maps, lam=1.0, eps=1e-10)
    c = oracle.capture(maps, lam=1.0, eps=1e-10, tau=0.2, want_mask=True)
    for n in range(2):
        a = np.where(np.tri(L, dtype=bool), maps[n].astype(np.float64), np.nan)
        np.testing.assert_allclose(t[n], _minmax_rows(a, 0), rtol=0, atol=1e-12, equal_nan=True)
        tri = np.tri(L, dtype=bool)
        np.testing.assert_array_equal(c["true_mask"][n][tri], (t[n][tri] >= 0.2).astype(np.uint8))


@pytest.mark.parametrize("lam", [0.0, 0.25, 1.0])
def test_capture_keep_sets_shrink_as_tau_and_mu_grow(lam):
    """A higher tau removes cells from M, a higher mu asks more of each pattern: kept sets can only shrink."""
    maps = W.capture_maps(layers=1, heads=4, L=128, n_avg=4, layer_offset=11)
    prev = None
    for tau in (0.1, 0.2, 0.3, 0.4, 0.5):
        c = oracle.capture(maps, lam=lam, tau=tau)
        if prev is not None:
            assert not (c["keep_diag"] & ~prev["keep_diag"]).any() and not (c["keep_vert"] & ~prev["keep_vert"]).any()
        prev = c
    prev = None
    for mu in (0.6, 0.7, 0.8, 0.9, 1.0):
        c = oracle.capture(maps, lam=lam, mu=mu)
        if prev is not None:
            assert not (c["keep_diag"] & ~prev["keep_diag"]).any() and not (c["keep_vert"] & ~prev["keep_vert"]).any()
        prev = c


def test_coverage_brute_force_and_special_cases():
    maps = W.capture_maps(layers=1, heads=3, L=70, n_avg=2, layer_offset=13)
    L = 70
    rng = np.random.default_rng(5)
    kd = (rng.random((3, L)) < 0.1).astype(np.uint8)
    kv = (rng.random((3, L)) < 0.1).astype(np.uint8)
    mass, cells = oracle.coverage(maps, kd, kv)
    i, j = np.tril_indices(L)
    for n in range(3):
        on = (kd[n][i - j] | kv[n][j]).astype(bool)
        a = maps[n][i, j].astype(np.float64)
        assert cells[n] == on.sum()
        assert abs(mass[n] - a[on].sum() / a.sum()) < 1e-12
    ones, zeros = np.ones((3, L), np.uint8), np.zeros((3, L), np.uint8)
    m1, c1 = oracle.coverage(maps, ones, zeros)                 # every diagonal: the whole causal window
    assert np.all(c1 == L * (L + 1) // 2) and np.allclose(m1, 1.0, rtol=0, atol=1e-12)
    d0 = zeros.copy()
    d0[:, 0] = 1
    m0, c0 = oracle.coverage(maps, d0, zeros)                   # diagonal 0 only: the trace share
    for n in range(3):
        assert c0[n] == L
        assert abs(m0[n] - np.trace(maps[n].astype(np.float64)) / np.tril(maps[n].astype(np.float64)).sum()) < 1e-12


def test_extension_restricted_to_capture_window_is_the_kept_union():
    maps = W.capture_maps(layers=1, heads=2, L=64, n_avg=4)
    c = oracle.capture(maps)
    diags, verts = oracle.extend(c["keep_diag"], c["keep_vert"], S=200)
    d = W.desc_from_lists(200, diags, verts)
    for h in range(2):
        kd, kv = c["keep_diag"][h].astype(bool), c["keep_vert"][h].astype(bool)
        for i in range(64):
            j = np.arange(i + 1)
            expect = kd[i - j] | kv[j]
            np.testing.assert_array_equal(oracle.row_mask(d, h, i).astype(bool), expect)


# ------------------------------------------------------------------ decode form (explicit query vectors)
def test_query_form_equals_row_form_on_q_rows():
    """Row n of attention_queries with qrows[n] = Q[b, h, i] is, bit for bit, row (b, h, i) of attention_rows."""
    rng = np.random.default_rng(41)
    d = _rand_desc(rng, 48, 4, ("diag", "vert", "block", "stripe"))
    q, k, v = W.qkv(41, 2, 4, 2, 48, 16, "bf16")
    rows = np.array([(b, h, i) for b in range(2) for h in range(4) for i in (0, 7, 31, 47)], np.int32)
    o1, l1 = oracle.attention_rows(d, q, k, v, rows)
    o2, l2 = oracle.attention_queries(d, np.stack([q[b, h, i] for b, h, i in rows]), k, v, rows)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_query_form_full_mask_is_textbook_single_query_attention():
    """With every causal key retained, a query vector at position t is softmax(q K[:t+1]^T / sqrt(d)) V[:t+1]."""
    S, dh = 80, 32
    d = W.tiny("all_ones", S=S)
    _, k, v = W.qkv(42, 1, 1, 1, S, dh, "f32")
    qv = np.random.default_rng(42).standard_normal((5, dh)).astype(np.float32)
    ts = [0, 1, 17, 50, 79]
    o, lse = oracle.attention_queries(d, qv, k, v, np.array([(0, 0, t) for t in ts], np.int32))
    for n, t in enumerate(ts):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qv[n:n + 1].astype(np.float64))[None, None],
            torch.from_numpy(k[0, 0, :t + 1].astype(np.float64))[None, None],
            torch.from_numpy(v[0, 0, :t + 1].astype(np.float64))[None, None])
        np.testing.assert_allclose(o[n], ref.numpy().reshape(dh), atol=1e-12)
        s = (k[0, 0, :t + 1].astype(np.float64) @ qv[n].astype(np.float64)) / np.sqrt(dh)
        np.testing.assert_allclose(lse[n], np.log(np.exp(s).sum()), atol=1e-12)


def test_query_form_diagonal_zero_returns_the_cache_row():
    """D = {0} only: the query at position t sees key t alone, so the output is V[t] exactly."""
    S, dh = 40, 16
    d = W.tiny("diag0", S=S)
    _, k, v = W.qkv(43, 1, 1, 1, S, dh, "bf16")
    qv = W.bf16_bits(np.random.default_rng(43).standard_normal((3, dh)).astype(np.float32))
    ts = [0, 9, 39]
    o, _ = oracle.attention_queries(d, qv, k, v, np.array([(0, 0, t) for t in ts], np.int32))
    for n, t in enumerate(ts):
        assert np.array_equal(o[n], W.bf16_bits_to_f32(v[0, 0, t]).astype(np.float64))


# ------------------------------------------------------------------ averaged attention maps (capture input)
def test_attention_maps_rows_sum_to_one_and_zero_above_diagonal():
    q, k, _ = W.qkv(51, 3, 4, 2, 40, 16, "bf16")
    m = oracle.attention_maps(q, k)
    np.testing.assert_allclose(m.sum(axis=2), 1.0, atol=1e-12)
    assert np.all(m[:, np.triu_indices(40, 1)[0], np.triu_indices(40, 1)[1]] == 0.0)


def test_attention_maps_equal_keys_give_uniform_rows():
    """Every key equal: each causal row is uniform, 1 / (i + 1), whatever the queries."""
    q, _, _ = W.qkv(52, 2, 2, 1, 30, 8, "f32")
    k = np.tile(np.random.default_rng(52).standard_normal((1, 1, 1, 8)).astype(np.float32), (2, 1, 30, 1))
    m = oracle.attention_maps(q, k)
    i = np.arange(30)
    expect = np.where(i[None, :] <= i[:, None], 1.0 / (i[:, None] + 1.0), 0.0)
    np.testing.assert_allclose(m, np.broadcast_to(expect, m.shape), atol=1e-14)


def test_attention_maps_match_torch_softmax_average():
    q, k, _ = W.qkv(53, 3, 4, 2, 33, 16, "f32")
    m = oracle.attention_maps(q, k, scale=0.3)
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(np.repeat(k, 2, axis=1).astype(np.float64))
    s = (qt @ kt.transpose(-1, -2)) * 0.3
    s = s.masked_fill(~torch.tril(torch.ones(33, 33, dtype=torch.bool)), float("-inf"))
    ref = torch.softmax(s, dim=-1).mean(dim=0).numpy()
    np.testing.assert_allclose(m, ref, atol=1e-13)


# ---------------------------------------------------------------------------
# runtime capture: sampled-row scores and pattern selection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,band,skip", [("f32", 0, False), ("bf16", 0, False), ("f32", 7, True)])
def test_sample_scores_brute_force(dtype, band, skip):
    """Numpy twin: softmax of the sampled rows over j <= i, mass added per diagonal i - j and per
    column j for the pairs with i - j >= band whose column is not skipped."""
    B, hq, hkv, S, d, row0, n = 2, 4, 2, 40, 16, 25, 10
    q, k, _ = W.qkv(61, B, hq, hkv, S, d, dtype)
    skip_cols = (np.random.default_rng(6).random((hq, S)) < 0.3).astype(np.uint8) if skip else None
    diag, vert, lse = oracle.sample_scores(q, k, row0, n, band=band, skip_cols=skip_cols)
    qf, kf = widen64(q), widen64(k)
    rd = np.zeros((hq, S))
    rv = np.zeros((hq, S))
    rl = np.zeros((B, hq, n))
    for b in range(B):
        for h in range(hq):
            g = h // (hq // hkv)
            for x in range(n):
                i = row0 + x
                s = kf[b, g, :i + 1] @ qf[b, h, i] / np.sqrt(d)
                rl[b, h, x] = np.log(np.exp(s - s.max()).sum()) + s.max()
                p = np.exp(s - s.max())
                p /= p.sum()
                j = np.arange(i + 1)
                out = i - j >= band
                if skip:
                    out &= skip_cols[h][j] == 0
                np.add.at(rd[h], (i - j)[out], p[out])
                np.add.at(rv[h], j[out], p[out])
    np.testing.assert_allclose(diag, rd, rtol=0, atol=1e-12)
    np.testing.assert_allclose(vert, rv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_sample_scores_totals_and_support():
    B, hq, hkv, S, d, row0, n = 3, 2, 1, 64, 8, 10, 20
    q, k, _ = W.qkv(62, B, hq, hkv, S, d, "f32")
    diag, vert, _ = oracle.sample_scores(q, k, row0, n, scale=0.7)
    np.testing.assert_allclose(diag.sum(1), B * n, rtol=1e-13)
    np.testing.assert_allclose(vert.sum(1), B * n, rtol=1e-13)
    last = row0 + n - 1
    assert not diag[:, last + 1:].any() and not vert[:, last + 1:].any()
    assert (diag[:, :last + 1] > 0).all() and (vert[:, :last + 1] > 0).all()
    d0, v0, l0 = oracle.sample_scores(q, k, 0, 1)          # row 0 sees key 0 only
    assert np.all(d0[:, 0] == B) and np.all(v0[:, 0] == B) and not d0[:, 1:].any()
    # the window's mass leaves both families; skipped columns leave both too
    db, vb, _ = oracle.sample_scores(q, k, row0, n, band=5, scale=0.7)
    assert not db[:, :5].any()
    np.testing.assert_allclose(db.sum(1), diag[:, 5:].sum(1), rtol=1e-13)
    np.testing.assert_allclose(vb.sum(1), db.sum(1), rtol=1e-13)
    sk = np.zeros((hq, S), np.uint8)
    sk[:, 3] = 1
    ds, vs, _ = oracle.sample_scores(q, k, row0, n, skip_cols=sk, scale=0.7)
    assert not vs[:, 3].any()
    np.testing.assert_allclose(vs.sum(1), vert.sum(1) - vert[:, 3], rtol=1e-13)


def _select_brute(v, alpha, rows, band=0):
    t_all = rows * (1 << 32)
    need = int(np.ceil(alpha * float(t_all))) - (t_all - int(v.sum()))
    keep = np.zeros(v.shape, np.uint8)
    if need > 0:
        run, theta = 0, 1
        for x in sorted(v.tolist(), reverse=True):
            run += x
            if run >= need:
                theta = x
                break
        keep = ((v >= theta) & (v > 0)).astype(np.uint8)
    keep[:band] = 1
    return keep


@pytest.mark.parametrize("alpha", [0.05, 0.5, 0.9, 0.97, 1.0])
def test_select_patterns_brute_force(alpha):
    rng = np.random.default_rng(int(alpha * 1000))
    n, S, rows = 3, 50, 4
    unit = 1 << 32
    a = rng.choice([0, 1, 2, 5, 5, 40, 300, unit // 8, unit // 8], size=(n, S)).astype(np.int64)   # many ties
    b = rng.integers(0, unit // 16, size=(n, S)).astype(np.int64)
    b[:, ::3] = 0
    for v, band in ((a, 4), (b, 0)):
        got = oracle.select_patterns(v, alpha, rows, band=band)
        for h in range(n):
            np.testing.assert_array_equal(got[h], _select_brute(v[h], alpha, rows, band), err_msg=str(h))


def test_select_patterns_special_cases():
    n, S = 2, 30
    unit = 1 << 32
    v = np.zeros((n, S), np.int64)
    v[:, 7] = unit // 2
    v[:, 9] = unit // 4
    v[:, 11] = unit // 4            # uncovered mass = 1 row: nothing covered yet
    k = oracle.select_patterns(v, 0.5, 1)
    assert k[:, 7].all() and k.sum() == n                       # the top pattern alone reaches half
    k = oracle.select_patterns(v, 0.6, 1)
    assert k[:, [7, 9, 11]].all() and k.sum() == 3 * n          # a tie at the threshold keeps both
    k = oracle.select_patterns(v, 0.2, 4, band=3)               # 3 of 4 rows already covered: need < 0
    assert k[:, :3].all() and k.sum() == 3 * n
    k = oracle.select_patterns(v, 1.0, 2)                       # more than the scores hold: all with mass
    np.testing.assert_array_equal(k, (v > 0).astype(np.uint8))
    np.testing.assert_array_equal(oracle.select_patterns(np.zeros((n, S), np.int64), 0.9, 1), 0)


def test_runtime_capture_covers_alpha_of_the_sampled_mass():
    """After both stages the window, kept columns and kept diagonals hold at least alpha of every
    head's sampled mass (to the fixed-point rounding), measured by a numpy softmax of the rows."""
    B, hq, hkv, S, d, n, band = 1, 4, 2, 512, 128, 32, 16
    q, k = W.runtime_qk(63, B, hq, hkv, S, d, "f32")
    for alpha_cols, alpha in ((0.5, 0.8), (0.8, 0.95), (0.95, 0.95)):
        kd, kv, _, _ = oracle.runtime_capture(q, k, S - n, n, alpha_cols, alpha, band)
        qf, kf = widen64(q), widen64(k)
        for h in range(hq):
            g = h // (hq // hkv)
            cov = 0.0
            for i in range(S - n, S):
                s = kf[0, g, :i + 1] @ qf[0, h, i] / np.sqrt(d)
                p = np.exp(s - s.max())
                p /= p.sum()
                j = np.arange(i + 1)
                cov += p[(i - j < band) | (kd[h][i - j] == 1) | (kv[h][j] == 1)].sum()
            assert cov / n >= alpha - 1e-6, (alpha, h, cov / n)
        assert kd.sum() < hq * S and kv.sum() < hq * S
        if alpha_cols < alpha:
            assert (kd.sum(1) > band).any()          # the diagonals close the gap
