"""GPU parity: sa_pattern_capture and sa_patterns_to_desc vs the oracle, bit for bit;
capture -> extension -> index -> attention end to end vs the oracle pipeline."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from golden.load import arr, load
from gpu_util import assert_close_bf16, note, rows_of_blocks, sa, to_dev, workload3_maps

pytestmark = pytest.mark.gpu


def _capture_both(maps, **kw):
    m = sa()
    got = m.pattern_capture(torch.from_numpy(maps).cuda(), return_hits=True, return_mask=True, **kw)
    torch.cuda.synchronize()
    ref = oracle.capture(maps, want_mask=True, **kw)
    for key in ("keep_diag", "keep_vert", "diag_hits", "vert_hits", "true_mask"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    return got, ref


def test_capture_golden_example():
    g = load("capture_example.txt")
    L = int(arr(g, "L")[0])
    maps = arr(g, "map_row", np.float32).reshape(1, L, L)
    for scope in (0, 1):
        got, _ = _capture_both(maps, norm_scope=scope)
        np.testing.assert_array_equal(got["keep_diag"][0].cpu().numpy(), arr(g, "keep_diag"))
        np.testing.assert_array_equal(got["keep_vert"][0].cpu().numpy(), arr(g, "keep_vert"))


@pytest.mark.parametrize("scope", [0, 1])
def test_capture_workload_all_512_maps(scope):
    """The whole capture workload: 16 layers x 32 heads of 512 x 512 maps at n_avg = 16, in one call,
    keep flags, hit counts and the true mask bit for bit."""
    note("capture all 512 workload maps scope=%d" % scope)
    got, ref = _capture_both(workload3_maps(), norm_scope=scope)
    kept = ref["keep_diag"].sum() + ref["keep_vert"].sum()
    assert kept > 0
    note("kept patterns: %d diagonals, %d verticals over 512 maps"
         % (int(ref["keep_diag"].sum()), int(ref["keep_vert"].sum())))


@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("eps", [1e-10])
def test_capture_workload_maps(scope, eps):
    note("capture scope=%d eps=%g" % (scope, eps))
    maps = W.capture_maps(layers=2, heads=32, n_avg=16)
    _capture_both(maps, norm_scope=scope, eps=eps)


@pytest.mark.parametrize("L", [1, 4, 5, 12, 64, 100, 300, 333, 508, 1024])
def test_capture_odd_sizes(L):
    """Sizes on both kernels: L % 4 == 0 and L <= 512 take the single-read tiled kernel (4, 12, 100, 300 and
    508 end in a partial chunk of rows), the others the three-pass kernel."""
    rng = np.random.default_rng(L)
    A = rng.random((3, L, L)).astype(np.float32)
    A = np.tril(A) / np.maximum(1, np.tril(A).sum(axis=2, keepdims=True))
    _capture_both(A.astype(np.float32))


def _edge_maps(L=96):
    """Rows that take each decision path of the capture kernel: ordinary rows, zeros and -0.0, entries in
    [-eps, 0) (per-element path), constant rows, rows of two values, rows whose values differ by one ulp,
    and values from 1e-30 to 1."""
    rng = np.random.default_rng(97)
    A = np.tril(rng.random((4, L, L))).astype(np.float32)
    A[0, 10, :11] = 0.25                                      # constant row
    A[0, 11, :12] = np.where(np.arange(12) % 2, 0.5, 0.0)     # two values
    A[0, 20, :21] = -0.0                                      # constant -0.0
    A[0, 21, :22] = 0.0
    A[0, 21, 5] = -0.0
    A[0, 30, :31] = np.nextafter(np.float32(0.3), np.float32(1.0))
    A[0, 30, 7] = np.float32(0.3)                             # one ulp apart
    A[1] = np.tril(np.float32(10.0) ** rng.uniform(-30, 0, (L, L)).astype(np.float32))
    A[2, 40, :41] = rng.uniform(-5e-9, 1e-9, 41).astype(np.float32)   # A + eps >= 0 with eps = 1e-8
    A[2, 41, :42] = np.float32(-5e-9)
    A[3] = np.tril(np.round(rng.random((L, L)) * 3) / 3).astype(np.float32)   # few distinct values
    return A


@pytest.mark.parametrize("tau", [-0.5, 0.0, 0.3, 1.0, 1.5])
@pytest.mark.parametrize("scope", [0, 1])
def test_capture_edge_rows(tau, scope):
    """Bit-exact against the oracle on rows that take every path (per-row thresholds at lambda = 0.5, the
    per-element path, constant rows) and on thresholds that keep all or nothing."""
    note("capture edge rows tau=%g scope=%d" % (tau, scope))
    _capture_both(_edge_maps(), tau=tau, norm_scope=scope)


def test_capture_longest_window():
    """L = 4096, the longest capture window (its per-row tables need more than 64 KiB of LDS)."""
    L = 4096
    rng = np.random.default_rng(4096)
    A = rng.random((2, L, L), dtype=np.float32) ** 4
    A = np.tril(A)
    A /= np.maximum(1e-30, A.sum(axis=2, keepdims=True))
    note("capture L=%d" % L)
    for scope in (0, 1):
        _capture_both(A.astype(np.float32), norm_scope=scope)


def test_capture_thresholds_and_mu():
    maps = W.capture_maps(layers=1, heads=4, n_avg=4, layer_offset=7)
    _capture_both(maps, tau=0.55, mu=0.6)


def test_capture_rejects_bad_lambda():
    m = sa()
    for lam, eps in ((float("nan"), 1e-8), (0.0, 0.0)):
        with pytest.raises(m.SAError) as e:
            m.pattern_capture(torch.zeros(1, 8, 8, device="cuda"), lam=lam, eps=eps)
        assert e.value.code == -1


@pytest.mark.parametrize("lam", [-0.5, 0.0, 0.25, 1.0, 2.0])
@pytest.mark.parametrize("scope", [0, 1])
def test_capture_other_lambdas(lam, scope):
    """Box-Cox through the device pow / log.  Those are a few ulp from the host's, so the comparison is
    exact only where no cell's normalised score is within 1e-9 of tau: the oracle's scores show that first."""
    note("capture lambda=%g scope=%d" % (lam, scope))
    maps = W.capture_maps(layers=1, heads=32, n_avg=8, layer_offset=17)
    t = oracle.capture_scores(maps, lam=lam, norm_scope=scope)
    assert not (np.abs(t - 0.3) < 1e-9).any()
    _capture_both(maps, lam=lam, norm_scope=scope)


@pytest.mark.parametrize("lam,tau,mu", [(0.5, 0.3, 0.8), (0.0, 0.5, 0.7), (1.0, 0.1, 0.9)])
def test_coverage_matches_oracle(lam, tau, mu):
    """Keep flags from the oracle's capture of the same maps feed both sides."""
    m = sa()
    maps = W.capture_maps(layers=1, heads=32, n_avg=8, layer_offset=19)
    c = oracle.capture(maps, lam=lam, tau=tau, mu=mu)
    mass, cells = m.pattern_coverage(torch.from_numpy(maps).cuda(), torch.from_numpy(c["keep_diag"]).cuda(),
                                     torch.from_numpy(c["keep_vert"]).cuda())
    torch.cuda.synchronize()
    rm, rc = oracle.coverage(maps, c["keep_diag"], c["keep_vert"])
    np.testing.assert_array_equal(cells.cpu().numpy(), rc)
    np.testing.assert_allclose(mass.cpu().numpy(), rm, rtol=0, atol=1e-12)
    assert 0.0 < rm.min() and rm.max() <= 1.0


def test_coverage_edge_cases():
    """Every diagonal kept: the whole window, mass 1; nothing kept: 0; L = 1."""
    m = sa()
    maps = W.capture_maps(layers=1, heads=4, L=200, n_avg=2)
    md = torch.from_numpy(maps).cuda()
    ones = torch.ones((4, 200), dtype=torch.uint8, device="cuda")
    zeros = torch.zeros_like(ones)
    mass, cells = m.pattern_coverage(md, ones, zeros)
    m0, c0 = m.pattern_coverage(md, zeros, zeros)
    one = torch.full((2, 1, 1), 0.7, device="cuda")
    m1, c1 = m.pattern_coverage(one, torch.zeros((2, 1), dtype=torch.uint8, device="cuda"),
                                torch.ones((2, 1), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert (cells == 200 * 201 // 2).all() and (mass - 1).abs().max().item() < 1e-12
    assert (c0 == 0).all() and (m0 == 0).all()
    assert (c1 == 1).all() and (m1 == 1).all()


@pytest.mark.parametrize("S", [300, 512, 16384])
def test_patterns_to_desc_matches_oracle_extension(S):
    m = sa()
    maps = W.capture_maps(layers=1, heads=32, n_avg=8)
    c = oracle.capture(maps)
    pat = m.patterns_to_desc(torch.from_numpy(c["keep_diag"]).cuda(), torch.from_numpy(c["keep_vert"]).cuda(), S)
    torch.cuda.synchronize()
    diags, verts = oracle.extend(c["keep_diag"], c["keep_vert"], S)
    dp, do = pat.diag_ptr.cpu().numpy(), pat.diag_off.cpu().numpy()
    vp, vc = pat.vert_ptr.cpu().numpy(), pat.vert_col.cpu().numpy()
    for h in range(32):
        np.testing.assert_array_equal(do[dp[h]:dp[h + 1]], diags[h])
        np.testing.assert_array_equal(vc[vp[h]:vp[h + 1]], verts[h])


def test_capture_to_attention_end_to_end():
    """All on the GPU: capture -> extension to S=16384 -> index -> attention; vs the oracle pipeline."""
    m = sa()
    S = 16384
    maps = W.capture_maps(layers=1, heads=32, n_avg=16, layer_offset=3)
    note("end-to-end capture -> attention S=%d" % S)
    got = m.pattern_capture(torch.from_numpy(maps).cuda())
    pat = m.patterns_to_desc(got["keep_diag"], got["keep_vert"], S)
    ix = m.build_index(pat, 64)
    q, k, v = W.qkv(3, 1, 32, 8, S, 64, "bf16", seed_extra=3)
    o = m.sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), ix)
    torch.cuda.synchronize()
    ref = oracle.capture(maps)
    diags, verts = oracle.extend(ref["keep_diag"], ref["keep_vert"], S)
    desc = W.desc_from_lists(S, diags, verts)
    assert int(ix.pair_count.sum().item()) == int(oracle.pair_count(desc).sum())
    rows = rows_of_blocks(1, 32, S, 64, 2, np.random.default_rng(33))
    ro, _ = oracle.attention_rows(desc, q, k, v, rows)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    go = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
    assert_close_bf16(go, ro, "end-to-end")


def test_capture_into_given_outputs():
    """`out` of an earlier call is written again: a second map set through the same tensors gives the
    oracle's flags, hits and mask for that set."""
    m = sa()
    rng = np.random.default_rng(12)
    a = (rng.random((6, 128, 128)) ** 3).astype(np.float32)
    b = (rng.random((6, 128, 128)) ** 2).astype(np.float32)
    note("capture into given outputs")
    out = m.pattern_capture(torch.from_numpy(a).cuda(), return_mask=True)
    got = m.pattern_capture(torch.from_numpy(b).cuda(), return_mask=True, out=out)
    torch.cuda.synchronize()
    ref = oracle.capture(b, want_mask=True)
    for key in ("keep_diag", "keep_vert", "diag_hits", "vert_hits", "true_mask"):
        assert got[key].data_ptr() == out[key].data_ptr()
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    with pytest.raises(ValueError):
        m.pattern_capture(torch.from_numpy(b[:3]).cuda(), out=out)   # shapes differ
