"""GPU parity: sa_sparse_attn_prefill vs the fp64 oracle.

Full parity (every row) at sizes the oracle finishes in seconds that span several
tiles and a ragged tail; at the full workload sizes (S = 8192, 16384, 65536,
131072), every row of the first, the last and seeded row blocks of every head,
in the same launch configuration the benchmark times.
Tolerances: bf16 max-abs 2e-2 and mean-abs 2e-3; fp32 max-abs 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (all_rows, assert_close_bf16, assert_close_f32, assert_lse, gather_lse, gather_rows, note,
                      rows_of_blocks, sa, to_dev, widen, workload3_maps)

pytestmark = pytest.mark.gpu


def _run(desc, q, k, v, BM, rows, what, scale=None, want_lse=False):
    m = sa()
    B, hq, S, d = q.shape
    note("attn %s S=%d hq=%d hkv=%d d=%d BM=%d dtype=%s rows=%d" % (what, S, hq, k.shape[1], d, BM, q.dtype,
                                                                     len(rows)))
    pat = m.DevicePatterns.from_host(desc)
    ix = m.build_index(pat, BM)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = m.sparse_attn_prefill(qd, kd, vd, ix, softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    got, got_lse = gather_rows(o, rows), gather_lse(lse, rows)
    ref, ref_lse = oracle.attention_rows(desc, q, k, v, rows, scale=scale)
    if q.dtype == np.float32:
        assert_close_f32(got, ref, what)
        assert_lse(got_lse, ref_lse, 1e-5, what)
    else:
        assert_close_bf16(got, ref, what)
        # bf16: the row sum is the sum of the bf16-rounded probabilities that also weight V, each
        # within 2^-9 relative of its exact value, so |lse - lse_exact| <= ln(1 + 2^-9) < 2^-8
        assert_lse(got_lse, ref_lse, 2.0 ** -8, what)
    return (o, ix, lse) if want_lse else (o, ix)


# ------------------------------------------------------------------ workload 1 (fp32) and its variants
@pytest.mark.parametrize("variant", ["base", "dense_causal", "all_ones", "diag0"])
@pytest.mark.parametrize("BM", [64, 128])
def test_tiny_fp32(variant, BM):
    desc = W.tiny(variant)
    q, k, v = W.qkv(1, 1, 1, 1, 512, 64, "f32")
    _run(desc, q, k, v, BM, all_rows(1, 1, 512), "tiny-" + variant)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_diagonal_zero_returns_v_exactly(dtype, d):
    m = sa()
    S = 300
    desc = W.tiny("diag0", S=S)
    q, k, v = W.qkv(11, 1, 1, 1, S, d, dtype)
    note("diag0 identity dtype=%s d=%d" % (dtype, d))
    ix = m.build_index(m.DevicePatterns.from_host(desc), 64)
    o = m.sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), ix)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), to_dev(v, "cpu"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_band_and_column_encodings_agree(dtype):
    S, d = 700, 64
    q, k, v = W.qkv(12, 1, 1, 1, S, d, dtype)
    rows = all_rows(1, 1, S)
    oa, _ = _run(W.tiny("dense_causal", S=S), q, k, v, 64, rows, "dense-band")
    ob, _ = _run(W.tiny("all_ones", S=S), q, k, v, 64, rows, "dense-cols")
    diff = (oa.float() - ob.float()).abs().max().item()
    assert diff <= (1e-5 if dtype == "f32" else 2e-2)


def test_constant_v_gives_ones():
    m = sa()
    S, d = 900, 128
    desc = W.llama8b_like(S=S, H=4)
    q, k, _ = W.qkv(13, 1, 4, 2, S, d, "bf16")
    v = W.bf16_bits(np.ones((1, 2, S, d), np.float32))
    note("constant v")
    ix = m.build_index(m.DevicePatterns.from_host(desc), 64)
    o = m.sparse_attn_prefill(to_dev(q), to_dev(k), to_dev(v), ix)
    torch.cuda.synchronize()
    assert (o.float() - 1.0).abs().max().item() <= 2e-2


def test_empty_rows_zero_output_minus_inf_lse():
    S, d = 200, 64
    desc = W.desc_from_lists(S, [np.zeros(0)], [np.array([70])])
    for dtype in ("f32", "bf16"):
        q, k, v = W.qkv(14, 1, 1, 1, S, d, dtype)
        o, _ = _run(desc, q, k, v, 64, all_rows(1, 1, S), "empty-rows-" + dtype)
        assert o[0, 0, :70].float().abs().max().item() == 0.0


def _short_desc(S, H):
    """Diagonals {0, 1, 5}, columns {0, S - 1}, 128 x 128 blocks and 128-row stripes, clipped to S; the last
    head holds no pattern at all (every row empty)."""
    rng = np.random.default_rng(S)
    nbq = -(-S // 128)
    bm = (rng.random((H, nbq, nbq)) < 0.5).astype(np.uint8)
    bm[H - 1] = 0
    diags = [np.array([r for r in (0, 1, 5) if r < S]) for _ in range(H - 1)] + [np.zeros(0)]
    verts = [np.unique([0, S - 1]) for _ in range(H - 1)] + [np.zeros(0)]
    stripes = [[np.sort(rng.choice(min(S, (t + 1) * 128), size=min(3, min(S, (t + 1) * 128)), replace=False))
                if h < H - 1 else np.zeros(0) for t in range(nbq)] for h in range(H)]
    return W.desc_from_lists(S, diags, verts, block_mask=bm, block_size=128, stripes=stripes, stripe_rows=128)


@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("dtype,d,BM", [("bf16", 128, 64), ("bf16", 128, 128), ("f32", 64, 64)])
def test_short_sequences_and_an_empty_head(S, dtype, d, BM):
    """Sequences shorter than one tile or a tile plus one row, every pattern kind, and a head with no pattern
    (zero output, lse -inf)."""
    H = 3
    q, k, v = W.qkv(23, 1, H, 1, S, d, dtype)
    o, _ = _run(_short_desc(S, H), q, k, v, BM, all_rows(1, H, S), "short-S")
    assert o[0, H - 1].float().abs().max().item() == 0.0


def test_batch_and_gqa_and_custom_scale():
    S, d = 333, 64
    desc = W.llama1b_like(S=S, H=6)
    q, k, v = W.qkv(15, 2, 6, 3, S, d, "bf16")
    _run(desc, q, k, v, 64, all_rows(2, 6, S), "batch-gqa-scale", scale=0.2)


@pytest.mark.parametrize("dtype,d,BM", [("bf16", 64, 64), ("bf16", 128, 128), ("f32", 64, 64)])
def test_group_major_schedule_every_row(dtype, d, BM):
    """Row-block counts that are a multiple of 32 take the kv-group-major workgroup order: with two batch
    elements, GQA 6/3 and every row checked, each (batch, head, row block) must be computed exactly once."""
    S = 32 * BM
    desc = W.llama1b_like(S=S, H=6)
    q, k, v = W.qkv(17, 2, 6, 3, S, d, dtype)
    _run(desc, q, k, v, BM, all_rows(2, 6, S), "group-major")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("BM", [64, 128])
def test_band_edges_partial_tiles(d, BM):
    """Bands whose width is not a multiple of the tile, a band with a hole and a lone far diagonal:
    tiles that lie below the block's first row but see offsets outside the band must stay masked."""
    S, H = 777, 4
    diags = [np.arange(150), np.arange(64), np.concatenate([np.arange(100), np.arange(140, 300)]),
             np.concatenate([np.arange(33), [500]])]
    desc = W.desc_from_lists(S, diags, [np.zeros(0)] * H)
    q, k, v = W.qkv(16, 1, H, 2, S, d, "bf16")
    _run(desc, q, k, v, BM, all_rows(1, H, S), "band-edges")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("BM", [64, 128])
def test_lone_and_paired_far_diagonals(dtype, d, BM):
    """Far diagonals without a band: a lone offset (rows below it empty), pairs 1, 63, 64 and 65 apart
    (one segment, two segments that touch, two apart), a diagonal next to the sequence end, and a
    head with 32 scattered offsets plus diagonal 0 (the 64K slash heads' far part).  Every row."""
    S, H = 1100, 8
    rng = np.random.default_rng(33)
    diags = [np.array([300]), np.array([300, 301]), np.array([300, 363]), np.array([300, 364]),
             np.array([300, 365]), np.array([0, S - 1]), np.concatenate([[0], np.sort(rng.choice(
                 np.arange(70, S), 32, replace=False))]), np.array([64, 128, 192, 640])]
    desc = W.desc_from_lists(S, diags, [np.zeros(0)] * H)
    q, k, v = W.qkv(34, 1, H, 2, S, d, dtype)
    _run(desc, q, k, v, BM, all_rows(1, H, S), "far-diagonals")


def _mixed_desc(S, H, seed):
    """Every pattern kind at once in each head: diagonal runs, verticals, 128 x 128 blocks and
    256-row stripe lists (the index builds these items with LDS bitmaps)."""
    rng = np.random.default_rng(seed)
    diags = [np.unique(np.concatenate([np.arange(rng.integers(1, 200)), rng.choice(S, 6, replace=False)]))
             for _ in range(H)]
    verts = [rng.choice(S, 9, replace=False) for _ in range(H)]
    nbq = -(-S // 128)
    bm = (rng.random((H, nbq, nbq)) < 0.2).astype(np.uint8)
    stripes = [[np.sort(rng.choice(S, size=int(rng.integers(0, 60)), replace=False)) for _ in range(-(-S // 256))]
               for _ in range(H)]
    return W.desc_from_lists(S, diags, verts, block_mask=bm, block_size=128, stripes=stripes, stripe_rows=256)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("BM", [64, 128])
def test_mixed_pattern_kinds_every_row(dtype, d, BM):
    S, H = 1500, 4
    q, k, v = W.qkv(18, 1, H, 2, S, d, dtype)
    _run(_mixed_desc(S, H, 21), q, k, v, BM, all_rows(1, H, S), "mixed-kinds")


# ------------------------------------------------------------------ workload 2 (1B-like, bf16, d=64)
@pytest.mark.parametrize("S,BM", [(1000, 64), (1000, 128)])
def test_llama1b_like_small_full(S, BM):
    desc = W.llama1b_like(S=S, H=8)
    q, k, v = W.qkv(2, 1, 8, 2, S, 64, "bf16")
    _run(desc, q, k, v, BM, all_rows(1, 8, S), "1b-like-small")


@pytest.mark.parametrize("BM", [64, 128])
def test_llama1b_like_full_size_every_row(BM):
    """The 1B-like workload at its full size (S = 8192, 32/8 heads, d = 64): every row of every head."""
    desc = W.llama1b_like()
    q, k, v = W.qkv(2, 1, 32, 8, 8192, 64, "bf16")
    _run(desc, q, k, v, BM, all_rows(1, 32, 8192), "1b-like")


# ------------------------------------------------------------------ workload 3 (capture -> S=16384)
def _layer_desc(layer, S=16384):
    """The kept sets of one layer of the capture workload (oracle capture of its 32 maps), extended to S."""
    maps = workload3_maps()[32 * layer:32 * (layer + 1)]
    c = oracle.capture(maps)
    diags, verts = oracle.extend(c["keep_diag"], c["keep_vert"], S)
    return W.desc_from_lists(S, diags, verts)


@pytest.mark.parametrize("layer", list(range(16)))
def test_capture_extended_attention_layer(layer):
    """The capture workload's attention run: one call per layer (32/8 heads, d = 64, S = 16384) with that
    layer's 32 kept sets; every row of the first, the last and 3 seeded row blocks of every head, and
    every row of every head for layer 0."""
    S = 16384
    desc = _layer_desc(layer, S)
    q, k, v = W.qkv(3, 1, 32, 8, S, 64, "bf16", seed_extra=layer)
    rows = all_rows(1, 32, S) if layer == 0 else rows_of_blocks(1, 32, S, 64, 3, np.random.default_rng([3, layer]))
    _run(desc, q, k, v, 64, rows, "capture-16k layer %d" % layer)


def _dense_cross_check(desc, q, k, v, o, lse, per_head, seed, what):
    """The dense form of the oracle (every key of the row, masked logits -inf) on `per_head` seeded rows of
    every head, against the same output: it shares no enumeration of retained keys with the sparse form."""
    B, hq, S, _ = q.shape
    rng = np.random.default_rng(seed)
    rows = np.array([(0, h, i) for h in range(hq) for i in np.concatenate([[S - 1], rng.choice(S, per_head - 1,
                                                                                                 replace=False)])],
                    dtype=np.int32)
    ref, ref_lse = oracle.attention_rows(desc, q, k, v, rows, mode=1)
    assert_close_bf16(gather_rows(o, rows), ref, what + " (dense -inf oracle)")
    assert_lse(gather_lse(lse, rows), ref_lse, 2.0 ** -8, what + " (dense -inf oracle)")


# ------------------------------------------------------------------ workload 4 (8B-like, d=128)
def test_llama8b_like_small_full():
    S = 2500
    desc = W.llama8b_like(S=S, H=8)
    q, k, v = W.qkv(4, 1, 8, 2, S, 128, "bf16")
    _run(desc, q, k, v, 64, all_rows(1, 8, S), "8b-like-small")


def test_llama8b_like_full_size_sampled():
    """Every row of the first, the last and 32 seeded row blocks of every head; then the dense (-inf) form
    of the oracle on 64 seeded rows of every head of the same output."""
    desc = W.llama8b_like()
    q, k, v = W.qkv(4, 1, 32, 8, 65536, 128, "bf16")
    rows = rows_of_blocks(1, 32, 65536, 64, 32, np.random.default_rng(4))
    o, _, lse = _run(desc, q, k, v, 64, rows, "8b-like", want_lse=True)
    _dense_cross_check(desc, q, k, v, o, lse, 64, 44, "8b-like")


# ------------------------------------------------------------------ workload 5 (stripes, S=131072)
@pytest.mark.parametrize("BM", [64, 128])
def test_long_stripes_small_full(BM):
    S = 3000
    desc = W.long_stripes(S=S, H=4, band=512)
    q, k, v = W.qkv(5, 1, 4, 2, S, 128, "bf16")
    _run(desc, q, k, v, BM, all_rows(1, 4, S), "stripes-small")


def test_long_stripes_full_size_sampled():
    """Every row of the first, the last and 32 seeded 128-row blocks of every head; then the dense (-inf)
    form of the oracle on 64 seeded rows of every head of the same output."""
    desc = W.long_stripes()
    q, k, v = W.qkv(5, 1, 32, 8, 131072, 128, "bf16")
    rows = rows_of_blocks(1, 32, 131072, 128, 32, np.random.default_rng(5))
    o, _, lse = _run(desc, q, k, v, 128, rows, "stripes-131k", want_lse=True)
    _dense_cross_check(desc, q, k, v, o, lse, 64, 55, "stripes-131k")


# ------------------------------------------------------------------ the longest accepted sequence
@pytest.mark.parametrize("dtype,d,BM", [("bf16", 128, 64), ("bf16", 128, 128), ("f32", 64, 128)])
def test_max_length_sampled(dtype, d, BM):
    """S = 262144 with every pattern kind: every row of the first, the last and 6 seeded row blocks
    of each head (K/V offsets up to the end of the slab, diagonals and columns up to S - 1)."""
    desc = W.max_length()
    q, k, v = W.qkv(22, 1, 2, 1, W.MAX_S, d, dtype)
    rows = rows_of_blocks(1, 2, W.MAX_S, BM, 6, np.random.default_rng(22))
    _run(desc, q, k, v, BM, rows, "max-length")


@pytest.mark.parametrize("kind,BM", [("blocks", 64), ("stripes", 128)])
def test_repeatable_on_a_side_stream_into_a_dirty_buffer(kind, BM):
    """No atomics or order-dependent sums: a second launch, on another stream and into an output buffer
    holding garbage, gives the same bits; refilling the index in place does not change them either."""
    m = sa()
    S = 3000
    desc = W.llama8b_like(S=S, H=8) if kind == "blocks" else W.long_stripes(S=S, H=8, band=512)
    q, k, v = W.qkv(19, 1, 8, 2, S, 128, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pat = m.DevicePatterns.from_host(desc)
    ix = m.build_index(pat, BM)
    note("repeatability BM=%d" % BM)
    o1, l1 = m.sparse_attn_prefill(qd, kd, vd, ix, return_lse=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2 = torch.full_like(o1, float("nan"))
        m.refill_index(pat, ix, stream=side)
        _, l2 = m.sparse_attn_prefill(qd, kd, vd, ix, return_lse=True, out=o2, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_rejects_bad_arguments():
    m = sa()
    desc = W.tiny("base")
    ix = m.build_index(m.DevicePatterns.from_host(desc), 64)
    q = torch.zeros(1, 1, 512, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 512, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.SAError):   # head_dim 32 unsupported
        m.sparse_attn_prefill(q[..., :32].contiguous(), k[..., :32].contiguous(), k[..., :32].contiguous(), ix)
    q2 = torch.zeros(1, 2, 512, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.SAError):   # index built for one head
        m.sparse_attn_prefill(q2, k, k, ix)
