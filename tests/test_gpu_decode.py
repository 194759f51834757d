"""GPU parity: sa_sparse_attn_decode vs the fp64 oracle's decode form.

A decode query of sequence b at position t is row t of the masked attention with an
explicit query vector (oracle.attention_queries).  Every (sequence, head) row is
checked.  Tolerances as for prefill: bf16 max-abs 2e-2 and mean-abs 2e-3 (LSE within
2^-8, as the probabilities are fp32 here, tighter than that bound needs); fp32
max-abs 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close_bf16, assert_close_f32, assert_lse, note, sa, to_dev

pytestmark = pytest.mark.gpu


def _decode(desc, qd, k, v, pos, BM, what, scale=None):
    """qd [B,hq,d] (numpy, f32 or bf16 bits), k/v [B,hkv,S,d], pos [B]: compare every row with the oracle."""
    m = sa()
    B, hq, d = qd.shape
    S = k.shape[2]
    note("decode %s S=%d B=%d hq=%d hkv=%d d=%d BM=%d dtype=%s" % (what, S, B, hq, k.shape[1], d, BM, qd.dtype))
    ix = m.build_index(m.DevicePatterns.from_host(desc), BM)
    posd = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
    o, lse = m.sparse_attn_decode(to_dev(qd), to_dev(k), to_dev(v), posd, ix, softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    rows = np.array([(b, h, pos[b]) for b in range(B) for h in range(hq)], np.int32)
    ref, ref_lse = oracle.attention_queries(desc, qd.reshape(B * hq, d), k, v, rows, scale=scale)
    got = o.float().cpu().numpy().reshape(B * hq, d).astype(np.float64)
    got_lse = lse.cpu().numpy().reshape(-1).astype(np.float64)
    if qd.dtype == np.float32:
        assert_close_f32(got, ref, what)
        assert_lse(got_lse, ref_lse, 1e-5, what)
    else:
        assert_close_bf16(got, ref, what)
        assert_lse(got_lse, ref_lse, 2.0 ** -8, what)
    return o


def _queries(seed, B, hq, d, dtype):
    x = np.random.default_rng([7, seed]).standard_normal((B, hq, d)).astype(np.float32)
    return x if dtype == "f32" else W.bf16_bits(x)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_decode_llama1b_like_positions(dtype, d):
    S, B = 1000, 4
    desc = W.llama1b_like(S=S, H=8)
    _, k, v = W.qkv(31, B, 8, 2, S, d, dtype)
    _decode(desc, _queries(1, B, 8, d, dtype), k, v, [0, 1, 517, S - 1], 64, "1b-like")


@pytest.mark.parametrize("BM", [64, 128])
def test_decode_every_pattern_kind(BM):
    """Diagonal runs, verticals, 128 x 128 blocks and 256-row stripe lists in every head (bitmap index path)."""
    rng = np.random.default_rng(33)
    S, H = 1500, 4
    diags = [np.unique(np.concatenate([np.arange(rng.integers(1, 200)), rng.choice(S, 6, replace=False)]))
             for _ in range(H)]
    verts = [rng.choice(S, 9, replace=False) for _ in range(H)]
    nbq = -(-S // 128)
    bm = (rng.random((H, nbq, nbq)) < 0.2).astype(np.uint8)
    stripes = [[np.sort(rng.choice(S, size=int(rng.integers(0, 60)), replace=False)) for _ in range(-(-S // 256))]
               for _ in range(H)]
    desc = W.desc_from_lists(S, diags, verts, block_mask=bm, block_size=128, stripes=stripes, stripe_rows=256)
    _, k, v = W.qkv(32, 3, H, 2, S, 64, "bf16")
    _decode(desc, _queries(2, 3, H, 64, "bf16"), k, v, [5, 777, 1499], BM, "all-kinds")


def test_decode_diagonal_zero_returns_cache_row():
    S, B = 300, 3
    desc = W.tiny("diag0", S=S)
    _, k, v = W.qkv(34, B, 1, 1, S, 128, "bf16")
    pos = [0, 150, 299]
    o = _decode(desc, _queries(3, B, 1, 128, "bf16"), k, v, pos, 64, "diag0")
    for b, t in enumerate(pos):
        assert torch.equal(o[b, 0].cpu(), to_dev(v[b, 0, t], "cpu"))


def test_decode_empty_row_and_positions_out_of_range():
    """A row without retained keys, and positions outside [0, S): zero output and -inf lse."""
    m = sa()
    S = 200
    desc = W.desc_from_lists(S, [np.zeros(0)], [np.array([70])])
    _, k, v = W.qkv(35, 4, 1, 1, S, 64, "f32")
    q = _queries(4, 4, 1, 64, "f32")
    ix = m.build_index(m.DevicePatterns.from_host(desc), 64)
    pos = torch.tensor([10, -1, S, 150], dtype=torch.int32, device="cuda")
    note("decode empty rows / out-of-range positions")
    o, lse = m.sparse_attn_decode(to_dev(q), to_dev(k), to_dev(v), pos, ix, return_lse=True)
    torch.cuda.synchronize()
    for b in (0, 1, 2):
        assert o[b].abs().max().item() == 0.0 and lse[b, 0].item() == float("-inf")
    ref, _ = oracle.attention_queries(desc, q[3], k, v, np.array([(3, 0, 150)], np.int32))
    assert_close_f32(o[3].cpu().numpy().astype(np.float64), ref, "decode row 150")


def test_decode_batch_gqa_and_custom_scale():
    S = 700
    desc = W.llama1b_like(S=S, H=6)
    _, k, v = W.qkv(36, 2, 6, 3, S, 128, "bf16")
    _decode(desc, _queries(5, 2, 6, 128, "bf16"), k, v, [699, 333], 128, "gqa-scale", scale=0.2)


def test_decode_llama8b_like_full_size():
    S, B = 65536, 2
    desc = W.llama8b_like()
    _, k, v = W.qkv(37, B, 8, 8, S, 128, "bf16")   # 8 kv heads, one query head each is enough to read every pattern
    d8 = W.desc_from_lists(S, [desc.diags(h) for h in range(8)], [desc.verts(h) for h in range(8)],
                           block_mask=desc.block_mask[:8], block_size=64)
    _decode(d8, _queries(6, B, 8, 128, "bf16"), k, v, [S - 1, 40000], 64, "8b-like-64k")


def test_decode_long_stripes_full_size():
    S = 131072
    desc = W.long_stripes(H=4)
    _, k, v = W.qkv(38, 1, 4, 1, S, 128, "bf16")
    _decode(desc, _queries(7, 1, 4, 128, "bf16"), k, v, [S - 1], 128, "stripes-131k")


def test_decode_max_length():
    """S = 262144, every pattern kind; the last position, the first and one in the middle."""
    S = W.MAX_S
    desc = W.max_length()
    _, k, v = W.qkv(39, 3, 2, 1, S, 128, "bf16")
    _decode(desc, _queries(8, 3, 2, 128, "bf16"), k, v, [S - 1, 0, 131071], 128, "max-length")


@pytest.mark.parametrize("S", [1, 2, 65, 129])
@pytest.mark.parametrize("BM", [64, 128])
def test_decode_short_sequences_and_an_empty_head(S, BM):
    """Caches shorter than one tile or a tile plus one row, every pattern kind, a head with no pattern."""
    from test_gpu_attn import _short_desc
    pos = sorted({0, S - 1, S // 2, max(0, S - 2)})
    B, H = len(pos), 3
    _, k, v = W.qkv(40, B, H, 1, S, 128, "bf16")
    o = _decode(_short_desc(S, H), _queries(9, B, H, 128, "bf16"), k, v, pos, BM, "short-S")
    assert o[:, H - 1].float().abs().max().item() == 0.0
