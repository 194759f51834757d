"""Seeded synthetic inputs for structured sparse prefill attention.

This module only draws inputs: pattern descriptors (diagonal offsets, vertical
columns, 64x64 block bitmaps, per-row-block stripe column lists), query/key/
value tensors and averaged attention maps for pattern capture.  It contains none
of the method's arithmetic (no masking, softmax of the method, transform,
threshold or scoring), so both the HIP library's tests and the CPU oracle can
take their inputs from here without sharing any of the computation.

Every generator is seeded with ``numpy.random.default_rng([config_id, ...])``.
The recipes (sizes, value distributions, pattern structure) follow the five
workloads the library is measured on:

1. Tiny       S=512, 1 head, d=64, fp32; diagonals r in 0..63, verticals
              {0,1,2,3} + 8 seeded columns in [4, 511]; variants dense-causal
              (all diagonals), all-ones (all verticals), diagonal-0 only.
2. 1B-like    S=8192, 32 q / 8 kv heads, d=64, bf16; per head a local band of
              width U{64..512}, 0..8 extra diagonals in [512, S-1], 4..64
              verticals (half sinks in [0, 63], the rest uniform).
3. Capture    16 layers x 32 heads of 512x512 averaged causal attention maps;
              each map is the mean of n_avg row-softmaxes of logits
              N(0,1) + 3 on diagonals r < 32 + 3 on columns c < 4 + 2 on four
              seeded columns in [4, 511]; stored fp32.
4. 8B-like    S=65536, 32 q / 8 kv heads, d=128, bf16; even heads vertical+slash
              (band r < 1024, 32..256 columns, 8..32 diagonals in [1024, S-1]);
              odd heads 64x64 block-sparse (Bernoulli(0.08) below the block
              diagonal, plus diagonal blocks and block column 0).
5. Long       S=131072, 32 q / 8 kv heads, d=128, bf16; per 128-row stripe a
              sorted column list: sinks 0..63, the block-aligned local band of
              2048 columns, and each other earlier column with probability 0.03.

Every generator also takes S (and head counts) as arguments so that tests can
draw the same structure at small or ragged sizes.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "PatternDesc", "bf16_bits", "bf16_bits_to_f32", "qkv",
    "tiny", "llama1b_like", "capture_maps", "llama8b_like", "long_stripes",
    "desc_from_lists", "CONFIG_SHAPES", "MAX_S", "max_length",
]

# (B, Hq, Hkv, d, S, dtype) of the five workloads
CONFIG_SHAPES = {
    1: dict(B=1, hq=1, hkv=1, d=64, S=512, dtype="f32"),
    2: dict(B=1, hq=32, hkv=8, d=64, S=8192, dtype="bf16"),
    3: dict(B=1, hq=32, hkv=8, d=64, S=16384, dtype="bf16", L=512, layers=16),
    4: dict(B=1, hq=32, hkv=8, d=128, S=65536, dtype="bf16"),
    5: dict(B=1, hq=32, hkv=8, d=128, S=131072, dtype="bf16"),
}


@dataclass
class PatternDesc:
    """Per-query-head pattern descriptor (host numpy arrays).

    diag_ptr/diag_off: CSR over heads of strictly increasing diagonal offsets r
    in [0, S) (pair (i, i-r)).  vert_ptr/vert_col: CSR over heads of strictly
    increasing vertical columns c in [0, S) (pair (i, c), i >= c).
    block_mask: None or uint8 [H, nbq, nbq] with nbq = ceil(S/block_size).
    stripe_ptr/stripe_col: None or CSR over (head, stripe) of strictly
    increasing columns; stripe t covers query rows [t*stripe_rows, ...).
    """
    S: int
    H: int
    diag_ptr: np.ndarray
    diag_off: np.ndarray
    vert_ptr: np.ndarray
    vert_col: np.ndarray
    block_mask: Optional[np.ndarray] = None
    block_size: int = 64
    stripe_ptr: Optional[np.ndarray] = None
    stripe_col: Optional[np.ndarray] = None
    stripe_rows: int = 128
    meta: dict = field(default_factory=dict)

    def diags(self, h: int) -> np.ndarray:
        return self.diag_off[self.diag_ptr[h]:self.diag_ptr[h + 1]]

    def verts(self, h: int) -> np.ndarray:
        return self.vert_col[self.vert_ptr[h]:self.vert_ptr[h + 1]]

    def stripe(self, h: int, t: int) -> np.ndarray:
        nst = -(-self.S // self.stripe_rows)
        a, b = self.stripe_ptr[h * nst + t], self.stripe_ptr[h * nst + t + 1]
        return self.stripe_col[a:b]


def _csr(lists: Sequence[np.ndarray], ptr_dtype=np.int32):
    ptr = np.zeros(len(lists) + 1, dtype=ptr_dtype)
    for n, a in enumerate(lists):
        ptr[n + 1] = ptr[n] + len(a)
    flat = np.concatenate([np.asarray(a, dtype=np.int32) for a in lists]) if lists else np.zeros(0, np.int32)
    return ptr, flat.astype(np.int32)


def desc_from_lists(S: int, diags: Sequence, verts: Sequence, block_mask=None, block_size=64,
                    stripes: Optional[List[List[np.ndarray]]] = None, stripe_rows=128, meta=None) -> PatternDesc:
    """Build a PatternDesc from per-head lists (each list is sorted and unique here)."""
    H = len(diags)
    dl = [np.unique(np.asarray(d, dtype=np.int64)).astype(np.int32) for d in diags]
    vl = [np.unique(np.asarray(v, dtype=np.int64)).astype(np.int32) for v in verts]
    dp, do = _csr(dl)
    vp, vc = _csr(vl)
    sp = sc = None
    if stripes is not None:
        flat = [np.asarray(s, dtype=np.int32) for per_head in stripes for s in per_head]
        sp, sc = _csr(flat, ptr_dtype=np.int64)
    return PatternDesc(S=S, H=H, diag_ptr=dp, diag_off=do, vert_ptr=vp, vert_col=vc,
                       block_mask=None if block_mask is None else np.ascontiguousarray(block_mask, dtype=np.uint8),
                       block_size=block_size, stripe_ptr=sp, stripe_col=sc, stripe_rows=stripe_rows,
                       meta=dict(meta or {}))


# ----------------------------------------------------------------------------
# value tensors
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def qkv(config_id: int, B: int, hq: int, hkv: int, S: int, d: int, dtype: str, seed_extra: int = 0):
    """Q [B,hq,S,d], K and V [B,hkv,S,d] ~ N(0,1); float32, or bf16 bit patterns (uint16)."""
    out = []
    for n, heads in enumerate((hq, hkv, hkv)):
        rng = np.random.default_rng([config_id, 1000 + seed_extra, n])
        x = rng.standard_normal((B, heads, S, d), dtype=np.float32)
        out.append(x if dtype == "f32" else bf16_bits(x))
    return tuple(out)


# ----------------------------------------------------------------------------
# pattern recipes
# ----------------------------------------------------------------------------
def tiny(variant: str = "base", S: int = 512) -> PatternDesc:
    """Workload 1: one head, diagonals 0..63 + verticals {0..3} + 8 seeded columns."""
    if variant == "base":
        rng = np.random.default_rng(0)
        extra = rng.choice(np.arange(4, S), size=8, replace=False)
        return desc_from_lists(S, [np.arange(0, min(64, S))], [np.concatenate([np.arange(4), extra])],
                               meta=dict(variant=variant))
    if variant == "dense_causal":   # every diagonal: the whole causal triangle, band encoding
        return desc_from_lists(S, [np.arange(S)], [np.zeros(0)], meta=dict(variant=variant))
    if variant == "all_ones":       # every vertical: the whole causal triangle, column encoding
        return desc_from_lists(S, [np.zeros(0)], [np.arange(S)], meta=dict(variant=variant))
    if variant == "diag0":
        return desc_from_lists(S, [np.array([0])], [np.zeros(0)], meta=dict(variant=variant))
    raise ValueError(variant)


def llama1b_like(S: int = 8192, H: int = 32) -> PatternDesc:
    """Workload 2: per head band U{64..512}, 0..8 far diagonals, 4..64 verticals (sink-biased)."""
    diags, verts = [], []
    for h in range(H):
        rng = np.random.default_rng([2, h])
        w = int(rng.integers(64, 513))
        band = np.arange(min(w, S))
        n_extra = int(rng.integers(0, 9))
        far = rng.choice(np.arange(512, S), size=min(n_extra, max(S - 512, 0)), replace=False) if S > 512 else np.zeros(0)
        n_v = int(rng.integers(4, 65))
        n_sink = (n_v + 1) // 2
        sinks = rng.choice(np.arange(min(64, S)), size=min(n_sink, min(64, S)), replace=False)
        rest = rng.choice(np.arange(64, S), size=min(n_v - n_sink, max(S - 64, 0)), replace=False) if S > 64 else np.zeros(0)
        diags.append(np.concatenate([band, far]))
        verts.append(np.concatenate([sinks, rest]))
    return desc_from_lists(S, diags, verts, meta=dict(workload="llama1b_like"))


def capture_maps(layers: int = 16, heads: int = 32, L: int = 512, n_avg: int = 16,
                 layer_offset: int = 0, threads: Optional[int] = None) -> np.ndarray:
    """Workload 3 maps: float32 [layers*heads, L, L] averaged causal row-softmaxes.

    Logits = N(0,1) + 3.0*[i-j < 32] + 3.0*[j < 4] + 2.0*[j in 4 seeded columns];
    positions j > i carry no weight.  Computed in float64, stored float32.  Each
    map has its own seed, so the maps are drawn on a thread pool (numpy releases
    the interpreter lock in its array loops) with the same values as in series.
    """
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    causal = j <= i
    base = 3.0 * ((i - j) < 32) + 3.0 * (j < 4)
    out = np.empty((layers * heads, L, L), dtype=np.float32)

    def one(m):
        l, h = divmod(m, heads)
        rng = np.random.default_rng([3, layer_offset + l, h])
        cols = rng.choice(np.arange(4, L), size=4, replace=False)
        boost = base + 2.0 * np.isin(j, cols)
        acc = np.zeros((L, L))
        for _ in range(n_avg):
            z = rng.standard_normal((L, L)) + boost
            z = np.where(causal, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            e = np.exp(z)
            acc += e / e.sum(axis=1, keepdims=True)
        out[m] = (acc / n_avg).astype(np.float32)

    n = layers * heads
    workers = threads or min(16, os.cpu_count() or 1, n)
    if workers <= 1:
        for m in range(n):
            one(m)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(n)))
    return out


def capture_qk(config_id: int, B: int, hq: int, hkv: int, L: int, d: int, dtype: str, n_freq: int = 12,
               local: float = 6.0, sink: float = 6.0):
    """Q [B,hq,L,d], K [B,hkv,L,d] whose causal attention carries local-band and sink-column structure.

    Dims 0..2*n_freq-1 hold a positional code: q_i and k_j carry cos/sin(w_m * pos) with
    w_m geometric in [pi/256, pi/16], so their product depends on i - j only and peaks at
    i = j with height `local` (in units of the 1/sqrt(d) scaled logit).  Dim 2*n_freq is a
    shared direction: every query has a, keys j < 4 and 4 seeded columns per kv head have a,
    with a*a/sqrt(d) = `sink`.  Remaining dims and all dims get N(0, 0.5^2) noise per sequence.
    """
    rt = np.sqrt(np.sqrt(d))
    w = np.geomspace(np.pi / 256, np.pi / 16, n_freq)
    pos = np.arange(L)[:, None] * w[None, :]
    code = np.concatenate([np.cos(pos), np.sin(pos)], axis=1) * np.sqrt(local / n_freq) * rt   # [L, 2*n_freq]
    a = np.sqrt(sink) * rt
    q = np.zeros((B, hq, L, d), np.float64)
    k = np.zeros((B, hkv, L, d), np.float64)
    q[..., :2 * n_freq] = code
    k[..., :2 * n_freq] = code
    q[..., 2 * n_freq] = a
    for g in range(hkv):
        rng = np.random.default_rng([config_id, 3000, g])
        cols = np.concatenate([np.arange(min(4, L)), rng.choice(np.arange(4, L), size=min(4, max(L - 4, 0)), replace=False)])
        k[:, g, cols, 2 * n_freq] = a
    rng = np.random.default_rng([config_id, 3001])
    q += 0.5 * rng.standard_normal(q.shape)
    k += 0.5 * rng.standard_normal(k.shape)
    q, k = q.astype(np.float32), k.astype(np.float32)
    return (q, k) if dtype == "f32" else (bf16_bits(q), bf16_bits(k))


def runtime_qk(config_id: int, B: int, hq: int, hkv: int, S: int, d: int, dtype: str, n_cols: int = 16):
    """Q [B,hq,S,d], K [B,hkv,S,d] for per-input capture at long S (float32 math, bf16 or f32 out).

    Dims 0..63 carry a positional code (cos/sin of 32 frequencies geometric in [pi/4096, pi/4]),
    so the logits peak at i = j with height 8 and fall off over tens of positions (a local band),
    with a texture of about one logit far from the diagonal; dim 64 is a shared direction: every
    query has d^(1/4) * f (f seeded per query head in [0.9, 1.1]), sink keys 0..3 have
    13 d^(1/4) and `n_cols` seeded columns per kv head have 11 d^(1/4), i.e. logit boosts of 13 f
    and 11 f (sinks that hold most of a long row's mass); every dim gets N(0, 0.3^2) noise.
    Needs d >= 65.  Generated one head at a time.
    """
    nf = 32
    assert d > 2 * nf
    rt = np.float32(np.sqrt(np.sqrt(d)))
    w = np.geomspace(np.pi / 4096, np.pi / 4, nf).astype(np.float32)
    pos = np.arange(S, dtype=np.float32)[:, None] * w[None, :]
    code = (np.concatenate([np.cos(pos), np.sin(pos)], axis=1) * np.float32(np.sqrt(8.0 / nf)) * rt).astype(np.float32)
    out_q = np.empty((B, hq, S, d), np.uint16 if dtype != "f32" else np.float32)
    out_k = np.empty((B, hkv, S, d), out_q.dtype)
    conv = (lambda x: x) if dtype == "f32" else bf16_bits
    for g in range(hkv):
        rng = np.random.default_rng([config_id, 4000, g])
        cols = rng.choice(np.arange(4, S), size=min(n_cols, max(S - 4, 0)), replace=False) if S > 4 else np.zeros(0, int)
        for b in range(B):
            x = 0.3 * rng.standard_normal((S, d), dtype=np.float32)
            x[:, :2 * nf] += code
            x[:min(4, S), 2 * nf] += 13.0 * rt
            x[cols, 2 * nf] += 11.0 * rt
            out_k[b, g] = conv(x)
    for h in range(hq):
        rng = np.random.default_rng([config_id, 4001, h])
        f = np.float32(rng.uniform(0.9, 1.1))
        for b in range(B):
            x = 0.3 * rng.standard_normal((S, d), dtype=np.float32)
            x[:, :2 * nf] += code
            x[:, 2 * nf] += rt * f
            out_q[b, h] = conv(x)
    return out_q, out_k


def llama8b_like(S: int = 65536, H: int = 32, band: int = 1024, block_p: float = 0.08,
                 block_size: int = 64) -> PatternDesc:
    """Workload 4: even heads vertical+slash, odd heads 64x64 block-sparse."""
    nbq = -(-S // block_size)
    bm = np.zeros((H, nbq, nbq), dtype=np.uint8)
    diags, verts = [], []
    for h in range(H):
        rng = np.random.default_rng([4, h])
        if h % 2 == 0:
            n_c = int(rng.integers(32, 257))
            n_d = int(rng.integers(8, 33))
            cols = rng.choice(S, size=min(n_c, S), replace=False)
            far = rng.choice(np.arange(band, S), size=min(n_d, max(S - band, 0)), replace=False) if S > band else np.zeros(0)
            diags.append(np.concatenate([np.arange(min(band, S)), far]))
            verts.append(cols)
        else:
            lower = np.tril(rng.random((nbq, nbq)) < block_p, k=-1)
            m = lower | np.eye(nbq, dtype=bool)
            m[:, 0] = True
            bm[h] = np.tril(m).astype(np.uint8)
            diags.append(np.zeros(0))
            verts.append(np.zeros(0))
    return desc_from_lists(S, diags, verts, block_mask=bm, block_size=block_size,
                           meta=dict(workload="llama8b_like"))


def long_stripes(S: int = 131072, H: int = 32, stripe_rows: int = 128, band: int = 2048,
                 sinks: int = 64, p: float = 0.03) -> PatternDesc:
    """Workload 5: per 128-row stripe, sinks + block-aligned local band + Bernoulli(p) columns.

    The Bernoulli columns of [sinks, lo) are drawn as a Bernoulli process via
    geometric gaps (the same distribution as one draw per column).
    """
    nst = -(-S // stripe_rows)
    stripes = []
    for h in range(H):
        rng = np.random.default_rng([5, h])
        per = []
        for t in range(nst):
            top = min(S, (t + 1) * stripe_rows) - 1
            lo = max(0, (t + 1) * stripe_rows - band)
            parts = [np.arange(min(sinks, top + 1))]
            if lo > sinks:
                n_max = lo - sinks
                gaps = rng.geometric(p, size=int(n_max * p * 1.5) + 32)
                pos = np.cumsum(gaps) - 1
                while pos[-1] < n_max - 1:
                    more = rng.geometric(p, size=int(n_max * p * 0.5) + 32)
                    pos = np.concatenate([pos, pos[-1] + np.cumsum(more)])
                parts.append(sinks + pos[pos < n_max])
            parts.append(np.arange(max(lo, 0), top + 1))
            per.append(np.unique(np.concatenate(parts)).astype(np.int32))
        stripes.append(per)
    return desc_from_lists(S, [np.zeros(0)] * H, [np.zeros(0)] * H, stripes=stripes,
                           stripe_rows=stripe_rows, meta=dict(workload="long_stripes"))


MAX_S = 262144   # the longest sequence the index accepts


def max_length(S: int = MAX_S, H: int = 2, seed: int = 9) -> PatternDesc:
    """Every pattern kind at the longest accepted sequence: a 256-wide band plus far diagonals up
    to S - 1, sinks plus verticals up to S - 1, 128 x 128 blocks at density 0.002 plus block
    column 0 and the last block row, and 128-row stripe lists of up to 8 random columns."""
    rng = np.random.default_rng([10, seed])
    nbq = -(-S // 128)
    bm = (rng.random((H, nbq, nbq)) < 0.002).astype(np.uint8)
    bm[:, :, 0] = 1
    bm[:, nbq - 1, :] = 1
    bm = np.tril(bm)
    diags, verts, stripes = [], [], []
    for h in range(H):
        diags.append(np.concatenate([np.arange(256), rng.choice(np.arange(256, S), 12, replace=False), [S - 1]]))
        verts.append(np.concatenate([np.arange(16), rng.choice(np.arange(16, S), 20, replace=False), [S - 1]]))
        per = []
        for t in range(-(-S // 128)):
            top = min(S, (t + 1) * 128) - 1
            per.append(np.sort(rng.choice(top + 1, size=min(top + 1, int(rng.integers(0, 9))), replace=False)))
        stripes.append(per)
    return desc_from_lists(S, diags, verts, block_mask=bm, block_size=128, stripes=stripes, stripe_rows=128,
                           meta=dict(workload="max_length"))
