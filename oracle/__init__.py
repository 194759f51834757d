"""CPU oracle for structured sparse prefill attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it never imports the
product package.  Inputs come from ``workloads`` (seeded draws, no method
arithmetic).

The arithmetic lives in ``sa_oracle.c`` (plain C, fp64, OpenMP over rows),
compiled here with gcc; ``extend`` (kept patterns -> descriptor) is plain numpy.
Citations are in the C source, by page title and section.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile sa_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Desc(C.Structure):
    _fields_ = [("S", C.c_int32), ("H", C.c_int32),
                ("diag_ptr", C.c_void_p), ("diag_off", C.c_void_p),
                ("vert_ptr", C.c_void_p), ("vert_col", C.c_void_p),
                ("block_mask", C.c_void_p), ("block_size", C.c_int32),
                ("stripe_ptr", C.c_void_p), ("stripe_col", C.c_void_p), ("stripe_rows", C.c_int32)]


class _Sizes(C.Structure):
    _fields_ = [("n_runs", C.c_int64), ("n_segs", C.c_int64), ("n_bcols", C.c_int64), ("n_cols", C.c_int64)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = C.CDLL(_LIB_PATH)
            lib.orc_row_mask.argtypes = [C.POINTER(_Desc), C.c_int32, C.c_int32, C.c_void_p]
            lib.orc_pair_count.argtypes = [C.POINTER(_Desc), C.c_void_p]
            lib.orc_build_index.restype = C.c_int
            lib.orc_build_index.argtypes = [C.POINTER(_Desc), C.c_int32] + \
                [C.c_void_p] * 3 + [C.c_int64] + [C.c_void_p] * 3 + [C.c_int64] + \
                [C.c_void_p] * 2 + [C.c_int64] + [C.c_void_p] * 2 + [C.c_int64] + [C.c_void_p, C.POINTER(_Sizes)]
            lib.orc_attention_rows.argtypes = [C.POINTER(_Desc), C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                                               C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                               C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p,
                                               C.c_void_p]
            lib.orc_attention_queries.argtypes = [C.POINTER(_Desc), C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                                                  C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                                  C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p,
                                                  C.c_void_p]
            lib.orc_attention_maps.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int32, C.c_int32, C.c_int32,
                                               C.c_int32, C.c_int32, C.c_double, C.c_void_p]
            lib.orc_capture.restype = C.c_int
            lib.orc_capture.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_double,
                                        C.c_double, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p]
            lib.orc_capture_scores.restype = C.c_int
            lib.orc_capture_scores.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_int32,
                                               C.c_void_p]
            lib.orc_sample_scores.restype = None
            lib.orc_sample_scores.argtypes = [C.c_void_p, C.c_void_p, C.c_int] + [C.c_int32] * 5 + \
                [C.c_double, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
            lib.orc_select_patterns.restype = None
            lib.orc_select_patterns.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_double, C.c_int64, C.c_int32,
                                                C.c_void_p]
            lib.orc_coverage.restype = None
            lib.orc_coverage.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p]
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class _DescHolder:
    """Keeps contiguous copies of the descriptor arrays alive while C reads them."""

    def __init__(self, d):
        self.arrays = dict(
            diag_ptr=np.ascontiguousarray(d.diag_ptr, dtype=np.int32),
            diag_off=np.ascontiguousarray(d.diag_off, dtype=np.int32),
            vert_ptr=np.ascontiguousarray(d.vert_ptr, dtype=np.int32),
            vert_col=np.ascontiguousarray(d.vert_col, dtype=np.int32),
            block_mask=None if d.block_mask is None else np.ascontiguousarray(d.block_mask, dtype=np.uint8),
            stripe_ptr=None if d.stripe_ptr is None else np.ascontiguousarray(d.stripe_ptr, dtype=np.int64),
            stripe_col=None if d.stripe_col is None else np.ascontiguousarray(d.stripe_col, dtype=np.int32),
        )
        a = self.arrays
        self.c = _Desc(d.S, d.H, _ptr(a["diag_ptr"]), _ptr(a["diag_off"]), _ptr(a["vert_ptr"]), _ptr(a["vert_col"]),
                       _ptr(a["block_mask"]), d.block_size, _ptr(a["stripe_ptr"]), _ptr(a["stripe_col"]),
                       d.stripe_rows)


def row_mask(desc, h: int, i: int) -> np.ndarray:
    """uint8[i+1]: 1 where (i, j) is retained for query head h."""
    lib = _load()
    hd = _DescHolder(desc)
    out = np.zeros(i + 1, dtype=np.uint8)
    lib.orc_row_mask(C.byref(hd.c), h, i, out.ctypes.data)
    return out


def pair_count(desc) -> np.ndarray:
    lib = _load()
    hd = _DescHolder(desc)
    out = np.zeros(desc.H, dtype=np.int64)
    lib.orc_pair_count(C.byref(hd.c), out.ctypes.data)
    return out


def build_index(desc, row_block: int, with_pairs: bool = True) -> dict:
    """Canonical index (runs, segments, in-segment columns, gathered columns, pair counts)."""
    lib = _load()
    hd = _DescHolder(desc)
    nb = -(-desc.S // row_block)
    nit = desc.H * nb
    run_ptr = np.zeros(desc.H + 1, np.int32)
    seg_ptr = np.zeros(nit + 1, np.int64)
    bcol_ptr = np.zeros(nit + 1, np.int64)
    col_ptr = np.zeros(nit + 1, np.int64)
    sz = _Sizes()
    rc0 = lib.orc_build_index(C.byref(hd.c), row_block, run_ptr.ctypes.data, None, None, 0,
                        seg_ptr.ctypes.data, None, None, 0, bcol_ptr.ctypes.data, None, 0,
                        col_ptr.ctypes.data, None, 0, None, C.byref(sz))
    if rc0 == 3:
        raise ValueError("row_block must divide block_size and stripe_rows")
    run_lo = np.zeros(max(sz.n_runs, 1), np.int32)
    run_hi = np.zeros(max(sz.n_runs, 1), np.int32)
    seg_lo = np.zeros(max(sz.n_segs, 1), np.int32)
    seg_hi = np.zeros(max(sz.n_segs, 1), np.int32)
    bcol = np.zeros(max(sz.n_bcols, 1), np.int32)
    col = np.zeros(max(sz.n_cols, 1), np.int32)
    pairs = np.zeros(desc.H, np.int64)
    rc = lib.orc_build_index(C.byref(hd.c), row_block, run_ptr.ctypes.data, run_lo.ctypes.data,
                             run_hi.ctypes.data, run_lo.size, seg_ptr.ctypes.data, seg_lo.ctypes.data,
                             seg_hi.ctypes.data, seg_lo.size, bcol_ptr.ctypes.data, bcol.ctypes.data, bcol.size,
                             col_ptr.ctypes.data, col.ctypes.data, col.size,
                             pairs.ctypes.data if with_pairs else None, C.byref(sz))
    assert rc == 0
    nwords = -(-desc.S // 32)
    dbits = np.zeros((desc.H, nwords), np.uint32)
    for h in range(desc.H):
        for r in desc.diags(h):   # bit r of head h: r is a diagonal offset
            dbits[h, r // 32] |= np.uint32(1) << np.uint32(r % 32)
    return dict(S=desc.S, n_heads=desc.H, row_block=row_block, n_row_blocks=nb, dbits=dbits.reshape(-1),
                run_ptr=run_ptr, run_lo=run_lo[:sz.n_runs], run_hi=run_hi[:sz.n_runs],
                seg_ptr=seg_ptr, seg_lo=seg_lo[:sz.n_segs], seg_hi=seg_hi[:sz.n_segs],
                bcol_ptr=bcol_ptr, bcol_idx=bcol[:sz.n_bcols], col_ptr=col_ptr, col_idx=col[:sz.n_cols],
                pair_count=pairs if with_pairs else None)


def attention_rows(desc, q, k, v, rows, scale: Optional[float] = None, mode: int = 0, return_counts: bool = False):
    """fp64 attention for the (b, h, i) triples in ``rows``.

    q [B,hq,S,d], k/v [B,hkv,S,d]: float32 arrays or uint16 bf16 bit patterns.
    mode 0 sums over retained keys only; mode 1 is the dense form with masked
    logits set to -inf.  Returns (o [n, d] float64, lse [n] float64) and, with
    return_counts, the number of retained keys of each row (int64 [n]).
    """
    lib = _load()
    hd = _DescHolder(desc)
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dtype = 0 if q.dtype == np.float32 else 1
    assert q.dtype in (np.float32, np.uint16) and k.dtype == q.dtype and v.dtype == q.dtype
    B, hq, S, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = rows.shape[0]
    o = np.zeros((n, d), np.float64)
    lse = np.zeros(n, np.float64)
    cnt = np.zeros(n, np.int64)
    lib.orc_attention_rows(C.byref(hd.c), q.ctypes.data, k.ctypes.data, v.ctypes.data, dtype, B, hq, hkv, S, d,
                           float(scale), rows.ctypes.data, n, mode, o.ctypes.data, lse.ctypes.data,
                           cnt.ctypes.data)
    return (o, lse, cnt) if return_counts else (o, lse)


def attention_queries(desc, qrows, k, v, rows, scale: Optional[float] = None, mode: int = 0):
    """fp64 attention of explicit query vectors: row n is query qrows[n] placed at position i of head h
    (rows[n] = (b, h, i)) against k/v [B,hkv,S,d] (the decode form).  Returns (o [n, d], lse [n])."""
    lib = _load()
    hd = _DescHolder(desc)
    qrows = np.ascontiguousarray(qrows)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dtype = 0 if qrows.dtype == np.float32 else 1
    assert qrows.dtype in (np.float32, np.uint16) and k.dtype == qrows.dtype and v.dtype == qrows.dtype
    B, hkv, S, d = k.shape
    hq = desc.H
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = rows.shape[0]
    assert qrows.shape == (n, d)
    o = np.zeros((n, d), np.float64)
    lse = np.zeros(n, np.float64)
    lib.orc_attention_queries(C.byref(hd.c), qrows.ctypes.data, k.ctypes.data, v.ctypes.data, dtype, hq, hkv, S, d,
                              float(scale), rows.ctypes.data, n, mode, o.ctypes.data, lse.ctypes.data, None)
    return o, lse


def attention_maps(q, k, scale: Optional[float] = None) -> np.ndarray:
    """Batch-averaged causal attention maps [hq, L, L] (float64) of q [B,hq,L,d] against k [B,hkv,L,d]."""
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    dtype = 0 if q.dtype == np.float32 else 1
    assert q.dtype in (np.float32, np.uint16) and k.dtype == q.dtype
    B, hq, L, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    maps = np.zeros((hq, L, L), np.float64)
    lib.orc_attention_maps(q.ctypes.data, k.ctypes.data, dtype, B, hq, hkv, L, d, float(scale), maps.ctypes.data)
    return maps


def capture(maps: np.ndarray, lam: float = 0.5, eps: float = 1e-8, tau: float = 0.3, mu: float = 0.8,
            norm_scope: int = 0, want_mask: bool = False) -> dict:
    """Pattern capture on float32 maps [n, L, L]: keep flags, hit counts, optional true mask."""
    lib = _load()
    maps = np.ascontiguousarray(maps, dtype=np.float32)
    n, L, _ = maps.shape
    kd = np.zeros((n, L), np.uint8)
    kv = np.zeros((n, L), np.uint8)
    hdg = np.zeros((n, L), np.int32)
    hv = np.zeros((n, L), np.int32)
    tm = np.zeros((n, L, L), np.uint8) if want_mask else None
    rc = lib.orc_capture(maps.ctypes.data, n, L, lam, eps, tau, mu, norm_scope, kd.ctypes.data, kv.ctypes.data,
                         hdg.ctypes.data, hv.ctypes.data, None if tm is None else tm.ctypes.data)
    if rc != 0:
        raise ValueError("lambda must be finite, and eps > 0 when lambda <= 0")
    return dict(keep_diag=kd, keep_vert=kv, diag_hits=hdg, vert_hits=hv, true_mask=tm)


def capture_scores(maps: np.ndarray, lam: float = 0.5, eps: float = 1e-8, norm_scope: int = 0) -> np.ndarray:
    """The normalised Box-Cox value t (float64 [n, L, L]) that capture compares with tau; NaN above the diagonal."""
    lib = _load()
    maps = np.ascontiguousarray(maps, dtype=np.float32)
    n, L, _ = maps.shape
    t = np.empty((n, L, L), np.float64)
    if lib.orc_capture_scores(maps.ctypes.data, n, L, lam, eps, norm_scope, t.ctypes.data) != 0:
        raise ValueError("lambda must be finite, and eps > 0 when lambda <= 0")
    return t


def coverage(maps: np.ndarray, keep_diag: np.ndarray, keep_vert: np.ndarray):
    """Per map: (attention mass share, cell count) of the kept patterns inside the L x L causal window."""
    lib = _load()
    maps = np.ascontiguousarray(maps, dtype=np.float32)
    n, L, _ = maps.shape
    kd = np.ascontiguousarray(keep_diag, dtype=np.uint8).reshape(n, L)
    kv = np.ascontiguousarray(keep_vert, dtype=np.uint8).reshape(n, L)
    mass = np.zeros(n, np.float64)
    cells = np.zeros(n, np.int64)
    lib.orc_coverage(maps.ctypes.data, n, L, kd.ctypes.data, kv.ctypes.data, mass.ctypes.data, cells.ctypes.data)
    return mass, cells


def extend(keep_diag: np.ndarray, keep_vert: np.ndarray, S: int):
    """Kept patterns of each map -> per-head descriptor lists at length S.

    [DAM] "What carries the argument" / "Circularity Check" step 1: the kept
    diagonal and vertical patterns are pasted into an S x S mask, which is the
    union of the matched patterns; a kept diagonal r keeps (i, i-r) and a kept
    vertical c keeps (i, c), i >= c, at every length.
    Returns (list of diagonal offset arrays, list of vertical column arrays).
    """
    diags = [np.nonzero(row)[0].astype(np.int32) for row in keep_diag]
    verts = [np.nonzero(row)[0].astype(np.int32) for row in keep_vert]
    diags = [d[d < S] for d in diags]
    verts = [c[c < S] for c in verts]
    return diags, verts


def sample_scores(q, k, row0: int, n_rows: int, band: int = 0, skip_cols: Optional[np.ndarray] = None,
                  scale: Optional[float] = None):
    """Runtime capture: per head, the attention mass that query rows row0 .. row0+n_rows-1 of every
    sequence put on each diagonal r and each vertical c, over the pairs outside the local window
    (i - j >= band) and off the columns in skip_cols (uint8 [hq, S]); float64 [hq, S] each, and
    each sampled row's natural-log LSE over all its keys [B, hq, n_rows]."""
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    assert q.dtype in (np.float32, np.uint16) and k.dtype == q.dtype
    dtype = 0 if q.dtype == np.float32 else 1
    B, hq, S, d = q.shape
    assert 0 <= row0 and row0 + n_rows <= S
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    skip = None if skip_cols is None else np.ascontiguousarray(skip_cols, dtype=np.uint8).reshape(hq, S)
    diag = np.zeros((hq, S), np.float64)
    vert = np.zeros((hq, S), np.float64)
    lse = np.zeros((B, hq, n_rows), np.float64)
    lib.orc_sample_scores(q.ctypes.data, k.ctypes.data, dtype, B, hq, k.shape[1], S, d, float(scale), row0, n_rows,
                          int(band), _ptr(skip), diag.ctypes.data, vert.ctypes.data, lse.ctypes.data)
    return diag, vert, lse


def fixed_point(x: np.ndarray) -> np.ndarray:
    """float64 masses -> int64 in units of 2^-32 (round to nearest)."""
    return np.rint(np.asarray(x, np.float64) * 4294967296.0).astype(np.int64)


def select_patterns(scores: np.ndarray, alpha: float, rows: int, band: int = 0) -> np.ndarray:
    """Keep flags (uint8 [n, S]) from integer scores of one family: the fewest top patterns that bring
    the covered mass of `rows` sampled rows to alpha (ties kept); patterns x < band always kept."""
    lib = _load()
    scores = np.ascontiguousarray(scores, dtype=np.int64)
    n, S = scores.shape
    keep = np.zeros((n, S), np.uint8)
    lib.orc_select_patterns(scores.ctypes.data, n, S, float(alpha), int(rows), int(band), keep.ctypes.data)
    return keep


def runtime_capture(q, k, row0: int, n_rows: int, alpha_cols: float, alpha: float, band: int,
                    scale: Optional[float] = None):
    """The two-stage per-input capture: the fewest columns that bring the covered mass (window
    counted) to alpha_cols, then the fewest diagonals, scored on the mass still uncovered, that bring
    it to alpha.  Returns keep_diag, keep_vert (uint8 [hq, S]) and the two stages' float64 scores."""
    B = q.shape[0]
    _, vert, _ = sample_scores(q, k, row0, n_rows, band=band, scale=scale)
    keep_vert = select_patterns(fixed_point(vert), alpha_cols, B * n_rows)
    diag, _, _ = sample_scores(q, k, row0, n_rows, band=band, skip_cols=keep_vert, scale=scale)
    keep_diag = select_patterns(fixed_point(diag), alpha, B * n_rows, band=band)
    return keep_diag, keep_vert, vert, diag
