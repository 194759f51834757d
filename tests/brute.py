"""Brute-force numpy twins used to pin the CPU oracle on tiny inputs.

Written independently of ``oracle/sa_oracle.c``: masks are built as whole
S x S boolean matrices from the descriptor lists, attention is a dense masked
softmax over the full matrix.  Only meant for S up to a few hundred.
"""
import numpy as np


def mask_matrix(desc, h):
    """bool [S, S]: R_h(i, j) from the descriptor, built from whole-matrix numpy ops."""
    S = desc.S
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = np.zeros((S, S), dtype=bool)
    offs = desc.diags(h)
    if offs.size:
        m |= np.isin(i - j, offs)
    cols = desc.verts(h)
    if cols.size:
        m |= np.isin(j, cols) & np.ones((S, 1), dtype=bool)
    if desc.block_mask is not None:
        bs = desc.block_size
        m |= desc.block_mask[h][i // bs, j // bs].astype(bool)
    if desc.stripe_ptr is not None:
        sr = desc.stripe_rows
        for t in range(-(-S // sr)):
            cols_t = desc.stripe(h, t)
            rows = slice(t * sr, min(S, (t + 1) * sr))
            m[rows, cols_t] = True
    return m & (j <= i)


def column_set(desc, h, b0, b1):
    """X for rows [b0, b1]: verticals, the block row's blocks and the stripe's columns, all <= b1."""
    cols = set(int(c) for c in desc.verts(h) if c <= b1)
    if desc.block_mask is not None:
        bs = desc.block_size
        for bc in np.nonzero(desc.block_mask[h][b0 // bs])[0]:
            cols.update(range(bc * bs, min(b1 + 1, (bc + 1) * bs)))
    if desc.stripe_ptr is not None:
        cols.update(int(c) for c in desc.stripe(h, b0 // desc.stripe_rows) if c <= b1)
    return cols


def index_brute(desc, BM):
    S, H = desc.S, desc.H
    nb = -(-S // BM)
    out = dict(run_lo=[], run_hi=[], run_ptr=[0], seg_ptr=[0], seg_lo=[], seg_hi=[], bcol_ptr=[0], bcol_idx=[],
               col_ptr=[0], col_idx=[])
    for h in range(H):
        offs = sorted(int(x) for x in desc.diags(h))
        runs = []
        for r in offs:
            if runs and runs[-1][1] == r - 1:
                runs[-1][1] = r
            else:
                runs.append([r, r])
        for lo, hi in runs:
            out["run_lo"].append(lo)
            out["run_hi"].append(hi)
        out["run_ptr"].append(out["run_ptr"][-1] + len(runs))
    for h in range(H):
        offs = desc.diags(h)
        for rb in range(nb):
            b0, b1 = rb * BM, min(S, (rb + 1) * BM) - 1
            U = set()
            for r in offs:
                for i in range(b0, b1 + 1):
                    if i - r >= 0:
                        U.add(int(i - r))
            us = sorted(U)
            segs = []
            for jj in us:
                if segs and segs[-1][1] == jj - 1:
                    segs[-1][1] = jj
                else:
                    segs.append([jj, jj])
            for lo, hi in segs:
                out["seg_lo"].append(lo)
                out["seg_hi"].append(hi)
            out["seg_ptr"].append(out["seg_ptr"][-1] + len(segs))
            X = column_set(desc, h, b0, b1)
            bc = sorted(X & U)
            cc = sorted(X - U)
            out["bcol_idx"] += bc
            out["col_idx"] += cc
            out["bcol_ptr"].append(out["bcol_ptr"][-1] + len(bc))
            out["col_ptr"].append(out["col_ptr"][-1] + len(cc))
    return {k: np.asarray(v) for k, v in out.items()}


def attention_brute(desc, q, k, v, scale=None):
    """Full dense masked attention in float64 for every row. q/k/v float64 [B,H,S,d]."""
    B, hq, S, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    lse = np.zeros((B, hq, S))
    for h in range(hq):
        m = mask_matrix(desc, h)
        g = h // (hq // hkv)
        for b in range(B):
            s = (q[b, h] @ k[b, g].T) * scale
            s = np.where(m, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            empty = ~np.isfinite(mx[:, 0])
            mx[empty] = 0.0
            p = np.exp(s - mx)
            l = p.sum(axis=1, keepdims=True)
            with np.errstate(invalid="ignore", divide="ignore"):
                o[b, h] = np.where(empty[:, None], 0.0, (p @ v[b, g]) / l)
                lse[b, h] = np.where(empty, -np.inf, mx[:, 0] + np.log(l[:, 0]))
    return o, lse
