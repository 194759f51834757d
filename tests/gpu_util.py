"""Helpers for the GPU parity tests (inputs from ``workloads``, expected values from ``oracle``)."""
import sys

import numpy as np
import torch

import workloads as W

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3   # bf16 path vs the fp64 oracle
F32_MAX_ABS = 1e-5                         # fp32 path vs the fp64 oracle


def sa():
    """The product package; raises (never skips) when libsa.so is missing."""
    import structured_sparse_attention_amd as m
    return m


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(x, device="cuda"):
    """numpy float32 or bf16 bit patterns (uint16) -> device tensor (float32 / bfloat16)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def widen(x):
    return W.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def rows_of_blocks(B, H, S, BM, blocks_per_head, rng):
    """(b, h, i) triples: every row of the first, the last and `blocks_per_head` seeded row blocks per head."""
    nb = -(-S // BM)
    out = []
    for b in range(B):
        for h in range(H):
            chosen = {0, nb - 1}
            if blocks_per_head and nb > 2:
                chosen |= set(rng.choice(np.arange(1, nb - 1), size=min(blocks_per_head, nb - 2),
                                         replace=False).tolist())
            for rb in sorted(chosen):
                for i in range(rb * BM, min(S, (rb + 1) * BM)):
                    out.append((b, h, i))
    return np.array(out, dtype=np.int32)


def all_rows(B, H, S):
    return np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S)], dtype=np.int32)


def gather_rows(o_dev, rows):
    """Rows (b, h, i) of a [B, H, S, d] device tensor -> float64 numpy [n, d]."""
    idx = torch.from_numpy(rows.astype(np.int64)).to(o_dev.device)
    sel = o_dev[idx[:, 0], idx[:, 1], idx[:, 2]]
    return sel.float().cpu().numpy().astype(np.float64)


def gather_lse(lse_dev, rows):
    idx = torch.from_numpy(rows.astype(np.int64)).to(lse_dev.device)
    return lse_dev[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)


def assert_close_bf16(got, ref, what=""):
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, "%s max-abs %.3g mean-abs %.3g" % (what, mx, mean)
    return mx, mean


def assert_close_f32(got, ref, what=""):
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= F32_MAX_ABS, "%s max-abs %.3g" % (what, mx)
    return mx


def assert_lse(got, ref, tol, what=""):
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), what + " empty-row pattern differs"
    fin = ~both_inf
    if fin.any():
        mx = float(np.abs(got[fin] - ref[fin]).max())
        assert mx <= tol, "%s lse max-abs %.3g" % (what, mx)


_MAPS = {}


def workload3_maps(layers=16, heads=32, n_avg=16):
    """The capture workload's maps (16 layers x 32 heads of 512 x 512 at n_avg = 16 by default), drawn once
    per process and shared by the tests that use them."""
    key = (layers, heads, n_avg)
    if key not in _MAPS:
        _MAPS[key] = W.capture_maps(layers=layers, heads=heads, n_avg=n_avg)
    return _MAPS[key]
