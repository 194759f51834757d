"""Benchmark: structured sparse prefill attention on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in HBM:
index build (count, scan, fill) from the pattern descriptor, then the sparse
attention forward.  Default workload: the LLaMA-3-8B-shaped layer (S = 65536,
32 query / 8 kv heads, d = 128, bf16; half vertical+slash heads, half 64x64
block-sparse heads).  Also reported: the attention time at S = 131072 (stripe
masks), the pattern-capture time on 16 x 32 maps of 512 x 512, one decode step
(16 sequences, one new query each, against 64K caches with the same patterns),
and the CPU oracle timed on a bounded sample of the same workload.

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOADS = {
    4: dict(name="llama8b_like", S=65536, hq=32, hkv=8, d=128, dtype="bf16", row_block=64),
    5: dict(name="long_stripes", S=131072, hq=32, hkv=8, d=128, dtype="bf16", row_block=128),
    2: dict(name="llama1b_like", S=8192, hq=32, hkv=8, d=64, dtype="bf16", row_block=64),
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def make_desc(W, cfg_id, S):
    if cfg_id == 4:
        return W.llama8b_like(S=S)
    if cfg_id == 5:
        return W.long_stripes(S=S)
    if cfg_id == 2:
        return W.llama1b_like(S=S)
    raise ValueError(cfg_id)


def to_dev(torch, x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def setup(cfg_id, B=1):
    import torch
    import structured_sparse_attention_amd as sa
    import workloads as W
    c = WORKLOADS[cfg_id]
    t = time.time()
    desc = make_desc(W, cfg_id, c["S"])
    q, k, v = W.qkv(cfg_id, B, c["hq"], c["hkv"], c["S"], c["d"], c["dtype"])
    log("generated workload %d (%s) in %.1fs" % (cfg_id, c["name"], time.time() - t))
    pat = sa.DevicePatterns.from_host(desc)
    qd, kd, vd = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
    ix = sa.build_index(pat, c["row_block"])
    torch.cuda.synchronize()
    return desc, (q, k, v), pat, (qd, kd, vd), ix


def time_attention_only(sa, torch, qkv_dev, ix, reps):
    qd, kd, vd = qkv_dev
    o = torch.empty_like(qd)
    sa.sparse_attn_prefill(qd, kd, vd, ix, out=o)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        sa.sparse_attn_prefill(qd, kd, vd, ix, out=o)
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def cpu_baseline(desc, qkv_host, cfg, target_s=15.0):
    """The oracle as it stands, on a bounded sample of whole row blocks (seeded), all host threads."""
    import oracle
    q, k, v = qkv_host
    S, hq, BM, d = cfg["S"], cfg["hq"], cfg["row_block"], cfg["d"]
    nb = -(-S // BM)
    rng = np.random.default_rng(1234)

    def sample(n_per_head):
        rows = []
        for h in range(hq):
            for rb in rng.choice(nb, size=n_per_head, replace=False):
                rows += [(0, h, i) for i in range(rb * BM, min(S, (rb + 1) * BM))]
        return np.array(rows, dtype=np.int32)

    t = time.time()
    rows = sample(1)
    _, _, cnt = oracle.attention_rows(desc, q, k, v, rows, return_counts=True)
    dt = time.time() - t
    n = max(1, min(nb, int(target_s / max(dt, 1e-3))))
    if n > 1:
        rows = sample(n)
        t = time.time()
        _, _, cnt = oracle.attention_rows(desc, q, k, v, rows, return_counts=True)
        dt = time.time() - t
    flops = 4.0 * d * float(cnt.sum())
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle", cpu=cpu_model(),
                sample="%d whole row blocks per head (%d rows, %d retained pairs, seeded), fp64 sparse "
                       "enumeration, %.1f s" % (n, len(rows), int(cnt.sum()), dt),
                seconds=dt)


def cpu_small_workloads():
    """The oracle on the three smaller workloads, whole problems: the tiny fp32 case and the 1B-shaped
    layer (every row of every head, sparse enumeration), and the capture of the 512 maps."""
    import oracle
    import workloads as W
    out = {}
    desc = W.tiny("base")
    q, k, v = W.qkv(1, 1, 1, 1, 512, 64, "f32")
    rows = np.array([(0, 0, i) for i in range(512)], dtype=np.int32)
    t = time.time()
    oracle.attention_rows(desc, q, k, v, rows)
    out["tiny_fp32_s"] = time.time() - t
    desc = W.llama1b_like()
    q, k, v = W.qkv(2, 1, 32, 8, 8192, 64, "bf16")
    rows = np.array([(0, h, i) for h in range(32) for i in range(8192)], dtype=np.int32)
    t = time.time()
    _, _, cnt = oracle.attention_rows(desc, q, k, v, rows, return_counts=True)
    out["llama1b_like_s"] = time.time() - t
    out["llama1b_like_tflops"] = 4.0 * 64 * float(cnt.sum()) / out["llama1b_like_s"] / 1e12
    maps = W.capture_maps(layers=16, heads=32, n_avg=16)
    t = time.time()
    oracle.capture(maps)
    out["capture_512_maps_s"] = time.time() - t
    return out


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; lscpu is not always installed)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_call(torch, fn, reps=10):
    """Mean HIP-event time (ms) of fn() on the current stream, after one untimed call."""
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def small_workloads(sa, torch):
    """The three smaller workloads' attention (and index refill) times: the tiny fp32 case (S = 512, one
    head, d = 64, diagonals 0..63 + verticals), the 1B-shaped layer (S = 8192, 32/8 heads, d = 64) and the
    capture workload's attention run (16 layers, each one call at S = 16384, 32/8 heads, d = 64, on the
    layer's kept sets from the GPU capture of its 32 maps, extended to S)."""
    import workloads as W
    out = {}
    # workload 1
    desc = W.tiny("base")
    q, k, v = W.qkv(1, 1, 1, 1, 512, 64, "f32")
    pat = sa.DevicePatterns.from_host(desc)
    ix = sa.build_index(pat, 64)
    qd, kd, vd = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
    o = torch.empty_like(qd)
    ms = time_call(torch, lambda: sa.sparse_attn_prefill(qd, kd, vd, ix, out=o), reps=50)
    ims = time_call(torch, lambda: sa.refill_index(pat, ix), reps=50)
    out["tiny_fp32"] = dict(S=512, heads="1/1", d=64, attn_ms=ms, index_ms=ims, retained_pairs=ix.total_pairs,
                            effective_tflops=4.0 * 64 * ix.total_pairs / (ms * 1e-3) / 1e12,
                            frac_of_fp32_peak=4.0 * 64 * ix.total_pairs / (ms * 1e-3) / 1e12 / PEAK_F32_TFLOPS)
    # workload 2
    desc = W.llama1b_like()
    q, k, v = W.qkv(2, 1, 32, 8, 8192, 64, "bf16")
    pat = sa.DevicePatterns.from_host(desc)
    ix = sa.build_index(pat, 64)
    qd, kd, vd = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
    o = torch.empty_like(qd)
    ms = time_call(torch, lambda: sa.sparse_attn_prefill(qd, kd, vd, ix, out=o))
    ims = time_call(torch, lambda: sa.refill_index(pat, ix))
    out["llama1b_like"] = dict(S=8192, heads="32/8", d=64, attn_ms=ms, index_ms=ims, retained_pairs=ix.total_pairs,
                               effective_tflops=4.0 * 64 * ix.total_pairs / (ms * 1e-3) / 1e12)
    del qd, kd, vd, o
    # workload 3: capture of the 512 maps on the GPU, then one attention call per layer at S = 16384
    maps = torch.from_numpy(W.capture_maps(layers=16, heads=32, n_avg=16)).cuda()
    cap = sa.pattern_capture(maps)
    S = 16384
    total_ms, pairs = 0.0, 0
    for layer in range(16):
        kd_ = cap["keep_diag"][32 * layer:32 * (layer + 1)].contiguous()
        kv_ = cap["keep_vert"][32 * layer:32 * (layer + 1)].contiguous()
        ix = sa.build_index(sa.patterns_to_desc(kd_, kv_, S), 64)
        q, k, v = W.qkv(3, 1, 32, 8, S, 64, "bf16", seed_extra=layer)
        qd, kd, vd = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
        o = torch.empty_like(qd)
        total_ms += time_call(torch, lambda: sa.sparse_attn_prefill(qd, kd, vd, ix, out=o), reps=5)
        pairs += ix.total_pairs
    del maps
    out["capture_16_layers_S16384"] = dict(S=S, heads="32/8", d=64, layers=16, attn_ms=total_ms, retained_pairs=pairs,
                                           effective_tflops=4.0 * 64 * pairs / (total_ms * 1e-3) / 1e12)
    return out


def capture_ms(sa, torch, reps=20):
    import workloads as W
    maps = W.capture_maps(layers=16, heads=32, n_avg=4)
    md = torch.from_numpy(maps).cuda()
    out = sa.pattern_capture(md)   # outputs reused below, so the timed calls allocate nothing
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        sa.pattern_capture(md, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    causal_bytes = 4.0 * maps.shape[0] * 512 * 513 / 2
    return dict(ms=ms, maps=int(maps.shape[0]), L=512, read_GBps=causal_bytes / (ms * 1e-3) / 1e9)


def maps_from_qk_ms(sa, torch, reps=10, warm=3):
    """Capture maps from Q/K: 16 layers x 32 query heads (8 kv heads per layer) stacked into one
    call, batch 16, L = 512, d = 64 (bf16), then the capture of those 512 maps.  One layer's
    structured Q/K is generated and repeated over the 16 layers (the work does not depend on values)."""
    import workloads as W
    q, k = W.capture_qk(47, 16, 32, 8, 512, 64, "bf16")
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16).repeat(1, 16, 1, 1).contiguous()
    kd = torch.from_numpy(k.view(np.int16)).cuda().view(torch.bfloat16).repeat(1, 16, 1, 1).contiguous()
    maps = torch.empty((512, 512, 512), dtype=torch.float32, device="cuda")
    for _ in range(warm):
        sa.attention_maps(qd, kd, out=maps)
    cap = sa.pattern_capture(maps)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(reps):
        sa.attention_maps(qd, kd, out=maps)
    ev[1].record()
    for _ in range(reps):
        sa.pattern_capture(maps, out=cap)
    ev[2].record()
    torch.cuda.synchronize()
    maps_ms, cap_ms = ev[0].elapsed_time(ev[1]) / reps, ev[1].elapsed_time(ev[2]) / reps
    nrb = 512 // 64
    flops = 2.0 * 2 * 16 * 512 * (nrb * (nrb + 1) // 2) * 64 * 64 * 64   # two score passes over the computed tiles
    return dict(maps_ms=maps_ms, capture_ms=cap_ms, B=16, heads=512, L=512, d=64,
                maps_tile_TFLOPs=flops / (maps_ms * 1e-3) / 1e12)


SWEEP_LAMBDA = (-0.5, 0.0, 0.25, 0.5, 1.0)
SWEEP_TAU = (0.1, 0.2, 0.3, 0.4, 0.5)
SWEEP_MU = (0.6, 0.7, 0.8, 0.9, 1.0)
SWEEP_PCL = (256, 512, 1024)


def capture_sweep(sa, torch, S=16384):
    """Sensitivity of the kept masks to the capture length (PCL), lambda, tau and mu, on two kinds of
    synthetic maps per PCL: the pattern-capture workload's maps (32 heads, 16 averaged softmaxes) and
    maps computed on the GPU from structured Q/K (batch 16, 32/8 heads, d 64).  For every grid point:
    kept diagonals and verticals per head, the kept patterns' share of the attention mass and of the
    cells inside the L x L window (sa_pattern_coverage), and the density of the mask extended to S
    (exact retained pairs from the index over all causal pairs)."""
    import workloads as W
    out = []
    causal_S = 32 * S * (S + 1) / 2.0
    for L in SWEEP_PCL:
        srcs = []
        t0 = time.time()
        srcs.append(("workload maps", torch.from_numpy(W.capture_maps(layers=1, heads=32, L=L, n_avg=16)).cuda()))
        q, k = W.capture_qk(48, 16, 32, 8, L, 64, "bf16")
        qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
        kd = torch.from_numpy(k.view(np.int16)).cuda().view(torch.bfloat16)
        srcs.append(("maps from Q/K", sa.attention_maps(qd, kd)))
        log("sweep: PCL %d maps ready in %.1fs" % (L, time.time() - t0))
        for name, maps in srcs:
            for lam in SWEEP_LAMBDA:
                for tau in SWEEP_TAU:
                    for mu in SWEEP_MU:
                        c = sa.pattern_capture(maps, lam=lam, tau=tau, mu=mu, return_hits=False)
                        mass, cells = sa.pattern_coverage(maps, c["keep_diag"], c["keep_vert"])
                        ix = sa.build_index(sa.patterns_to_desc(c["keep_diag"], c["keep_vert"], S), 64)
                        out.append(dict(maps=name, pcl=L, lam=lam, tau=tau, mu=mu,
                                        diags=float(c["keep_diag"].float().sum(1).mean().item()),
                                        verts=float(c["keep_vert"].float().sum(1).mean().item()),
                                        mass=float(mass.mean().item()), mass_min=float(mass.min().item()),
                                        cells=float(cells.double().mean().item()) / (L * (L + 1) / 2.0),
                                        density_S=ix.total_pairs / causal_S))
    # timing of one capture of the 512 workload maps per transform kind
    maps = torch.from_numpy(W.capture_maps(layers=16, heads=32, n_avg=4)).cuda()
    timing = {}
    for lam in (0.5, 0.0, 0.25):
        sa.pattern_capture(maps, lam=lam)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            sa.pattern_capture(maps, lam=lam)
        b.record()
        torch.cuda.synchronize()
        timing[str(lam)] = a.elapsed_time(b) / 5
    return dict(S=S, points=out, capture_ms_512_maps=timing)


def machine_calibration(sa, torch, reps=5):
    """Measured counterparts of the vendor figures used for the rooflines: dense bf16 MFMA throughput
    (sa_calib_mfma_bf16: 2048 workgroups x 4 waves x 2048 rounds x 4 MFMAs of 32x32x16) and random 16 KiB
    chunk reads (sa_calib_gather: 8192 workgroups x 16 chunks = 2 GiB requested) from regions of 2 MiB
    (L2), 32 MiB, 256 MiB (the MALL's size) and 2 GiB (HBM)."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    n_wg, iters = 2048, 2048
    ms = timed(lambda: sa.calib_mfma_bf16(n_wg, iters))
    out = dict(mfma_bf16_dense_TFLOPs=n_wg * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12)
    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    gather = {}
    for name, region in (("2MiB", 2 << 20), ("32MiB", 32 << 20), ("256MiB", 256 << 20), ("2GiB", 1 << 31)):
        ms = timed(lambda: sa.calib_gather(buf, region, 16384, 8192, 16))
        gather[name] = 8192 * 16 * 16384 / (ms * 1e-3) / 1e12
    del buf
    out["random_16KiB_read_TBps"] = gather
    return out


def decode_row_keys(ixn, h, t, nb, BM, nwords):
    """Retained keys of row t of head h, read off the index (segments filtered by the diagonal bitmap
    and the in-segment columns, then the gathered columns <= t)."""
    it = h * nb + t // BM
    dbits = ixn["dbits"].reshape(-1, nwords)[h]
    bcols = ixn["bcol_idx"][ixn["bcol_ptr"][it]:ixn["bcol_ptr"][it + 1]]
    n = 0
    for s in range(ixn["seg_ptr"][it], ixn["seg_ptr"][it + 1]):
        lo, hi = int(ixn["seg_lo"][s]), min(int(ixn["seg_hi"][s]), t)
        if lo > t:
            break
        js = np.arange(lo, hi + 1)
        r = t - js
        on = ((dbits[r >> 5] >> (r & 31)) & 1).astype(bool) | np.isin(js, bcols)
        n += int(on.sum())
    cols = ixn["col_idx"][ixn["col_ptr"][it]:ixn["col_ptr"][it + 1]]
    return n + int((cols <= t).sum())


def runtime_capture_bench(sa, torch, S=65536, n_rows=128, band=1024, alpha_cols=0.8, alpha=0.9, reps=3):
    """Per-input capture then attention at the 64K layer shape (batch 1, 32/8 heads, head_dim 128,
    bf16): the last `n_rows` query rows are sampled; columns to alpha_cols of the sampled mass, then
    diagonals on the mass the columns leave, to alpha; window of `band` diagonals; the kept patterns
    are extended to S, indexed and run.
    Q/K carry sinks, seeded columns and a positional band (workloads.runtime_qk); V is N(0,1)."""
    import workloads as W
    t0 = time.time()
    q, k = W.runtime_qk(84, 1, 32, 8, S, 128, "bf16")
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    kd = torch.from_numpy(k.view(np.int16)).cuda().view(torch.bfloat16)
    del q, k
    gen = torch.Generator(device="cuda")
    gen.manual_seed(84)
    vd = torch.randn(kd.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    log("runtime capture: inputs ready in %.1fs" % (time.time() - t0))
    row0 = S - n_rows

    def capture():
        _, vs, lse = sa.sample_scores(qd, kd, row0, n_rows, band=band, families=(False, True))
        keep_v = sa.select_patterns(vs, alpha_cols, n_rows)
        ds, _, _ = sa.sample_scores(qd, kd, row0, n_rows, band=band, skip_cols=keep_v, row_lse=lse, lse_given=True,
                                    families=(True, False))
        keep_d = sa.select_patterns(ds, alpha, n_rows, band=band)
        return keep_d, keep_v

    keep_d, keep_v = capture()
    ix = sa.build_index(sa.patterns_to_desc(keep_d, keep_v, S), 64)
    o = sa.sparse_attn_prefill(qd, kd, vd, ix)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    cap_ms, full_ms, attn_ms = [], [], []
    for _ in range(reps):
        ev[0].record()
        keep_d, keep_v = capture()
        ev[1].record()
        ix = sa.build_index(sa.patterns_to_desc(keep_d, keep_v, S), 64)   # size query: one host sync
        a0 = torch.cuda.Event(enable_timing=True)
        a0.record()
        sa.sparse_attn_prefill(qd, kd, vd, ix, out=o)
        ev[2].record()
        torch.cuda.synchronize()
        cap_ms.append(ev[0].elapsed_time(ev[1]))
        full_ms.append(ev[0].elapsed_time(ev[2]))
        attn_ms.append(a0.elapsed_time(ev[2]))
    pairs = ix.total_pairs
    cap, full, att = min(cap_ms), min(full_ms), min(attn_ms)
    return dict(workload="runtime capture: last %d rows sampled, window %d, columns to %g, diagonals to %g, 64K layer "
                         "shape" % (n_rows, band, alpha_cols, alpha),
                S=S, capture_ms=cap, index_and_attention_ms=full - cap, attention_ms=att, total_ms=full,
                kept_columns_per_head=float(keep_v.float().sum(1).mean().item()),
                kept_diagonals_beyond_window_per_head=float(keep_d.float().sum(1).mean().item()) - band,
                retained_pairs=pairs, density=pairs / (32 * S * (S + 1) / 2.0),
                effective_tflops=4.0 * 128 * pairs / (att * 1e-3) / 1e12)


def decode_bench(sa, torch, B=16, reps=20):
    """Decode (one new query per sequence) on the 64K workload's patterns: B sequences whose
    positions sit near the end of a 64K cache, all 32 query heads."""
    import workloads as W
    cfg = WORKLOADS[4]
    S, hq, hkv, d, BM = cfg["S"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["row_block"]
    desc = W.llama8b_like(S=S)
    ix = sa.build_index(sa.DevicePatterns.from_host(desc), BM)
    g = torch.Generator(device="cuda").manual_seed(4)
    k = torch.randn(B, hkv, S, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, hkv, S, d, device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn(B, hq, d, device="cuda", generator=g).to(torch.bfloat16)
    pos_h = [S - 1 - 37 * b for b in range(B)]
    pos = torch.tensor(pos_h, dtype=torch.int32, device="cuda")
    o = sa.sparse_attn_decode(q, k, v, pos, ix)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        sa.sparse_attn_decode(q, k, v, pos, ix, out=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    ixn = ix.to_numpy()
    nw = -(-S // 32)
    keys = sum(decode_row_keys(ixn, h, t, ix.n_row_blocks, BM, nw) for t in pos_h for h in range(hq))
    kv_bytes = keys * 2 * d * 2  # one K row and one V row (bf16) per retained key and query head
    del k, v, q, o, ix
    torch.cuda.empty_cache()
    return dict(workload="llama8b_like patterns, %d sequences at positions %d..%d of a %d-row cache, %d/%d heads, "
                          "head_dim %d, bf16" % (B, pos_h[-1], pos_h[0], S, hq, hkv, d),
                ms=ms, tokens_per_s=B / (ms * 1e-3), retained_keys=keys, kv_bytes=kv_bytes,
                kv_GBps=kv_bytes / (ms * 1e-3) / 1e9, kv_frac_of_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)


def measured_traffic(cfg):
    """HBM bytes per launch of the attention kernel, from profiles/traffic.json (hardware counters
    FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy), or None when the kernel source has changed
    since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "structured_sparse_attention_amd", "csrc", "sa_attn.hip")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    entry = rec.get(cfg["name"])
    if not entry or entry.get("sa_attn_sha256") != digest:
        return None
    return entry.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the S=131072 and capture measurements")
    ap.add_argument("--capture-sweep", action="store_true",
                    help="only run the capture sensitivity sweep (PCL, lambda, tau, mu) and print it as JSON")
    ap.add_argument("--capture-only", action="store_true",
                    help="only time the capture of the 512 workload maps and of the 512 maps from Q/K (JSON)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one device copy of 1 GiB (reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the work would shard by "
              "query heads, one kv group per GPU); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import structured_sparse_attention_amd as sa

    if args.capture_sweep:
        print(json.dumps(capture_sweep(sa, torch)))
        return
    if args.capture_only:
        print(json.dumps(dict(capture=capture_ms(sa, torch), capture_from_qk=maps_from_qk_ms(sa, torch))))
        return

    cfg = WORKLOADS[args.config]
    desc, qkv_host, pat, qkv_dev, ix = setup(args.config)
    qd, kd, vd = qkv_dev
    o = torch.empty_like(qd)
    pairs = ix.total_pairs
    B = qd.shape[0]
    flops = 4.0 * cfg["d"] * pairs * B

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sa.refill_index(pat, ix)
        if ev is not None:
            ev[1].record()
        sa.sparse_attn_prefill(qd, kd, vd, ix, out=o)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = float(np.mean([a1.elapsed_time(a2) for _, a1, a2 in evs]))
    index_ms = float(np.mean([a0.elapsed_time(a1) for a0, a1, _ in evs]))
    assert int(ix.status.item()) == 0
    log("step %.3f ms (index %.3f ms, attention %.3f ms), %d retained pairs" % (ms_per_step, index_ms, attn_ms,
                                                                              pairs))

    prefill_ms = {str(cfg["S"]): attn_ms}
    extras = {}
    if not args.no_extras:
        del o, qd, kd, vd, qkv_dev
        torch.cuda.empty_cache()
        other = 5 if args.config != 5 else 4
        ocfg = WORKLOADS[other]
        _, _, opat, oqkv, oix = setup(other)
        oms = time_attention_only(sa, torch, oqkv, oix, reps=5)
        prefill_ms[str(ocfg["S"])] = oms
        extras["other_workload"] = dict(workload=ocfg["name"], S=ocfg["S"], attn_ms=oms,
                                        effective_tflops=4.0 * ocfg["d"] * oix.total_pairs / (oms * 1e-3) / 1e12,
                                        retained_pairs=oix.total_pairs)
        log("workload %s: attention %.3f ms" % (ocfg["name"], oms))
        del oqkv, oix, opat
        torch.cuda.empty_cache()
        extras["capture"] = capture_ms(sa, torch)
        log("capture: %.3f ms" % extras["capture"]["ms"])
        extras["capture_from_qk"] = maps_from_qk_ms(sa, torch)
        log("capture from Q/K: maps %.3f ms + capture %.3f ms" % (extras["capture_from_qk"]["maps_ms"],
                                                                extras["capture_from_qk"]["capture_ms"]))
        extras["runtime_capture"] = runtime_capture_bench(sa, torch)
        rc = extras["runtime_capture"]
        log("runtime capture at 64K: capture %.3f ms, index + attention %.3f ms (attention %.3f ms), density %.4f"
            % (rc["capture_ms"], rc["index_and_attention_ms"], rc["attention_ms"], rc["density"]))
        extras["decode"] = decode_bench(sa, torch)
        extras["small_workloads"] = small_workloads(sa, torch)
        sw = extras["small_workloads"]
        log("tiny fp32: %.4f ms; 1B-like S=8192: %.3f ms (%.0f TFLOP/s); capture run, 16 layers at S=16384: %.3f ms "
            "(%.0f TFLOP/s)" % (sw["tiny_fp32"]["attn_ms"], sw["llama1b_like"]["attn_ms"],
                                sw["llama1b_like"]["effective_tflops"], sw["capture_16_layers_S16384"]["attn_ms"],
                                sw["capture_16_layers_S16384"]["effective_tflops"]))
        extras["machine"] = machine_calibration(sa, torch)
        log("machine: dense bf16 MFMA %.0f TFLOP/s; random 16 KiB reads %s TB/s" % (
            extras["machine"]["mfma_bf16_dense_TFLOPs"],
            ", ".join("%s %.1f" % kv for kv in extras["machine"]["random_16KiB_read_TBps"].items())))
        log("decode: %.3f ms for %d tokens (%.0f GB/s of retained K/V rows)" % (
            extras["decode"]["ms"], 16, extras["decode"]["kv_GBps"]))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(desc, qkv_host, cfg)
        log("cpu oracle: %.4f TFLOP/s on %d threads (%s)" % (cpu["value"], cpu["cores"], cpu["sample"]))
        if not args.no_extras:
            cpu["small_workloads"] = cpu_small_workloads()
            log("cpu oracle, smaller workloads: %s" % json.dumps(cpu["small_workloads"]))

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    achieved = flops / (attn_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(cfg),
                "kernel": "attention forward, bf16, head_dim %d, row block %d" % (cfg["d"], cfg["row_block"])}
    if "machine" in extras:
        # the same launch against what this chip measurably sustains: dense bf16 MFMA from registers, and
        # random 16 KiB reads from a region the size of one kv head's K/V (the fabric ceiling of the gathers)
        mfma = extras["machine"]["mfma_bf16_dense_TFLOPs"]
        roofline["measured_peak"] = mfma
        roofline["frac_of_measured_peak"] = achieved / mfma
        tr = roofline["traffic"]
        if tr:
            gb = extras["machine"]["random_16KiB_read_TBps"]["32MiB"]
            roofline["traffic_TBps"] = tr / (attn_ms * 1e-3) / 1e12
            roofline["traffic_frac_of_measured_gather"] = roofline["traffic_TBps"] / gb
    out = {
        "metric": "effective TFLOP/s (retained pairs) + prefill attn ms at S=64K/131K, 1 GPU",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": "%s: batch 1, S=%d, %d q / %d kv heads, head_dim %d, row block %d"
                               % (cfg["name"], cfg["S"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["row_block"]),
                   "batch": B, "seq_len": cfg["S"], "hq": cfg["hq"], "hkv": cfg["hkv"], "head_dim": cfg["d"]},
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind", "sample",
                                                                         "cpu", "small_workloads") if k2 in cpu},
        "prefill_attn_ms": prefill_ms,
        "index_build_ms": index_ms,
        "retained_pairs": pairs,
        "effective_flops_per_step": flops,
    }
    out.update(extras)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
