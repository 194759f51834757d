"""structured_sparse_attention_amd -- Python binding of libsa.so (gfx950).

Argument marshalling only: every step of the path (index build, sparse attention,
decode, attention maps, pattern capture and coverage, pattern extension, runtime
capture from sampled rows) runs in the HIP kernels of ``libsa.so``;
PyTorch supplies device memory and the current HIP stream.  The C ABI is declared
in ``include/sa.h``.  Importing this package loads ``libsa.so`` and raises if it
has not been built (``python structured_sparse_attention_amd/build.py``); there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional

import numpy as np
import torch

__all__ = ["SAError", "DevicePatterns", "SparseIndex", "build_index", "sparse_attn_prefill", "sparse_attn_decode",
           "attention_maps", "pattern_capture", "pattern_coverage", "patterns_to_desc", "sample_scores",
           "select_patterns", "calib_mfma_bf16", "calib_gather", "library_path", "version", "lib"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsa.so")

SA_DTYPE_F32, SA_DTYPE_BF16 = 0, 1
SA_BUILD_VALIDATE = 1
STATUS_OVERFLOW, STATUS_DESC_INVALID = 1, 2


class SAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, _lib.sa_status_string(code).decode(), code))


class _Desc(C.Structure):
    _fields_ = [("S", C.c_int32), ("n_heads", C.c_int32),
                ("diag_ptr", C.c_void_p), ("diag_off", C.c_void_p), ("vert_ptr", C.c_void_p),
                ("vert_col", C.c_void_p), ("block_mask", C.c_void_p), ("block_size", C.c_int32),
                ("stripe_ptr", C.c_void_p), ("stripe_col", C.c_void_p), ("stripe_rows", C.c_int32)]


class _Sizes(C.Structure):
    _fields_ = [("n_runs", C.c_int64), ("n_segs", C.c_int64), ("n_bcols", C.c_int64), ("n_cols", C.c_int64)]


class _Index(C.Structure):
    _fields_ = [("S", C.c_int32), ("n_heads", C.c_int32), ("row_block", C.c_int32), ("n_row_blocks", C.c_int32),
                ("run_ptr", C.c_void_p), ("run_lo", C.c_void_p), ("run_hi", C.c_void_p),
                ("seg_ptr", C.c_void_p), ("seg_lo", C.c_void_p), ("seg_hi", C.c_void_p),
                ("bcol_ptr", C.c_void_p), ("bcol_idx", C.c_void_p), ("col_ptr", C.c_void_p),
                ("col_idx", C.c_void_p), ("pair_count", C.c_void_p), ("dbits", C.c_void_p),
                ("status", C.c_void_p), ("capacity", _Sizes)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libsa.so is not built (%s); run `python structured_sparse_attention_amd/build.py`"
                          % _LIB_PATH)
    lib = C.CDLL(_LIB_PATH)
    lib.sa_status_string.restype = C.c_char_p
    lib.sa_status_string.argtypes = [C.c_int32]
    lib.sa_version.restype = C.c_char_p
    lib.sa_version.argtypes = []
    lib.sa_build_index.restype = C.c_int32
    lib.sa_build_index.argtypes = [C.POINTER(_Desc), C.POINTER(_Index), C.POINTER(_Sizes), C.c_int32, C.c_void_p]
    lib.sa_sparse_attn_prefill.restype = C.c_int32
    lib.sa_sparse_attn_prefill.argtypes = [C.c_void_p] * 4 + [C.c_void_p] + [C.c_int32] * 6 + \
        [C.c_float, C.POINTER(_Index), C.c_void_p]
    lib.sa_sparse_attn_decode.restype = C.c_int32
    lib.sa_sparse_attn_decode.argtypes = [C.c_void_p] * 6 + [C.c_int32] * 6 + [C.c_float, C.POINTER(_Index),
                                                                                 C.c_void_p]
    lib.sa_attention_maps.restype = C.c_int32
    lib.sa_attention_maps.argtypes = [C.c_void_p, C.c_void_p] + [C.c_int32] * 6 + [C.c_float, C.c_void_p, C.c_void_p]
    lib.sa_pattern_capture.restype = C.c_int32
    lib.sa_pattern_capture.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_double,
                                       C.c_double, C.c_int32] + [C.c_void_p] * 5 + [C.c_void_p]
    lib.sa_sample_scores.restype = C.c_int32
    lib.sa_sample_scores.argtypes = [C.c_void_p, C.c_void_p] + [C.c_int32] * 6 + [C.c_float] + [C.c_int32] * 3 + \
        [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t] + [C.c_void_p] * 2 + [C.c_void_p]
    lib.sa_sample_scores_noalloc.restype = C.c_int32
    lib.sa_sample_scores_noalloc.argtypes = [C.c_void_p, C.c_void_p] + [C.c_int32] * 6 + [C.c_float] + \
        [C.c_int32] * 3 + [C.c_void_p, C.c_int32, C.c_void_p] + [C.c_void_p] * 2 + [C.c_void_p]
    lib.sa_build_index_workspace_bytes.restype = C.c_size_t
    lib.sa_build_index_workspace_bytes.argtypes = [C.c_void_p, C.c_int32]
    lib.sa_sample_scores_workspace.restype = C.c_size_t
    lib.sa_sample_scores_workspace.argtypes = [C.c_int32] * 4
    lib.sa_select_patterns.restype = C.c_int32
    lib.sa_select_patterns.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_double, C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_void_p]
    lib.sa_pattern_coverage.restype = C.c_int32
    lib.sa_pattern_coverage.argtypes = [C.c_void_p, C.c_int32, C.c_int32] + [C.c_void_p] * 4 + [C.c_void_p]
    lib.sa_calib_mfma_bf16.restype = C.c_int32
    lib.sa_calib_mfma_bf16.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    lib.sa_calib_gather.restype = C.c_int32
    lib.sa_calib_gather.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_uint64, C.c_void_p,
                                    C.c_void_p]
    lib.sa_patterns_to_desc.restype = C.c_int32
    lib.sa_patterns_to_desc.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32] + \
        [C.c_void_p] * 4 + [C.c_void_p]
    return lib


_lib = _load()
lib = _lib


def calib_mfma_bf16(n_workgroups: int, iters: int, stream=None) -> torch.Tensor:
    """sa_calib_mfma_bf16 (measurement support): launches the dense bf16 MFMA loop; returns its sink."""
    sink = torch.empty(n_workgroups * 256, dtype=torch.float32, device="cuda")
    _check(_lib.sa_calib_mfma_bf16(n_workgroups, iters, sink.data_ptr(), _stream(stream)), "sa_calib_mfma_bf16")
    return sink


def calib_gather(buf: torch.Tensor, region_bytes: int, chunk_bytes: int, n_workgroups: int, reads: int, seed: int = 1,
                 stream=None) -> torch.Tensor:
    """sa_calib_gather (measurement support): random chunk reads from buf[0 .. region_bytes); returns its sink."""
    if buf.numel() * buf.element_size() < region_bytes:
        raise ValueError("buf is smaller than region_bytes")
    sink = torch.empty(n_workgroups * 256, dtype=torch.float32, device=buf.device)
    _check(_lib.sa_calib_gather(buf.data_ptr(), region_bytes, chunk_bytes, n_workgroups, reads, seed, sink.data_ptr(),
                                _stream(stream)), "sa_calib_gather")
    return sink


def library_path() -> str:
    return _LIB_PATH


def version() -> str:
    return _lib.sa_version().decode()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _torch_stream(stream) -> torch.cuda.Stream:
    """The launch stream as a torch stream object (a raw hipStream_t handle is wrapped, not owned)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _hold(t: Optional[torch.Tensor], stream) -> None:
    """A temporary that a call on `stream` reads is not handed to another allocation before that stream
    has used it (torch's allocator otherwise only tracks the current stream).  Raw stream handles
    cannot be tracked: with one, temporaries are made on the current stream and the caller orders it."""
    if t is not None and stream is not None and isinstance(stream, torch.cuda.Stream):
        t.record_stream(stream)


def _check(code: int, where: str):
    if code != 0:
        raise SAError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev_array(a, dtype: torch.dtype, device) -> torch.Tensor:
    """Host or device array -> contiguous device tensor with at least one element."""
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
    t = t.to(device=device, dtype=dtype).contiguous()
    if t.numel() == 0:
        t = torch.zeros(1, dtype=dtype, device=device)
    return t


class DevicePatterns:
    """A pattern descriptor (see sa_pattern_desc in include/sa.h) held in device memory."""

    def __init__(self, S: int, n_heads: int, diag_ptr, diag_off, vert_ptr, vert_col, block_mask=None,
                 block_size: int = 64, stripe_ptr=None, stripe_col=None, stripe_rows: int = 128, device="cuda"):
        self.S, self.n_heads = int(S), int(n_heads)
        self.diag_ptr = _dev_array(diag_ptr, torch.int32, device)
        self.diag_off = _dev_array(diag_off, torch.int32, device)
        self.vert_ptr = _dev_array(vert_ptr, torch.int32, device)
        self.vert_col = _dev_array(vert_col, torch.int32, device)
        self.block_mask = None if block_mask is None else _dev_array(block_mask, torch.uint8, device)
        self.block_size = int(block_size)
        self.stripe_ptr = None if stripe_ptr is None else _dev_array(stripe_ptr, torch.int64, device)
        self.stripe_col = None if stripe_ptr is None else _dev_array(stripe_col, torch.int32, device)
        self.stripe_rows = int(stripe_rows)

    @classmethod
    def from_host(cls, desc, device="cuda") -> "DevicePatterns":
        """From any object with the descriptor fields (S, H or n_heads, diag_ptr, ...)."""
        H = getattr(desc, "n_heads", None) or getattr(desc, "H")
        return cls(desc.S, H, desc.diag_ptr, desc.diag_off, desc.vert_ptr, desc.vert_col,
                   getattr(desc, "block_mask", None), getattr(desc, "block_size", 64),
                   getattr(desc, "stripe_ptr", None), getattr(desc, "stripe_col", None),
                   getattr(desc, "stripe_rows", 128), device=device)

    def c_struct(self) -> _Desc:
        return _Desc(self.S, self.n_heads, _ptr(self.diag_ptr), _ptr(self.diag_off), _ptr(self.vert_ptr),
                     _ptr(self.vert_col), _ptr(self.block_mask), self.block_size, _ptr(self.stripe_ptr),
                     _ptr(self.stripe_col), self.stripe_rows)


class SparseIndex:
    """Canonical sparse index (sa_index in include/sa.h) in device memory."""

    KEYS = ("run_ptr", "run_lo", "run_hi", "seg_ptr", "seg_lo", "seg_hi", "bcol_ptr", "bcol_idx", "col_ptr",
            "col_idx", "pair_count", "dbits")

    def __init__(self, S, n_heads, row_block, device):
        self.S, self.n_heads, self.row_block = S, n_heads, row_block
        self.n_row_blocks = -(-S // row_block)
        n = n_heads * self.n_row_blocks
        self.run_ptr = torch.zeros(n_heads + 1, dtype=torch.int32, device=device)
        self.seg_ptr = torch.zeros(n + 1, dtype=torch.int64, device=device)
        self.bcol_ptr = torch.zeros(n + 1, dtype=torch.int64, device=device)
        self.col_ptr = torch.zeros(n + 1, dtype=torch.int64, device=device)
        self.pair_count = torch.zeros(n_heads, dtype=torch.int64, device=device)
        self.dbits = torch.zeros(n_heads * (-(-S // 32)), dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.run_lo = self.run_hi = self.seg_lo = self.seg_hi = self.bcol_idx = self.col_idx = None
        self.sizes = None

    def _alloc_payload(self, sizes: _Sizes, device):
        mk = lambda n: torch.zeros(max(1, int(n)), dtype=torch.int32, device=device)
        self.run_lo, self.run_hi = mk(sizes.n_runs), mk(sizes.n_runs)
        self.seg_lo, self.seg_hi = mk(sizes.n_segs), mk(sizes.n_segs)
        self.bcol_idx, self.col_idx = mk(sizes.n_bcols), mk(sizes.n_cols)
        self.sizes = dict(n_runs=sizes.n_runs, n_segs=sizes.n_segs, n_bcols=sizes.n_bcols, n_cols=sizes.n_cols)

    def c_struct(self) -> _Index:
        cap = _Sizes(*(self.sizes[k] if self.sizes else 0 for k in ("n_runs", "n_segs", "n_bcols", "n_cols")))
        return _Index(self.S, self.n_heads, self.row_block, self.n_row_blocks, _ptr(self.run_ptr),
                      _ptr(self.run_lo), _ptr(self.run_hi), _ptr(self.seg_ptr), _ptr(self.seg_lo),
                      _ptr(self.seg_hi), _ptr(self.bcol_ptr), _ptr(self.bcol_idx), _ptr(self.col_ptr),
                      _ptr(self.col_idx), _ptr(self.pair_count), _ptr(self.dbits), _ptr(self.status), cap)

    def to_numpy(self) -> dict:
        out = dict(S=self.S, n_heads=self.n_heads, row_block=self.row_block, n_row_blocks=self.n_row_blocks)
        for k in self.KEYS:
            t = getattr(self, k).cpu().numpy()
            size_key = {"run_lo": "n_runs", "run_hi": "n_runs", "seg_lo": "n_segs", "seg_hi": "n_segs",
                        "bcol_idx": "n_bcols", "col_idx": "n_cols"}.get(k)
            out[k] = t[:self.sizes[size_key]] if size_key else t
        out["dbits"] = out["dbits"].view(np.uint32)
        return out

    @property
    def total_pairs(self) -> int:
        return int(self.pair_count.sum().item())


def build_index(patterns: DevicePatterns, row_block: int, validate: bool = False, stream=None) -> SparseIndex:
    """sa_build_index: size query (synchronises the stream), allocation, then the fill."""
    dev = patterns.diag_ptr.device
    ix = SparseIndex(patterns.S, patterns.n_heads, row_block, dev)
    d = patterns.c_struct()
    c = ix.c_struct()
    sizes = _Sizes()
    flags = SA_BUILD_VALIDATE if validate else 0
    _check(_lib.sa_build_index(C.byref(d), C.byref(c), C.byref(sizes), flags, _stream(stream)), "sa_build_index")
    ix._alloc_payload(sizes, dev)
    refill_index(patterns, ix, stream)
    ix._patterns = patterns
    return ix


def refill_index(patterns: DevicePatterns, ix: SparseIndex, stream=None):
    """Re-run the whole build (count, scan, fill) into an existing index without synchronising."""
    d = patterns.c_struct()
    c = ix.c_struct()
    _check(_lib.sa_build_index(C.byref(d), C.byref(c), None, 0, _stream(stream)), "sa_build_index")


def sparse_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: SparseIndex,
                        softmax_scale: Optional[float] = None, return_lse: bool = False,
                        out: Optional[torch.Tensor] = None, stream=None):
    """sa_sparse_attn_prefill: q [B,Hq,S,d], k/v [B,Hkv,S,d] (bf16 or fp32, contiguous, on the GPU)."""
    if q.dtype == torch.bfloat16:
        dt = SA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = SA_DTYPE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q [B,Hq,S,d] and k, v [B,Hkv,S,d] expected")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, hq, S, d = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must match q")
    lse = torch.empty((B, hq, S), dtype=torch.float32, device=q.device) if return_lse else None
    c = index.c_struct()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.sa_sparse_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, hq,
                                       k.shape[1], S, d, dt, scale, C.byref(c), _stream(stream)),
           "sa_sparse_attn_prefill")
    return (o, lse) if return_lse else o


def sparse_attn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, index: SparseIndex,
                       softmax_scale: Optional[float] = None, return_lse: bool = False,
                       out: Optional[torch.Tensor] = None, stream=None):
    """sa_sparse_attn_decode: q [B,Hq,d] at positions pos (int32 [B], on the GPU) against the cache
    k/v [B,Hkv,S,d] (bf16 or fp32, contiguous)."""
    if q.dtype == torch.bfloat16:
        dt = SA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = SA_DTYPE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q [B,Hq,d] and k, v [B,Hkv,S,d] expected")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, hq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    if pos.dtype != torch.int32 or pos.shape != (B,) or pos.device != q.device:
        raise ValueError("pos must be an int32 [B] tensor on q's device")
    S = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must match q")
    lse = torch.empty((B, hq), dtype=torch.float32, device=q.device) if return_lse else None
    c = index.c_struct()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.sa_sparse_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), pos.data_ptr(), o.data_ptr(),
                                      _ptr(lse), B, hq, k.shape[1], S, d, dt, scale, C.byref(c), _stream(stream)),
           "sa_sparse_attn_decode")
    return (o, lse) if return_lse else o


def attention_maps(q: torch.Tensor, k: torch.Tensor, softmax_scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sa_attention_maps: batch-averaged causal attention maps [Hq, L, L] (float32) of q [B,Hq,L,d] against
    k [B,Hkv,L,d] (bf16 or fp32, contiguous, on the GPU); the input of pattern_capture."""
    if q.dtype == torch.bfloat16:
        dt = SA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = SA_DTYPE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    if k.dtype != q.dtype:
        raise TypeError("q and k must share one dtype")
    if q.dim() != 4 or k.dim() != 4 or not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("contiguous q [B,Hq,L,d] and k [B,Hkv,L,d] expected")
    B, hq, L, d = q.shape
    if k.shape[0] != B or k.shape[2] != L or k.shape[3] != d:
        raise ValueError("k shape does not match q")
    maps = torch.empty((hq, L, L), dtype=torch.float32, device=q.device) if out is None else out
    if maps.shape != (hq, L, L) or maps.dtype != torch.float32 or not maps.is_contiguous():
        raise ValueError("out must be a contiguous float32 [Hq, L, L] tensor")
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.sa_attention_maps(q.data_ptr(), k.data_ptr(), B, hq, k.shape[1], L, d, dt, scale, maps.data_ptr(),
                                  _stream(stream)), "sa_attention_maps")
    return maps


def pattern_capture(maps: torch.Tensor, lam: float = 0.5, eps: float = 1e-8, tau: float = 0.3, mu: float = 0.8,
                    norm_scope: int = 0, return_hits: bool = True, return_mask: bool = False, out: Optional[dict] = None,
                    stream=None) -> dict:
    """sa_pattern_capture on float32 maps [n, L, L] in device memory.  `out`: a dict returned by an earlier
    call with the same shapes and flags, whose tensors are written again instead of new ones."""
    if maps.dtype != torch.float32 or maps.dim() != 3 or maps.shape[1] != maps.shape[2] or not maps.is_contiguous():
        raise ValueError("maps must be a contiguous float32 [n, L, L] tensor")
    n, L, _ = maps.shape
    dev = maps.device
    if out is not None:
        kd, kv, hd, hv, tm = (out.get(x) for x in ("keep_diag", "keep_vert", "diag_hits", "vert_hits", "true_mask"))
        want = [(kd, (n, L), torch.uint8), (kv, (n, L), torch.uint8)]
        want += [(hd, (n, L), torch.int32), (hv, (n, L), torch.int32)] if return_hits else []
        want += [(tm, (n, L, L), torch.uint8)] if return_mask else []
        for t, shape, dt in want:
            if t is None or tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device != dev:
                raise ValueError("out does not match the maps and the requested outputs")
        if not return_hits:
            hd = hv = None
        if not return_mask:
            tm = None
    else:
        kd = torch.empty((n, L), dtype=torch.uint8, device=dev)
        kv = torch.empty((n, L), dtype=torch.uint8, device=dev)
        hd = torch.empty((n, L), dtype=torch.int32, device=dev) if return_hits else None
        hv = torch.empty((n, L), dtype=torch.int32, device=dev) if return_hits else None
        tm = torch.empty((n, L, L), dtype=torch.uint8, device=dev) if return_mask else None
    _check(_lib.sa_pattern_capture(maps.data_ptr(), n, L, lam, eps, tau, mu, norm_scope, kd.data_ptr(),
                                   kv.data_ptr(), _ptr(hd), _ptr(hv), _ptr(tm), _stream(stream)),
           "sa_pattern_capture")
    return dict(keep_diag=kd, keep_vert=kv, diag_hits=hd, vert_hits=hv, true_mask=tm)


def pattern_coverage(maps: torch.Tensor, keep_diag: torch.Tensor, keep_vert: torch.Tensor, stream=None):
    """sa_pattern_coverage: per map, (attention-mass share float64 [n], cell count int64 [n]) of the kept
    diagonals and verticals inside the L x L causal window."""
    if maps.dtype != torch.float32 or maps.dim() != 3 or maps.shape[1] != maps.shape[2] or not maps.is_contiguous():
        raise ValueError("maps must be a contiguous float32 [n, L, L] tensor")
    n, L, _ = maps.shape
    for f in (keep_diag, keep_vert):
        if f.dtype != torch.uint8 or tuple(f.shape) != (n, L) or not f.is_contiguous():
            raise ValueError("keep flags must be contiguous uint8 [n, L] tensors")
    mass = torch.empty(n, dtype=torch.float64, device=maps.device)
    cells = torch.empty(n, dtype=torch.int64, device=maps.device)
    _check(_lib.sa_pattern_coverage(maps.data_ptr(), n, L, keep_diag.data_ptr(), keep_vert.data_ptr(),
                                    mass.data_ptr(), cells.data_ptr(), _stream(stream)), "sa_pattern_coverage")
    return mass, cells


def sample_scores(q: torch.Tensor, k: torch.Tensor, row0: int, n_rows: int, band: int = 0,
                  skip_cols: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None, scores=None,
                  row_lse: Optional[torch.Tensor] = None, lse_given: bool = False, families=(True, True),
                  no_alloc: bool = False, stream=None):
    """sa_sample_scores: adds the attention mass of query rows row0 .. row0+n_rows-1 on the pairs outside
    the window (i - j >= band) and off `skip_cols` onto per-head diagonal and vertical scores (int64
    [Hq, S] each, fixed point 2^-32).  `scores` = (diag, vert) to accumulate into, new zeroed arrays
    otherwise (only the families flagged in `families` = (diagonals, verticals); None for the other);
    `row_lse` [B, Hq, n_rows] is written, or read when lse_given.  no_alloc: the library's
    allocation-free entry point (its scratch is a static 16 MiB device array; the outputs are still
    made here unless passed in).  Returns (diag, vert, row_lse)."""
    if q.dtype == torch.bfloat16:
        dt = SA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = SA_DTYPE_F32
    else:
        raise TypeError("q must be bfloat16 or float32")
    if k.dtype != q.dtype or q.dim() != 4 or k.dim() != 4 or not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("contiguous q [B,Hq,S,d] and k [B,Hkv,S,d] of one dtype expected")
    B, hq, S, d = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != d:
        raise ValueError("k shape does not match q")
    ts = _torch_stream(stream)
    cur = torch.cuda.current_stream(q.device)
    if scores is None:
        # zeroed on the current stream; the launch stream waits for it below
        scores = tuple(torch.zeros((hq, S), dtype=torch.int64, device=q.device) if want else None
                       for want in families)
    diag, vert = scores
    if diag is None and vert is None:
        raise ValueError("at least one family of scores is needed")
    for t in (diag, vert):
        if t is not None and (t.dtype != torch.int64 or tuple(t.shape) != (hq, S) or not t.is_contiguous()):
            raise ValueError("scores must be contiguous int64 [Hq, S] tensors")
    if skip_cols is not None and (skip_cols.dtype != torch.uint8 or tuple(skip_cols.shape) != (hq, S)
                                  or not skip_cols.is_contiguous()):
        raise ValueError("skip_cols must be a contiguous uint8 [Hq, S] tensor")
    if row_lse is None:
        if lse_given:
            raise ValueError("lse_given needs row_lse")
        row_lse = torch.empty((B, hq, max(n_rows, 1)), dtype=torch.float32, device=q.device)
    elif (row_lse.dtype != torch.float32 or tuple(row_lse.shape) != (B, hq, n_rows)
          or not row_lse.is_contiguous() or row_lse.device != q.device):
        raise ValueError("row_lse must be a contiguous float32 [B, Hq, n_rows] tensor on q's device")
    for t in (diag, vert, skip_cols):
        if t is not None and t.device != q.device:
            raise ValueError("scores and skip_cols must be on q's device")
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    ws_bytes = 0 if (lse_given or no_alloc) else int(_lib.sa_sample_scores_workspace(B, hq, row0, n_rows))
    ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=q.device) if ws_bytes else None
    if ts != cur:
        # the zeroed scores and the fresh buffers were made on the current stream: order the launch after them,
        # and keep them from being reused before the launch stream is done with them
        ts.wait_stream(cur)
    if no_alloc:
        _check(_lib.sa_sample_scores_noalloc(q.data_ptr(), k.data_ptr(), B, hq, k.shape[1], S, d, dt, scale, row0,
                                             n_rows, band, _ptr(skip_cols), int(bool(lse_given)), row_lse.data_ptr(),
                                             _ptr(diag), _ptr(vert), ts.cuda_stream), "sa_sample_scores_noalloc")
    else:
        _check(_lib.sa_sample_scores(q.data_ptr(), k.data_ptr(), B, hq, k.shape[1], S, d, dt, scale, row0, n_rows,
                                     band, _ptr(skip_cols), int(bool(lse_given)), row_lse.data_ptr(), _ptr(ws),
                                     ws_bytes, _ptr(diag), _ptr(vert), ts.cuda_stream), "sa_sample_scores")
    if ts != cur:
        for t in (ws, diag, vert, row_lse):
            if t is not None:
                t.record_stream(ts)
    return diag, vert, row_lse


def select_patterns(scores: torch.Tensor, alpha: float, rows: int, band: int = 0, stream=None) -> torch.Tensor:
    """sa_select_patterns for one family: keep flags (uint8 [Hq, S]) of the fewest top patterns that bring
    the covered mass of `rows` sampled rows to `alpha`; patterns x < band always kept."""
    if scores.dtype != torch.int64 or scores.dim() != 2 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous int64 [Hq, S] tensor")
    n, S = scores.shape
    keep = torch.empty((n, S), dtype=torch.uint8, device=scores.device)
    _check(_lib.sa_select_patterns(scores.data_ptr(), n, S, float(alpha), int(rows), int(band), keep.data_ptr(),
                                   _stream(stream)), "sa_select_patterns")
    return keep


def patterns_to_desc(keep_diag: torch.Tensor, keep_vert: torch.Tensor, S: int, stream=None) -> DevicePatterns:
    """sa_patterns_to_desc: kept patterns of each map (one map per query head) -> descriptor at length S."""
    n, L = keep_diag.shape
    dev = keep_diag.device
    cap = max(1, n * min(L, S))
    dp = torch.empty(n + 1, dtype=torch.int32, device=dev)
    vp = torch.empty(n + 1, dtype=torch.int32, device=dev)
    do = torch.empty(cap, dtype=torch.int32, device=dev)
    vc = torch.empty(cap, dtype=torch.int32, device=dev)
    kd, kv = keep_diag.contiguous(), keep_vert.contiguous()
    _check(_lib.sa_patterns_to_desc(kd.data_ptr(), kv.data_ptr(), n, L, S, dp.data_ptr(), do.data_ptr(), vp.data_ptr(),
                                    vc.data_ptr(), _stream(stream)), "sa_patterns_to_desc")
    _hold(kd, stream)
    _hold(kv, stream)
    return DevicePatterns(S, n, dp, do, vp, vc, device=dev)
