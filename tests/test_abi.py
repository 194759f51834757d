"""CPU tests of the C ABI: the library loads, exports every declared entry point, and
its host-side validation rejects bad arguments before anything touches a GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


@pytest.fixture(scope="module")
def m():
    import structured_sparse_attention_amd as pkg   # raises if libsa.so is not built
    return pkg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("sa_build_index", "sa_build_index_workspace_bytes", "sa_sparse_attn_prefill", "sa_sparse_attn_decode", "sa_attention_maps",
              "sa_pattern_capture", "sa_pattern_coverage", "sa_patterns_to_desc", "sa_sample_scores",
              "sa_sample_scores_workspace", "sa_select_patterns", "sa_calib_mfma_bf16", "sa_calib_gather", "sa_status_string", "sa_version"):
        assert f in names


def test_library_exports_every_declared_symbol(m):
    lib = C.CDLL(m.library_path())
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_build_index_needs_no_workspace(m):
    f = m.lib.sa_build_index_workspace_bytes
    f.restype = C.c_size_t
    f.argtypes = [C.c_void_p, C.c_int32]
    assert f(None, 64) == 0 and f(None, 128) == 0


def test_status_strings_and_version(m):
    for code in (0, -1, -2, -3, -4, -5):
        assert m.lib.sa_status_string(code)
    assert b"gfx950" in m.lib.sa_version()


FAKE = C.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _desc(m, S=512, H=1, **kw):
    d = m._Desc(S, H, FAKE.value, FAKE.value, FAKE.value, FAKE.value, None, 64, None, None, 128)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _index(m, S=512, H=1, BM=64, **kw):
    ix = m._Index(S, H, BM, -(-S // BM), *([FAKE.value] * 13), m._Sizes(10, 10, 10, 10))
    for k, v in kw.items():
        setattr(ix, k, v)
    return ix


def test_build_index_validation(m):
    f = m.lib.sa_build_index
    sz = m._Sizes()
    assert f(None, C.byref(_index(m)), C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m)), None, C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m, S=0)), C.byref(_index(m, S=0)), C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m)), C.byref(_index(m, BM=32)), C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m)), C.byref(_index(m, n_row_blocks=3)), C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m, H=2)), C.byref(_index(m)), C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m, diag_off=None)), C.byref(_index(m)), C.byref(sz), 0, None) == -1
    # block size must be a multiple of the row block
    assert f(C.byref(_desc(m, block_mask=FAKE.value, block_size=64)), C.byref(_index(m, BM=128)),
             C.byref(sz), 0, None) == -1
    assert f(C.byref(_desc(m, stripe_ptr=FAKE.value, stripe_col=FAKE.value, stripe_rows=96)),
             C.byref(_index(m, BM=64)), C.byref(sz), 0, None) == -1
    # size query needs `sizes` when the payload arrays are missing
    assert f(C.byref(_desc(m)), C.byref(_index(m, col_idx=None)), None, 0, None) == -1
    # too long for the LDS bitmaps
    S = 300000
    assert f(C.byref(_desc(m, S=S)), C.byref(_index(m, S=S)), C.byref(sz), 0, None) == -2


def test_attention_validation(m):
    f = m.lib.sa_sparse_attn_prefill
    ix = _index(m)
    p = FAKE.value
    assert f(None, p, p, p, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1
    assert f(p, p, p, p, None, 1, 3, 2, 512, 64, 1, 0.0, C.byref(ix), None) == -1   # hq % hkv
    assert f(p, p, p, p, None, 1, 1, 1, 512, 64, 7, 0.0, C.byref(ix), None) == -1   # dtype
    assert f(p, p, p, p, None, 1, 1, 1, 512, 96, 1, 0.0, C.byref(ix), None) == -2   # head_dim
    assert f(p, p, p, p, None, 1, 1, 1, 256, 64, 1, 0.0, C.byref(ix), None) == -1   # S != index S
    assert f(p, p, p, p, None, 1, 2, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1   # heads != index heads
    assert f(p, p, p, p, None, 0, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1   # batch
    assert f(p, p, p, p, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(_index(m, col_idx=None)), None) == -1
    assert f(p, p, p, p + 8, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1  # o not 16-byte aligned


def test_decode_validation(m):
    f = m.lib.sa_sparse_attn_decode
    ix = _index(m)
    p = FAKE.value
    assert f(p, p, p, None, p, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1   # pos
    assert f(None, p, p, p, p, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1  # q
    assert f(p, p, p, p, p, None, 1, 3, 2, 512, 64, 1, 0.0, C.byref(ix), None) == -1     # hq % hkv
    assert f(p, p, p, p, p, None, 1, 1, 1, 512, 64, 7, 0.0, C.byref(ix), None) == -1     # dtype
    assert f(p, p, p, p, p, None, 1, 1, 1, 512, 96, 1, 0.0, C.byref(ix), None) == -2     # head_dim
    assert f(p, p, p, p, p, None, 1, 1, 1, 256, 64, 1, 0.0, C.byref(ix), None) == -1     # S != index S
    assert f(p, p, p, p, p, None, 0, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1     # batch
    assert f(p, p, p, p, p, None, 1, 1, 1, 512, 64, 1, float("inf"), C.byref(ix), None) == -1
    assert f(p, p, p + 2, p, p, None, 1, 1, 1, 512, 64, 1, 0.0, C.byref(ix), None) == -1  # v not 16-byte aligned


def test_attention_maps_validation(m):
    f = m.lib.sa_attention_maps
    p = FAKE.value
    assert f(None, p, 1, 1, 1, 64, 64, 1, 0.0, p, None) == -1
    assert f(p, p, 1, 1, 1, 64, 64, 1, 0.0, None, None) == -1
    assert f(p, p, 1, 3, 2, 64, 64, 1, 0.0, p, None) == -1      # hq % hkv
    assert f(p, p, 0, 1, 1, 64, 64, 1, 0.0, p, None) == -1      # batch
    assert f(p, p, 1, 1, 1, 64, 64, 9, 0.0, p, None) == -1      # dtype
    assert f(p, p, 1, 1, 1, 64, 80, 1, 0.0, p, None) == -2      # head_dim
    assert f(p, p, 1, 1, 1, 5000, 64, 1, 0.0, p, None) == -2    # L above the capture window
    assert f(p + 4, p, 1, 1, 1, 64, 64, 1, 0.0, p, None) == -1  # q not 16-byte aligned
    assert f(p, p, 1, 1, 1, 64, 64, 1, 0.0, p + 8, None) == -1  # maps not 16-byte aligned


def test_sample_and_select_validation(m):
    f = m.lib.sa_sample_scores
    p = FAKE.value
    # q, k, batch, hq, hkv, S, d, dtype, scale, row0, n_rows, band, skip, lse_given, lse, ws, ws_bytes, diag, vert,
    # stream; valid but for the field changed
    ws = m.lib.sa_sample_scores_workspace(1, 4, 448, 64)
    assert ws == 4 * 64 * 2 * 8                                   # 512 keys: two 256-key splits
    args = [p, p, 1, 4, 2, 512, 64, 1, 0.0, 448, 64, 16, None, 0, p, p, ws, p, p, None]

    def bad(changes, code):
        a = list(args)
        for i, val in changes:
            a[i] = val
        assert f(*a) == code, changes
    bad([(0, None)], -1)            # q
    bad([(17, None), (18, None)], -1)   # neither family
    bad([(18, p + 4)], -1)          # vert not 8-byte aligned
    bad([(17, p + 4)], -1)          # diag not 8-byte aligned
    bad([(15, None)], -1)           # workspace needed to compute the LSE
    bad([(16, ws - 8)], -4)         # workspace too small
    bad([(3, 3)], -1)               # hq % hkv
    bad([(7, 5)], -1)               # dtype
    bad([(6, 96)], -2)              # head_dim
    bad([(9, -1)], -1)              # row0
    bad([(10, 0)], -1)              # n_rows
    bad([(10, 65)], -1)             # row0 + n_rows > S
    bad([(11, -1)], -1)             # band
    bad([(5, 8192), (9, 0), (10, 4096)], -2)              # more rows than one call takes
    bad([(2, 1024), (5, 8192), (9, 0), (10, 2048)], -2)   # batch * rows above 2^20
    g = m.lib.sa_select_patterns
    assert g(None, 1, 8, 0.9, 4, 0, p, None) == -1
    assert g(p, 1, 8, 0.0, 4, 0, p, None) == -1       # alpha
    assert g(p, 1, 8, 1.5, 4, 0, p, None) == -1
    assert g(p, 1, 8, float("nan"), 4, 0, p, None) == -1
    assert g(p, 1, 8, 0.9, 0, 0, p, None) == -1       # rows
    assert g(p, 1, 8, 0.9, 1 << 31, 0, p, None) == -1
    assert g(p, 1, 8, 0.9, 4, -1, p, None) == -1      # band
    assert g(p, 0, 8, 0.9, 4, 0, p, None) == -1
    assert g(p + 4, 1, 8, 0.9, 4, 0, p, None) == -1   # scores not 8-byte aligned


def test_calibration_validation(m):
    p = FAKE.value
    assert m.lib.sa_calib_mfma_bf16(0, 10, p, None) == -1
    assert m.lib.sa_calib_mfma_bf16(4, 10, None, None) == -1
    g = m.lib.sa_calib_gather
    assert g(p, 1 << 20, 16384, 8, 4, 1, None, None) == -1          # sink
    assert g(p, 1 << 20, 100, 8, 4, 1, p, None) == -1               # chunk not a multiple of 16
    assert g(p, 4096, 16384, 8, 4, 1, p, None) == -1                # chunk larger than the region
    assert g(p + 8, 1 << 20, 16384, 8, 4, 1, p, None) == -1         # buffer not 16-byte aligned


def test_capture_validation(m):
    f = m.lib.sa_pattern_capture
    p = FAKE.value
    assert f(None, 1, 8, 0.5, 1e-8, 0.3, 0.8, 0, p, p, None, None, None, None) == -1
    assert f(p, 0, 8, 0.5, 1e-8, 0.3, 0.8, 0, p, p, None, None, None, None) == -1
    assert f(p, 1, 8, 0.5, 1e-8, 0.3, 0.8, 2, p, p, None, None, None, None) == -1
    assert f(p, 1, 8, float("inf"), 1e-8, 0.3, 0.8, 0, p, p, None, None, None, None) == -1   # lambda
    assert f(p, 1, 8, 0.0, 0.0, 0.3, 0.8, 0, p, p, None, None, None, None) == -1   # log 0 possible
    assert f(p, 1, 8, -0.5, 0.0, 0.3, 0.8, 0, p, p, None, None, None, None) == -1  # 0^-0.5 possible
    assert f(p, 1, 5000, 0.5, 1e-8, 0.3, 0.8, 0, p, p, None, None, None, None) == -2
    assert f(p, 1, 8, 0.5, float("nan"), 0.3, 0.8, 0, p, p, None, None, None, None) == -1
    c = m.lib.sa_pattern_coverage
    assert c(None, 1, 8, p, p, p, None, None) == -1
    assert c(p, 1, 8, p, p, None, None, None) == -1     # mass is required
    assert c(p, 0, 8, p, p, p, None, None) == -1
    assert c(p, 1, 5000, p, p, p, None, None) == -2
    g = m.lib.sa_patterns_to_desc
    assert g(None, p, 1, 8, 8, p, p, p, p, None) == -1
    assert g(p, p, 1, 8, 0, p, p, p, p, None) == -1


def test_product_package_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "structured_sparse_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"\boracle\b|sa_oracle|liboracle|workloads", text), fn
