"""Host-side checks of the C-ABI (no GPU needed: every rejected call returns
before any HIP call, and the size queries are pure host code)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_row_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sparse_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exported_set():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert B.sparse_attn_version() == 10000
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert B.status_string(st) and B.status_string(st) != "unknown status"
    assert B.status_string(-99) == "unknown status"


def _shape(**kw):
    base = dict(batch=1, heads=12, head_dim=128, grid=(20, 32, 48), dtype="bf16")
    base.update(kw)
    return B.make_shape(base["batch"], base["heads"], base["head_dim"], base["grid"], base["dtype"],
                        base.get("scale", 0.0), base.get("tile", (1, 8, 8)))


def test_capacity_and_workspace_formulas():
    s = _shape()
    nB = 20 * 4 * 6
    assert nB == 480
    rows = 12 * nB
    assert B.sparse_attn_csr_capacity(s) == rows * nB
    nbp = 512
    expect = 0
    al = lambda x: (x + 255) // 256 * 256
    expect = al(expect + 4 * 12)
    expect = al(expect + 4 * 12 * ((nB + 15) // 16) * 16 * 128)   # key block means (bf16 hi | lo), 16-key groups
    expect = al(expect + 4 * rows * 128)                  # query block means (raster selection)
    expect = al(expect + 8 * 12 * ((nB + 15) // 16))      # selection look-back words per 16-row group
    expect = al(expect + 16)                              # selection ticket counter
    expect = al(expect + 8 * rows * 128)                  # exact key means (fp64)
    expect = al(expect + 4 * rows)                        # their norms
    expect = al(expect + 8 * rows * 128)                  # exact query means (raster selection)
    expect = al(expect + 8 * rows * (nbp // 64))
    expect = al(expect + 4 * rows)
    expect = al(expect + 4 * 12 * ((nB + 15) // 16))     # kept-block totals per 16-row group
    pairs = 12 * ((nB + 1) // 2)
    slots = min(512, 4 * pairs) + (384 * 4 if pairs >= 2 * 512 else 0)   # long-row and last-round pieces
    expect = al(expect + 32 * slots)                      # pieces
    expect = al(expect + 16)                              # plan counts
    expect = al(expect + 4 * pairs)                       # per-pair split flags
    expect = al(expect + 12 * slots)                      # merge list
    expect = al(expect + 4 * slots * 2 * 64 * 128)        # partial outputs (fp32)
    expect = al(expect + 4 * slots * 2 * 64)              # partial log-sum-exp
    expect = al(expect + 4 * slots * 2 * 64 * 128)        # backward: second partial rows (dK)
    expect = al(expect + 4 * (rows + 1))                  # backward: transposed row pointers
    expect = al(expect + 4 * rows * 64)                   # backward: lse in log2 units
    expect = al(expect + 4 * rows * 64)                   # backward: dO . O
    per_head = 4 * ((nB + 1) // 2) * nbp                  # clustering selector: a row per query-block pair
    expect = al(expect + min(12, max(1, (64 << 20) // per_head)) * per_head)
    expect = al(expect + 8 * nB)                          # partial tiles: token slots per block
    assert B.sparse_attn_workspace_size(s) == expect


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), B.SPARSE_ATTN_UNSUPPORTED),
    (dict(dtype=7), B.SPARSE_ATTN_UNSUPPORTED),
    (dict(tile=(1, 4, 8)), B.SPARSE_ATTN_UNSUPPORTED),             # 32-token tile
    (dict(batch=0), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(heads=-1), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(scale=float("nan")), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(scale=float("inf")), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(scale=-0.1), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(heads=4000, grid=(64, 48, 80)), B.SPARSE_ATTN_UNSUPPORTED),  # worst-case nnz overflows int32
])
def test_bad_shapes_rejected(kw, status):
    s = _shape(**kw)
    assert B.sparse_attn_csr_capacity(s) == status
    assert B.sparse_attn_workspace_size(s) == status


def test_other_64_token_tiles_accepted():
    s = _shape(tile=(4, 4, 4), grid=(20, 32, 48))
    assert B.sparse_attn_csr_capacity(s) == (12 * 5 * 8 * 12) * (5 * 8 * 12)


# Fake but well-aligned device addresses: every call below must fail its
# host-side checks before it could dereference or launch anything.
A = 1 << 20


def _select(shape, thr=0.9, head_thr=None, q=A, k=A, rp=A, ci=A, cap=None, ws=A, wsb=None):
    params = B.SelectParams(thr, head_thr, -1, -1, -1)
    cap = B.sparse_attn_csr_capacity(shape) if cap is None else cap
    wsb = B.sparse_attn_workspace_size(shape) if wsb is None else wsb
    return B.lib().sparse_attn_select(ctypes.byref(shape), ctypes.byref(params), q, k, rp, ci, cap, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(thr=0.0), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(thr=-0.5), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(thr=float("nan")), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(q=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(k=A + 8), B.SPARSE_ATTN_INVALID_ARGUMENT),              # misaligned
    (dict(rp=A + 2), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(ci=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(ws=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cap=10), B.SPARSE_ATTN_CAPACITY),
    (dict(wsb=1024), B.SPARSE_ATTN_WORKSPACE),
])
def test_select_rejects_before_launch(kw, status):
    assert _select(_shape(), **kw) == status


def _select_raster(shape, qt=2 * A, kt=3 * A, cap=None, wsb=None):
    params = B.SelectParams(0.9, None, -1, -1, -1)
    cap = B.sparse_attn_csr_capacity(shape) if cap is None else cap
    wsb = B.sparse_attn_workspace_size(shape) if wsb is None else wsb
    return B.lib().sparse_attn_select_raster(ctypes.byref(shape), ctypes.byref(params), A, A, qt, kt, A, A, cap, A,
                                             wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qt=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(kt=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(qt=2 * A, kt=2 * A), B.SPARSE_ATTN_INVALID_ARGUMENT),    # one buffer for both copies
    (dict(qt=A), B.SPARSE_ATTN_INVALID_ARGUMENT),                  # copy over its own input
    (dict(kt=3 * A + 8), B.SPARSE_ATTN_INVALID_ARGUMENT),          # misaligned
    (dict(cap=10), B.SPARSE_ATTN_CAPACITY),
    (dict(wsb=1024), B.SPARSE_ATTN_WORKSPACE),
])
def test_raster_select_rejects_before_launch(kw, status):
    assert _select_raster(_shape(), **kw) == status


def test_select_rejects_bad_head_threshold():
    arr = (ctypes.c_float * 12)(*([0.9] * 11 + [float("nan")]))
    assert _select(_shape(), head_thr=ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))) == \
        B.SPARSE_ATTN_INVALID_ARGUMENT


def test_select_rejects_too_many_blocks():
    s = _shape(heads=1, grid=(65, 64, 64))      # 4,160 blocks: a row no longer fits the selection's registers
    assert _select(s) == B.SPARSE_ATTN_UNSUPPORTED
    s = _shape(heads=1, grid=(64, 64, 64))      # 4,096 blocks: accepted, fails later on the fake workspace size
    assert _select(s, wsb=1024) == B.SPARSE_ATTN_WORKSPACE


def _forward(shape, q=A, k=A, v=A, rp=A, ci=A, cc=100, out=A, lse=None, ws=A, wsb=None):
    wsb = B.sparse_attn_workspace_size(shape) if wsb is None else wsb
    return B.lib().sparse_attn_forward(ctypes.byref(shape), q, k, v, rp, ci, cc, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(v=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(out=A + 4), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(lse=A + 2), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cc=-1), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(ci=None, cc=5), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(rp=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(wsb=0), B.SPARSE_ATTN_WORKSPACE),
])
def test_forward_rejects_before_launch(kw, status):
    assert _forward(_shape(), **kw) == status


def test_forward_rejects_bad_shape():
    assert _forward(_shape(head_dim=32)) == B.SPARSE_ATTN_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(mask=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cap=0), B.SPARSE_ATTN_CAPACITY),
    (dict(wsb=16), B.SPARSE_ATTN_WORKSPACE),
    (dict(rp=A + 1), B.SPARSE_ATTN_INVALID_ARGUMENT),
])
def test_mask_to_csr_rejects_before_launch(kw, status):
    s = _shape()
    cap = kw.get("cap", B.sparse_attn_csr_capacity(s))
    wsb = kw.get("wsb", B.sparse_attn_workspace_size(s))
    mask = kw.get("mask", A)
    rp = kw.get("rp", A)
    assert B.lib().sparse_attn_mask_to_csr(ctypes.byref(s), mask, rp, A, cap, A, wsb, None) == status


@pytest.mark.parametrize("fn", ["sparse_attn_to_tiles", "sparse_attn_from_tiles"])
def test_reorder_rejects_before_launch(fn):
    f = getattr(B.lib(), fn)
    s = _shape()
    assert f(ctypes.byref(s), A, A, None) == B.SPARSE_ATTN_INVALID_ARGUMENT          # same buffer
    assert f(ctypes.byref(s), A, A + 8, None) == B.SPARSE_ATTN_INVALID_ARGUMENT      # misaligned
    assert f(ctypes.byref(s), None, A, None) == B.SPARSE_ATTN_INVALID_ARGUMENT


def test_full_csr_rejects_before_launch():
    f = B.lib().sparse_attn_full_csr
    s = _shape()
    cap = B.sparse_attn_csr_capacity(s)
    assert f(ctypes.byref(s), A, A, cap - 1, None) == B.SPARSE_ATTN_CAPACITY
    assert f(ctypes.byref(s), None, A, cap, None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert f(ctypes.byref(s), A, A + 2, cap, None) == B.SPARSE_ATTN_INVALID_ARGUMENT


def test_backward_rejects_before_launch():
    f = B.lib().sparse_attn_backward
    s = _shape()
    wsb = B.sparse_attn_workspace_size(s)
    ok = dict(q=A, k=A, v=A, o=A, lse=A, g=A, rp=A, ci=A, cc=10, dq=A, dk=A, dv=A, ti=A, ws=A, wsb=wsb)

    def call(**kw):
        x = dict(ok, **kw)
        return f(ctypes.byref(x.pop("shape", s)), x["q"], x["k"], x["v"], x["o"], x["lse"], x["g"], x["rp"], x["ci"],
                 x["cc"], x["dq"], x["dk"], x["dv"], x["ti"], x["ws"], x["wsb"], None)
    # fp32 passes the dtype check and stops at the missing lse, like bf16
    assert call(shape=_shape(dtype="f32"), lse=None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(lse=None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(ti=None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(dk=A + 4) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(cc=-1) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(wsb=wsb - 1) == B.SPARSE_ATTN_WORKSPACE


def test_forward_biased_rejects_before_launch():
    f = B.lib().sparse_attn_forward_biased
    s = _shape()
    wsb = B.sparse_attn_workspace_size(s)

    def call(shape=None, cb=A, cc=100, ws=A, w=None):
        return f(ctypes.byref(shape or s), A, A, A, A, A, cb, cc, A, None, ws, wsb if w is None else w, None)
    # fp32 passes the dtype check and stops at the missing offsets, like bf16
    assert call(shape=_shape(dtype="f32"), cb=None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(cb=None) == B.SPARSE_ATTN_INVALID_ARGUMENT            # offsets needed for a non-empty list
    assert call(cb=A + 2) == B.SPARSE_ATTN_INVALID_ARGUMENT           # misaligned
    assert call(cc=-1) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert call(w=16) == B.SPARSE_ATTN_WORKSPACE


def _sip(shape, budget=48.0, q=A, k=A, rp=A, ci=A, cb=A, cap=None, wsb=None):
    params = B.SipParams(budget, 7)
    cap = B.sparse_attn_csr_capacity(shape) if cap is None else cap
    wsb = B.sparse_attn_workspace_size(shape) if wsb is None else wsb
    return B.lib().sparse_attn_select_sip(ctypes.byref(shape), ctypes.byref(params), q, k, rp, ci, cb, cap, A, wsb,
                                          None)


@pytest.mark.parametrize("kw,status", [
    (dict(budget=0.0), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(budget=-3.0), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(budget=float("nan")), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(budget=float("inf")), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cb=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cb=A + 2), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(q=None), B.SPARSE_ATTN_INVALID_ARGUMENT),
    (dict(cap=10), B.SPARSE_ATTN_CAPACITY),
    (dict(wsb=1024), B.SPARSE_ATTN_WORKSPACE),
])
def test_select_sip_rejects_before_launch(kw, status):
    assert _sip(_shape(), **kw) == status


def test_select_sip_takes_fp32_and_rejects_too_many_blocks():
    # fp32 passes the dtype check and stops at the bad budget, like bf16
    assert _sip(_shape(dtype="f32"), budget=0.0) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert _sip(_shape(heads=1, grid=(65, 64, 64))) == B.SPARSE_ATTN_UNSUPPORTED


@pytest.mark.parametrize("r0,gamma,lam,status", [
    (-1.0, 0.5, 0, B.SPARSE_ATTN_INVALID_ARGUMENT),
    (float("inf"), 0.5, 0, B.SPARSE_ATTN_INVALID_ARGUMENT),
    (float("nan"), 0.5, 0, B.SPARSE_ATTN_INVALID_ARGUMENT),
    (2.0, 0.0, 0, B.SPARSE_ATTN_INVALID_ARGUMENT),
    (2.0, 1.5, 0, B.SPARSE_ATTN_INVALID_ARGUMENT),
    (2.0, 0.5, -1, B.SPARSE_ATTN_INVALID_ARGUMENT),
])
def test_radial_csr_rejects_before_launch(r0, gamma, lam, status):
    s = _shape()
    p = B.RadialParams(r0, gamma, lam)
    cap = B.sparse_attn_csr_capacity(s)
    assert B.lib().sparse_attn_radial_csr(ctypes.byref(s), ctypes.byref(p), A, A, cap, A,
                                          B.sparse_attn_workspace_size(s), None) == status
    ok = B.RadialParams(2.0, 0.5, 0)
    assert B.lib().sparse_attn_radial_csr(ctypes.byref(s), ctypes.byref(ok), A, A, cap - 1, A,
                                          B.sparse_attn_workspace_size(s), None) == B.SPARSE_ATTN_CAPACITY


def test_select_ibcs_rejects_before_launch():
    f = B.lib().sparse_attn_select_ibcs
    s = _shape()
    cap = B.sparse_attn_csr_capacity(s)
    wsb = B.sparse_attn_workspace_size(s)
    ok = B.SelectParams(0.9, None, -1, -1, -1)
    bad = B.SelectParams(0.0, None, -1, -1, -1)
    # fp32 passes the dtype check and stops at the bad threshold, like bf16
    assert f(ctypes.byref(_shape(dtype="f32")), ctypes.byref(bad), A, A, A, A, cap, A, wsb, None) == \
        B.SPARSE_ATTN_INVALID_ARGUMENT
    assert f(ctypes.byref(s), ctypes.byref(bad), A, A, A, A, cap, A, wsb, None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert f(ctypes.byref(s), ctypes.byref(ok), A, A, A, A, cap - 1, A, wsb, None) == B.SPARSE_ATTN_CAPACITY
    assert f(ctypes.byref(s), ctypes.byref(ok), A, A, A, A, cap, A, wsb - 1, None) == B.SPARSE_ATTN_WORKSPACE
    assert f(ctypes.byref(s), ctypes.byref(ok), None, A, A, A, cap, A, wsb, None) == B.SPARSE_ATTN_INVALID_ARGUMENT



# ---------------------------------------------------------------- binding checks
# Every call that takes tensors checks them against the shape first (dtype, size,
# contiguity, device) and raises ValueError without touching the GPU.

def _small():
    return B.make_shape(1, 2, 64, (2, 8, 16), "bf16")      # N = 256, nB = 4


def _tok(dtype=None, n=None):
    import torch
    return torch.zeros(n if n is not None else 2 * 256 * 64, dtype=dtype or torch.bfloat16)


def test_binding_rejects_wrong_dtype_before_any_call():
    import torch
    s = _small()
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        B.sparse_attn_select(s, _tok(torch.float32), _tok())
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        B.sparse_attn_forward(s, _tok(), _tok(torch.float16), _tok(), None, None)


def test_binding_rejects_wrong_size_and_layout():
    import torch
    s = _small()
    with pytest.raises(ValueError, match="must hold 32768 elements"):
        B.sparse_attn_select(s, _tok(n=100), _tok())
    nc = torch.zeros(2 * 64, 256, dtype=torch.bfloat16).t()        # right size, not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        B.sparse_attn_forward(s, nc, _tok(), _tok(), None, None)


def test_binding_rejects_host_tensors():
    s = _small()
    with pytest.raises(ValueError, match="GPU tensor"):
        B.sparse_attn_select(s, _tok(), _tok())
    with pytest.raises(ValueError, match="GPU tensor"):
        B.sparse_attn_to_tiles(s, _tok(), _tok())


def test_binding_rejects_bad_csr_and_lse():
    import torch
    s = _small()
    ok = dict(dtype=torch.int32)
    # the dtype checks come before the device check, so host tensors reach them
    with pytest.raises(ValueError, match="row_ptr must be torch.int32"):
        B._req_csr(s, torch.zeros(9, dtype=torch.int64), torch.zeros(4, **ok), None)
    with pytest.raises(ValueError, match="at least 9 elements"):
        B._req_csr(s, torch.zeros(8, **ok), torch.zeros(4, **ok), None)
    with pytest.raises(ValueError, match="at least 32 elements"):
        B._req(torch.zeros(31, **ok), "col_idx", torch.int32, min_numel=32)
    with pytest.raises(ValueError, match="lse must be torch.float32"):
        B._req_lse(s, torch.zeros(512, dtype=torch.float64), None)
    with pytest.raises(ValueError, match="lse must hold 512 elements"):
        B._req_lse(s, torch.zeros(511, dtype=torch.float32), None)


def test_select_check_rejects_bad_arguments_on_the_host():
    L = B.lib()
    s = _small()
    ws = B.sparse_attn_workspace_size(s)
    assert L.sparse_attn_select_check(ctypes.byref(s), None, ws, None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert L.sparse_attn_select_check(ctypes.byref(s), 16, ws - 1, None) == B.SPARSE_ATTN_WORKSPACE
    assert L.sparse_attn_select_check(ctypes.byref(s), 8, ws, None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    bad = B.make_shape(1, 2, 96, (2, 8, 16), "bf16")
    assert L.sparse_attn_select_check(ctypes.byref(bad), 16, ws, None) == B.SPARSE_ATTN_UNSUPPORTED
    assert "look-back" in B.status_string(B.SPARSE_ATTN_LOOKBACK_FAULT)


def test_noalloc_selection_rejects_what_its_scratch_cannot_hold():
    """The allocation-free selection checks the shape against its static scratch on the
    host: 64 heads of 3,840 blocks at d = 128 need ~380 MB of key means and are refused
    with SPARSE_ATTN_SCRATCH before any HIP call (the pointers are never touched)."""
    L = B.lib()
    params = B.SelectParams(0.9, None, -1, -1, -1)
    big = B.make_shape(1, 64, 128, (64, 48, 80), "bf16")
    assert B.sparse_attn_select_noalloc_bytes(big) > B.SPARSE_ATTN_SCRATCH_BYTES
    cap = B.sparse_attn_csr_capacity(big)
    assert L.sparse_attn_select_noalloc(ctypes.byref(big), ctypes.byref(params), 16, 16, 16, 16, cap,
                                        None) == B.SPARSE_ATTN_SCRATCH
    # the five workloads fit
    for grid, heads in (((20, 32, 48), 12), ((21, 48, 80), 40), ((32, 48, 80), 24), ((64, 48, 80), 12)):
        s = B.make_shape(1, heads, 128, grid, "bf16")
        assert 0 < B.sparse_attn_select_noalloc_bytes(s) <= B.SPARSE_ATTN_SCRATCH_BYTES
    # the usual argument checks come first
    small = _small()
    assert L.sparse_attn_select_noalloc(ctypes.byref(small), ctypes.byref(params), None, 16, 16, 16,
                                        B.sparse_attn_csr_capacity(small), None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert L.sparse_attn_select_noalloc(ctypes.byref(small), ctypes.byref(params), 16, 16, 16, 16,
                                        B.sparse_attn_csr_capacity(small) - 1, None) == B.SPARSE_ATTN_CAPACITY
    assert "static scratch" in B.status_string(B.SPARSE_ATTN_SCRATCH)



def test_partial_tiles_size_by_ceil_grid():
    """A grid that is not a whole number of tiles has ceil(grid / tile) tiles, the last
    ones partial: 20 x 30 x 45 tokens in 1 x 8 x 8 tiles give 20 x 4 x 6 = 480 blocks,
    whose tile-major tensors hold 64 * 480 slots a head."""
    s = _shape(grid=(20, 30, 45))
    nB = 480
    assert B.sparse_attn_csr_capacity(s) == 12 * nB * nB
    assert B.sparse_attn_workspace_size(s) == B.sparse_attn_workspace_size(_shape(grid=(20, 32, 48)))
    assert B._dims(s) == (64 * nB, nB, 12 * nB)
    assert B._raster_tokens(s) == 20 * 30 * 45


def test_partial_tiles_refused_where_whole_tiles_are_needed():
    """The clustering selector (128-token clusters of whole tiles) takes whole tiles
    only: SPARSE_ATTN_UNSUPPORTED on the host, before any launch.  The backward takes
    partial tiles: on such a grid it passes the shape checks and stops at the null
    pointer (no launch)."""
    L = B.lib()
    s = _shape(grid=(20, 30, 45))
    ws = B.sparse_attn_workspace_size(s)
    cap = B.sparse_attn_csr_capacity(s)
    params = B.SelectParams(0.9, None, -1, -1, -1)
    assert L.sparse_attn_select_ibcs(ctypes.byref(s), ctypes.byref(params), A, A, A, A, cap, A, ws,
                                     None) == B.SPARSE_ATTN_UNSUPPORTED
    assert L.sparse_attn_backward(ctypes.byref(s), None, A, A, A, A, A, A, A, cap, A, A, A, A, A, ws,
                                  None) == B.SPARSE_ATTN_INVALID_ARGUMENT


def test_fine_selection_sizes_and_host_checks():
    """The 4-token selection's sizes, and the shapes and arguments it refuses on the
    host before any HIP call (no GPU needed: no pointer is touched)."""
    L = B.lib()
    s = B.make_shape(1, 12, 128, (20, 32, 48), "bf16")          # nB = 480, nK = 7680
    rows = 12 * 480
    assert B.sparse_attn_fine_csr_capacity(s) == rows * 7680
    ws = B.sparse_attn_fine_workspace_size(s)
    # thresholds, fp32 key means and norms, look-back words of 8-row groups, ticket
    assert ws >= 4 * 12 * 7680 * 128 + 4 * 12 * 7680 + 8 * 12 * 60 + 16
    params = B.SelectParams(0.9, None, -1, -1, -1)
    cap = rows * 7680
    ok = (ctypes.byref(s), ctypes.byref(params), 16, 16, 16, 16, cap, 16, ws, None)
    # unsupported: fp32, partial tiles, more than 512 blocks, a window
    for bad in (B.make_shape(1, 1, 128, (2, 8, 8), "f32"), B.make_shape(1, 1, 128, (2, 12, 20), "bf16"),
                B.make_shape(1, 1, 128, (9, 64, 64), "bf16")):   # 576 blocks
        assert B.sparse_attn_fine_csr_capacity(bad) == B.SPARSE_ATTN_UNSUPPORTED
        assert L.sparse_attn_select_fine(ctypes.byref(bad), ctypes.byref(params), 16, 16, 16, 16, 1 << 40, 16,
                                         1 << 40, None) == B.SPARSE_ATTN_UNSUPPORTED
    win = B.SelectParams(0.9, None, 1, 1, 1)
    assert L.sparse_attn_select_fine(ctypes.byref(s), ctypes.byref(win), 16, 16, 16, 16, cap, 16, ws,
                                     None) == B.SPARSE_ATTN_UNSUPPORTED
    # argument checks
    assert L.sparse_attn_select_fine(ctypes.byref(s), ctypes.byref(params), None, 16, 16, 16, cap, 16, ws,
                                     None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert L.sparse_attn_select_fine(ctypes.byref(s), ctypes.byref(B.SelectParams(0.0, None, -1, -1, -1)), 16, 16,
                                     16, 16, cap, 16, ws, None) == B.SPARSE_ATTN_INVALID_ARGUMENT
    assert L.sparse_attn_select_fine(*ok[:6], cap - 1, *ok[7:]) == B.SPARSE_ATTN_CAPACITY
    assert L.sparse_attn_select_fine(*ok[:8], ws - 1, None) == B.SPARSE_ATTN_WORKSPACE
