"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, and its argument validation returns the
documented codes before any device work (on a GPU-less host, valid calls
report TRI_ERR_NO_DEVICE)."""
import ctypes
import os
import re

import pytest
import torch

from long_reasoning_decode_amd import triattn as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "triattn.h")

needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(tri_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("tri_calib_load", "tri_score", "tri_select_topb", "tri_compact", "tri_prune_window"):
        assert n in names
    assert set(names) == set(T.EXPORTS)


def test_path_constants_match_the_header():
    """The binding's TRI_PATH_* values are the header's."""
    hdr = open(HEADER).read()
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (TRI_PATH_\w+) (\d+)", hdr)}
    assert vals == {"TRI_PATH_AUTO": T.TRI_PATH_AUTO, "TRI_PATH_FULL": T.TRI_PATH_FULL,
                    "TRI_PATH_CANDIDATES": T.TRI_PATH_CANDIDATES}


def test_timing_mask_is_host_only():
    """Restricting the timed kernels needs no GPU; unknown names are refused."""
    T.tri_timing_enable(True, only=["score", "decode_attn"])
    T.tri_timing_enable(False)
    assert T.load().tri_timing_mask(0xFFFFFFFF) == T.TRI_OK
    with pytest.raises(ValueError):
        T.tri_timing_enable(True, only=["no_such_kernel"])
    T.tri_timing_enable(False)


def test_library_exports_every_declared_symbol():
    lib = T.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_strerror_and_timing_names():
    assert T.tri_strerror(0) == "ok"
    assert "workspace" in T.tri_strerror(T.TRI_ERR_WORKSPACE)
    assert T.tri_strerror(12345) == "unknown status"
    lib = T.load()
    names = []
    while lib.tri_timing_name(len(names)) is not None:
        names.append(lib.tri_timing_name(len(names)).decode())
    assert {"phase", "score", "select_gather", "gather", "decode_attn"} <= set(names)
    assert lib.tri_timing_name(-1) is None
    assert lib.tri_timing_read(len(names), ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_double())) == -1


def _calib_args(L=2, Hq=8, Hkv=2, d=64):
    F = d // 2
    mag = torch.ones(L, Hq, F)
    ph = torch.zeros(L, Hq, F)
    R = torch.full((L, Hq, F), 0.5)
    off = torch.tensor([1, 2, 4], dtype=torch.int32)
    return mag, ph, R, off


def _calib_rc(L=2, Hq=8, Hkv=2, d=64, theta=1e4, mag=None, R=None, off=None, n_off=None):
    lib = T.load()
    m, ph, r, o = _calib_args(L, Hq, Hkv, d)
    m = m if mag is None else mag
    r = r if R is None else R
    o = o if off is None else off
    h = ctypes.c_void_p()
    return lib.tri_calib_load(ctypes.byref(h), L, Hq, Hkv, d, theta, T._p(m), T._p(ph), T._p(r), T._p(o),
                              o.numel() if n_off is None else n_off, None)


def test_calib_validation():
    assert _calib_rc(d=63) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(Hq=6, Hkv=4) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(theta=-1.0) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(R=torch.full((2, 8, 32), 1.5)) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(mag=torch.full((2, 8, 32), -1.0)) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(off=torch.tensor([1, -2], dtype=torch.int32)) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(n_off=0) == T.TRI_ERR_INVALID_ARG
    assert _calib_rc(d=96) == T.TRI_ERR_UNSUPPORTED
    assert _calib_rc(Hq=48, Hkv=2) == T.TRI_ERR_UNSUPPORTED      # group 24


@needs_no_gpu
def test_calib_no_device():
    assert _calib_rc() == T.TRI_ERR_NO_DEVICE


def _desc(**kw):
    k = torch.zeros(4, 16, 64, dtype=torch.bfloat16)
    pos = torch.zeros(4, 16, dtype=torch.int32)
    ln = torch.zeros(4, dtype=torch.int32)
    d = T.cache_desc(k, k.clone(), pos, ln, n_layers=1, n_seq=2, n_kv_heads=2)
    for a, v in kw.items():
        setattr(d, a, v)
    return d


def test_cache_descriptor_validation():
    lib = T.load()
    idx = torch.zeros(4, 8, dtype=torch.int32)
    nk = torch.zeros(4, dtype=torch.int32)
    good = _desc()
    dst = _desc()

    def compact(src, dst, budget=8):
        return lib.tri_compact(ctypes.byref(src), T._p(idx), T._p(nk), budget, ctypes.byref(dst), None)

    assert compact(_desc(dtype=7), dst) == T.TRI_ERR_INVALID_ARG
    assert compact(_desc(layout=3), dst) == T.TRI_ERR_INVALID_ARG
    assert compact(_desc(head_dim=63), dst) == T.TRI_ERR_INVALID_ARG
    assert compact(_desc(head_dim=96), _desc(head_dim=96)) == T.TRI_ERR_UNSUPPORTED
    assert compact(_desc(k=None), dst) == T.TRI_ERR_INVALID_ARG
    assert compact(_desc(n_seq=0), dst) == T.TRI_ERR_INVALID_ARG
    assert compact(_desc(layout=T.TRI_LAYOUT_PAGED), dst) == T.TRI_ERR_INVALID_ARG   # no page table
    assert compact(good, good) == T.TRI_ERR_INVALID_ARG          # in place is refused
    assert compact(good, _desc(n_kv_heads=1, n_seq=4)) == T.TRI_ERR_INVALID_ARG
    assert compact(good, dst, budget=0) == T.TRI_ERR_INVALID_ARG
    assert compact(good, dst, budget=17) == T.TRI_ERR_INVALID_ARG  # dst capacity 16 < budget
    assert lib.tri_compact(ctypes.byref(good), None, T._p(nk), 8, ctypes.byref(dst), None) == T.TRI_ERR_INVALID_ARG


def test_select_validation():
    lib = T.load()
    A = torch.zeros(2, 100)
    ln = torch.zeros(2, dtype=torch.int32)
    idx = torch.zeros(2, 10, dtype=torch.int32)
    sel = lambda n_seg, cap, B, a=A: lib.tri_select_topb(T._p(a), T._p(ln), n_seg, cap, B, T._p(idx), None,
                                                          None, 0, None)
    assert sel(2, 100, 0) == T.TRI_ERR_INVALID_ARG
    assert sel(-1, 100, 10) == T.TRI_ERR_INVALID_ARG
    assert sel(2, 0, 10) == T.TRI_ERR_INVALID_ARG
    assert sel(2, 70000, 10) == T.TRI_ERR_UNSUPPORTED
    assert sel(2, 100, 9000) == T.TRI_ERR_UNSUPPORTED
    assert sel(0, 100, 10) == T.TRI_OK                         # nothing to do
    assert lib.tri_select_topb(None, T._p(ln), 2, 100, 10, T._p(idx), None, None, 0, None) == T.TRI_ERR_INVALID_ARG


@needs_no_gpu
def test_valid_calls_report_no_device():
    lib = T.load()
    A = torch.zeros(2, 100)
    ln = torch.zeros(2, dtype=torch.int32)
    idx = torch.zeros(2, 10, dtype=torch.int32)
    assert lib.tri_select_topb(T._p(A), T._p(ln), 2, 100, 10, T._p(idx), None, None, 0, None) == \
        T.TRI_ERR_NO_DEVICE
    nk = torch.zeros(4, dtype=torch.int32)
    idx4 = torch.zeros(4, 8, dtype=torch.int32)
    src, dst = _desc(), _desc()
    assert lib.tri_compact(ctypes.byref(src), T._p(idx4), T._p(nk), 8, ctypes.byref(dst), None) == \
        T.TRI_ERR_NO_DEVICE
    d = _desc()
    kn = torch.zeros(4, 64, dtype=torch.bfloat16)
    p = torch.zeros(2, dtype=torch.int32)
    assert lib.tri_append(ctypes.byref(d), T._p(kn), T._p(kn), T._p(p), None) == T.TRI_ERR_NO_DEVICE
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 2, 4, 64)
    assert lib.tri_decode_attn(ctypes.byref(d), 4, T._p(q), 0.125, T._p(out), None) == T.TRI_ERR_NO_DEVICE
    assert lib.tri_decode_attn(ctypes.byref(d), 3, T._p(q), 0.125, T._p(out), None) == T.TRI_ERR_INVALID_ARG
    assert lib.tri_decode_attn(ctypes.byref(d), 4, None, 0.125, T._p(out), None) == T.TRI_ERR_INVALID_ARG
    assert lib.tri_decode_attn(ctypes.byref(d), 4, T._p(q), 0.125, None, None) == T.TRI_ERR_INVALID_ARG
    assert lib.tri_decode_attn(ctypes.byref(d), 4, T._p(q), float("nan"), T._p(out), None) == T.TRI_ERR_INVALID_ARG
    assert lib.tri_decode_attn(ctypes.byref(d), 4, T._p(q), float("inf"), T._p(out), None) == T.TRI_ERR_INVALID_ARG
    # two KV heads x 16 query heads each: a group the kernels do not build
    assert lib.tri_decode_attn(ctypes.byref(d), 32, T._p(q), 0.125, T._p(out), None) == T.TRI_ERR_UNSUPPORTED


def test_calib_variant_validation():
    lib = T.load()
    m, ph, r, o = _calib_args()
    h = ctypes.c_void_p()
    rc = lambda v: lib.tri_calib_load_ex(ctypes.byref(h), 2, 8, 2, 64, 1e4, T._p(m), T._p(ph), T._p(r), T._p(o),
                                         o.numel(), v, None)
    assert rc(T.TRI_VARIANT_TRIG_ONLY | T.TRI_VARIANT_NORM_ONLY) == T.TRI_ERR_INVALID_ARG
    assert rc(16) == T.TRI_ERR_INVALID_ARG
    assert rc(-1) == T.TRI_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert rc(T.TRI_VARIANT_FIXED_WEIGHT | T.TRI_VARIANT_R_WEIGHTED_TRIG) == T.TRI_ERR_NO_DEVICE


def test_calib_free_null_is_noop():
    assert T.load().tri_calib_free(None) == 0


def test_calibrate_validation():
    lib = T.load()
    q = torch.zeros(2, 10, 4, 64)
    out = torch.zeros(2, 4, 32)
    raw = torch.zeros((1 << 16) + 256, dtype=torch.uint8)
    skip = (-raw.data_ptr()) % 256
    ws = raw[skip:skip + (1 << 16)]                           # workspaces start on 256-byte boundaries
    n = ctypes.c_size_t(0)
    assert lib.tri_calibrate_workspace_size(2, 10, 4, 64, ctypes.byref(n)) == T.TRI_OK and n.value > 0
    assert lib.tri_calibrate_workspace_size(2, 10, 4, 63, ctypes.byref(n)) == T.TRI_ERR_INVALID_ARG
    assert lib.tri_calibrate_workspace_size(2, 10, 4, 96, ctypes.byref(n)) == T.TRI_ERR_UNSUPPORTED
    assert lib.tri_calibrate_workspace_size(0, 10, 4, 64, ctypes.byref(n)) == T.TRI_ERR_INVALID_ARG
    cal = lambda *, dt=T.TRI_DTYPE_F32, L=2, ns=10, qp=T._p(q), wb=ws.numel(): lib.tri_calibrate(
        qp, dt, L, ns, 4, 64, T._p(out), T._p(out), T._p(out), T._p(ws), wb, None)
    assert cal(dt=5) == T.TRI_ERR_INVALID_ARG
    assert cal(ns=0) == T.TRI_ERR_INVALID_ARG
    assert cal(qp=None) == T.TRI_ERR_INVALID_ARG
    assert cal(qp=ctypes.c_void_p(q.data_ptr() + 4)) == T.TRI_ERR_INVALID_ARG   # rows must be 16-byte aligned
    assert cal(wb=16) == T.TRI_ERR_WORKSPACE
    assert lib.tri_calibrate(T._p(q), T.TRI_DTYPE_F32, 2, 10, 4, 64, T._p(out), T._p(out), T._p(out),
                             ctypes.c_void_p(ws.data_ptr() + 16), ws.numel() - 16, None) == T.TRI_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert cal() == T.TRI_ERR_NO_DEVICE


def test_append_refuses_paged_caches():
    lib = T.load()
    k = torch.zeros(8, 16, 64, dtype=torch.bfloat16)          # pool of 8 pages x 16 rows
    pos = torch.zeros(8, 16, dtype=torch.int32)
    ln = torch.zeros(4, dtype=torch.int32)
    pt = torch.zeros(4, 2, dtype=torch.int32)
    d = T.cache_desc(k, k.clone(), pos, ln, n_layers=1, n_seq=2, n_kv_heads=2, page_table=pt, page_size=16,
                     max_pages=2)
    kn = torch.zeros(4, 64, dtype=torch.bfloat16)
    p = torch.zeros(2, dtype=torch.int32)
    assert lib.tri_append(ctypes.byref(d), T._p(kn), T._p(kn), T._p(p), None) == T.TRI_ERR_UNSUPPORTED
    assert lib.tri_append(ctypes.byref(d), None, T._p(kn), T._p(p), None) == T.TRI_ERR_INVALID_ARG


def test_compaction_refuses_overlapping_storage():
    """Out-of-place compaction: dense arrays that overlap src's by any byte are
    refused before any launch; adjacent arrays are not; a paged dst on src's
    pool through another page table (fresh pages of a shared pool) is
    accepted, the same page table is not (that is src itself)."""
    lib = T.load()
    idx = torch.zeros(4, 8, dtype=torch.int32)
    nk = torch.zeros(4, dtype=torch.int32)
    big = torch.zeros(3 * 4 * 16 * 64, dtype=torch.bfloat16)        # room for k, v and a shifted k
    pos = torch.zeros(2 * 4 * 16, dtype=torch.int32)
    ln = torch.zeros(4, dtype=torch.int32)
    kv_elems = 4 * 16 * 64

    def dense(k_off, v_off, p_off):
        d = T.cache_desc(big[:kv_elems].view(4, 16, 64), big[:kv_elems].view(4, 16, 64), pos[:64].view(4, 16), ln,
                         n_layers=1, n_seq=2, n_kv_heads=2)
        d.k = big.data_ptr() + 2 * k_off
        d.v = big.data_ptr() + 2 * v_off
        d.pos = pos.data_ptr() + 4 * p_off
        return d

    def compact(src, dst):
        return lib.tri_compact(ctypes.byref(src), T._p(idx), T._p(nk), 8, ctypes.byref(dst), None)

    src = dense(0, kv_elems, 0)
    ok = T.TRI_ERR_NO_DEVICE if not torch.cuda.is_available() else None
    assert compact(src, dense(2 * kv_elems - 64, 2 * kv_elems + 0, 64)) == T.TRI_ERR_INVALID_ARG   # dst.k in src.v
    assert compact(src, dense(2 * kv_elems, 2 * kv_elems, 32)) == T.TRI_ERR_INVALID_ARG            # pos overlap
    if ok is not None:
        assert compact(src, dense(2 * kv_elems, 2 * kv_elems, 64)) == ok                           # adjacent
    pool = torch.zeros(16, 16, 64, dtype=torch.bfloat16)
    ppos = torch.zeros(16, 16, dtype=torch.int32)
    pt_src = torch.arange(8, dtype=torch.int32).view(4, 2)
    pt_dst = torch.arange(8, 16, dtype=torch.int32).view(4, 2)
    paged = lambda pt: T.cache_desc(pool, pool, ppos, ln, n_layers=1, n_seq=2, n_kv_heads=2, page_table=pt,
                                    page_size=16, max_pages=2)
    assert compact(paged(pt_src), paged(pt_src)) == T.TRI_ERR_INVALID_ARG
    if ok is not None:
        assert compact(paged(pt_src), paged(pt_dst)) == ok
