"""Thin Python binding of libtriattn.so (the C ABI in include/triattn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the pruning path runs in the library's HIP kernels.
The functions keep the C names.  Failures raise TriError with the library's
status code; a missing library raises at load time (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TRIATTN_LIB: another build of the same library (the CPU sanitizer test loads
# one built with AddressSanitizer); by default the in-tree build.
LIB_PATH = os.environ.get("TRIATTN_LIB") or os.path.join(_HERE, "libtriattn.so")

TRI_OK = 0
TRI_ERR_INVALID_ARG = -1
TRI_ERR_UNSUPPORTED = -2
TRI_ERR_WORKSPACE = -3
TRI_ERR_HIP = -4
TRI_ERR_NO_DEVICE = -5
TRI_DTYPE_F32 = 0
TRI_DTYPE_BF16 = 1
TRI_LAYOUT_DENSE = 0
TRI_LAYOUT_PAGED = 1
TRI_VARIANT_TRIG_ONLY = 1
TRI_VARIANT_NORM_ONLY = 2
TRI_VARIANT_FIXED_WEIGHT = 4
TRI_VARIANT_R_WEIGHTED_TRIG = 8
TRI_PATH_AUTO = 0
TRI_PATH_FULL = 1
TRI_PATH_CANDIDATES = 2
TRI_INPLACE_FILL_FREED = 16
TRI_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "tri_calib_load", "tri_calib_free", "tri_workspace_size", "tri_score", "tri_select_topb",
    "tri_compact", "tri_prune_window", "tri_append", "tri_decode_attn", "tri_strerror",
    "tri_timing_enable", "tri_timing_reset", "tri_timing_read", "tri_timing_name", "tri_last_error",
    "tri_timing_mask",
    "tri_prune_fallbacks", "tri_calibrate_workspace_size", "tri_calibrate", "tri_calib_load_ex",
    "tri_prune_window_ex", "tri_select_topb_ex", "tri_prune_window_static",
)


class TriError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.tri_strerror(code).decode() if _lib is not None else str(code)
        detail = _lib.tri_last_error().decode() if (_lib is not None and code == TRI_ERR_HIP) else ""
        super().__init__(f"{fn} failed: {msg} ({code})" + (f": {detail}" if detail else ""))


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32), ("n_layers", ctypes.c_int32),
        ("layer0", ctypes.c_int32), ("n_seq", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
        ("lengths", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load the built library (no build here: build with long_reasoning_decode_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} missing "
                           "(run python -m long_reasoning_decode_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, D, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float
    I32 = ctypes.c_int32
    SZ = ctypes.c_size_t
    DP = ctypes.POINTER(CacheDesc)
    sig = {
        "tri_calib_load": [ctypes.POINTER(P), I, I, I, I, D, P, P, P, P, I, P],
        "tri_calib_load_ex": [ctypes.POINTER(P), I, I, I, I, D, P, P, P, P, I, I, P],
        "tri_calib_free": [P],
        "tri_workspace_size": [P, DP, I, ctypes.POINTER(SZ)],
        "tri_score": [P, DP, P, P, P, P, P, SZ, P],
        "tri_select_topb": [P, P, I, I, I, P, P, P, SZ, P],
        "tri_select_topb_ex": [P, P, P, I, I, I, P, P, P, SZ, P],
        "tri_compact": [DP, P, P, I, DP, P],
        "tri_prune_window": [P, DP, P, I, DP, P, P, SZ, P],
        "tri_prune_window_ex": [P, DP, P, I, DP, P, P, SZ, I, P],
        "tri_prune_window_static": [P, DP, P, I, DP, P, I, P],
        "tri_append": [DP, P, P, P, P],
        "tri_decode_attn": [DP, I, P, F, P, P],
        "tri_strerror": [I],
        "tri_timing_enable": [I],
        "tri_timing_mask": [ctypes.c_uint32],
        "tri_timing_reset": [],
        "tri_timing_read": [I, ctypes.POINTER(I64), ctypes.POINTER(D)],
        "tri_timing_name": [I],
        "tri_last_error": [],
        "tri_prune_fallbacks": [P, SZ, ctypes.POINTER(I32), P],
        "tri_calibrate_workspace_size": [I, I, I, I, ctypes.POINTER(SZ)],
        "tri_calibrate": [P, I, I, I, I, I, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("tri_strerror", "tri_timing_name", "tri_last_error") else ctypes.c_int
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != TRI_OK:
        raise TriError(fn, rc)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return TRI_DTYPE_BF16
    if dt == torch.float32:
        return TRI_DTYPE_F32
    raise ValueError(f"unsupported cache dtype {dt}")


def cache_desc(k, v, pos, lengths, *, n_layers, n_seq, n_kv_heads, layer0=0, page_table=None,
               page_size=0, max_pages=0):
    """Describe a cache held in torch tensors.  Dense: k/v [n_seg, capacity, d],
    pos [n_seg, capacity]; paged: k/v [n_pages, page_size, d], pos [n_pages,
    page_size] plus page_table [n_seg, max_pages]."""
    for t in (k, v, pos, lengths) + ((page_table,) if page_table is not None else ()):
        if not t.is_contiguous():
            raise ValueError("cache tensors must be contiguous")
    if pos.dtype != torch.int32 or lengths.dtype != torch.int32:
        raise ValueError("positions and lengths are int32")
    d = CacheDesc()
    d.dtype = _dtype_code(k.dtype)
    d.n_layers, d.layer0, d.n_seq, d.n_kv_heads = n_layers, layer0, n_seq, n_kv_heads
    d.head_dim = k.shape[-1]
    d.k, d.v, d.pos, d.lengths = k.data_ptr(), v.data_ptr(), pos.data_ptr(), lengths.data_ptr()
    if page_table is None:
        d.layout = TRI_LAYOUT_DENSE
        d.capacity = k.shape[1]
        d.page_size, d.max_pages, d.page_table = 0, 0, None
    else:
        if page_table.dtype != torch.int32:
            raise ValueError("page table is int32")
        d.layout = TRI_LAYOUT_PAGED
        d.page_size, d.max_pages = page_size, max_pages
        d.capacity = page_size * max_pages
        d.page_table = page_table.data_ptr()
    d._keep = (k, v, pos, lengths, page_table)     # keep the tensors alive with the record
    return d


class Calib:
    """Owns a tri_calib_t."""

    def __init__(self, handle, n_layers, n_q_heads, n_kv_heads, head_dim):
        self.handle = handle
        self.n_layers, self.n_q_heads, self.n_kv_heads, self.head_dim = n_layers, n_q_heads, n_kv_heads, head_dim
        self.group = n_q_heads // n_kv_heads

    def free(self):
        if self.handle:
            _check("tri_calib_free", load().tri_calib_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def tri_calib_load(mag, phase, conc, offsets, *, n_kv_heads, rope_theta, variant=0, stream=None):
    """mag/phase/conc: host fp32 [L, Hq, F]; offsets: host int32 [n_off];
    variant: TRI_VARIANT_* flags (tri_calib_load_ex), 0 = the method as read."""
    lib = load()
    mag = mag.detach().to("cpu", torch.float32).contiguous()
    phase = phase.detach().to("cpu", torch.float32).contiguous()
    conc = conc.detach().to("cpu", torch.float32).contiguous()
    offsets = torch.as_tensor(offsets, dtype=torch.int32).contiguous()
    L, Hq, F = mag.shape
    h = ctypes.c_void_p()
    rc = lib.tri_calib_load_ex(ctypes.byref(h), L, Hq, n_kv_heads, 2 * F, float(rope_theta), _p(mag),
                               _p(phase), _p(conc), _p(offsets), int(offsets.numel()), int(variant), _stream(stream))
    _check("tri_calib_load_ex", rc)
    return Calib(h, L, Hq, n_kv_heads, 2 * F)


def tri_workspace_size(calib, desc, budget):
    n = ctypes.c_size_t(0)
    _check("tri_workspace_size", load().tri_workspace_size(calib.handle, ctypes.byref(desc), int(budget),
                                                            ctypes.byref(n)))
    return n.value


def workspace(calib, desc, budget, device="cuda"):
    return torch.empty(tri_workspace_size(calib, desc, budget), dtype=torch.uint8, device=device)


def tri_score(calib, desc, t, agg, ws, scores=None, mu_sigma=None, stream=None):
    rc = load().tri_score(calib.handle, ctypes.byref(desc), _p(t), _p(scores), _p(agg), _p(mu_sigma),
                          _p(ws), ws.numel(), _stream(stream))
    _check("tri_score", rc)


def tri_select_topb(agg, lengths, budget, idx, n_kept=None, stream=None, pos=None):
    """pos None: tri_select_topb (ties at the cut to the lower slot); else
    tri_select_topb_ex with the slots' positions [n_seg, capacity]."""
    n_seg, cap = agg.shape
    if pos is None:
        rc = load().tri_select_topb(_p(agg), _p(lengths), n_seg, cap, int(budget), _p(idx), _p(n_kept), None, 0,
                                    _stream(stream))
        _check("tri_select_topb", rc)
    else:
        if pos.dtype != torch.int32 or tuple(pos.shape) != (n_seg, cap) or not pos.is_contiguous():
            raise ValueError("pos must be contiguous int32 [n_seg, capacity]")
        rc = load().tri_select_topb_ex(_p(agg), _p(pos), _p(lengths), n_seg, cap, int(budget), _p(idx), _p(n_kept),
                                       None, 0, _stream(stream))
        _check("tri_select_topb_ex", rc)


def tri_compact(src, idx, n_kept, budget, dst, stream=None):
    rc = load().tri_compact(ctypes.byref(src), _p(idx), _p(n_kept), int(budget), ctypes.byref(dst),
                            _stream(stream))
    _check("tri_compact", rc)


def tri_prune_window(calib, src, t, budget, dst, n_kept, ws, stream=None, path=None):
    """path None: tri_prune_window (the automatic path); else tri_prune_window_ex
    with TRI_PATH_AUTO / TRI_PATH_FULL / TRI_PATH_CANDIDATES, optionally or'ed
    with TRI_INPLACE_FILL_FREED."""
    if path is None:
        rc = load().tri_prune_window(calib.handle, ctypes.byref(src), _p(t), int(budget), ctypes.byref(dst),
                                     _p(n_kept), _p(ws), ws.numel(), _stream(stream))
        _check("tri_prune_window", rc)
    else:
        rc = load().tri_prune_window_ex(calib.handle, ctypes.byref(src), _p(t), int(budget), ctypes.byref(dst),
                                        _p(n_kept), _p(ws), ws.numel(), int(path), _stream(stream))
        _check("tri_prune_window_ex", rc)


def tri_prune_window_static(calib, src, t, budget, dst, n_kept, path=TRI_PATH_AUTO, stream=None):
    """tri_prune_window_ex on the library's own scratch (no workspace argument)."""
    rc = load().tri_prune_window_static(calib.handle, ctypes.byref(src), _p(t), int(budget), ctypes.byref(dst),
                                        _p(n_kept), int(path), _stream(stream))
    _check("tri_prune_window_static", rc)


def tri_calibrate(q, mag, phase, conc, ws=None, stream=None):
    """q: device [L, n_samples, Hq, d] pre-RoPE rows (bf16 or fp32); mag, phase,
    conc: device fp32 [L, Hq, d/2] outputs.  Allocates the workspace when none is given."""
    L, n, Hq, d = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    lib = load()
    need = ctypes.c_size_t(0)
    _check("tri_calibrate_workspace_size", lib.tri_calibrate_workspace_size(L, n, Hq, d, ctypes.byref(need)))
    if ws is None:
        ws = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    rc = lib.tri_calibrate(_p(q), _dtype_code(q.dtype), L, n, Hq, d, _p(mag), _p(phase), _p(conc), _p(ws), ws.numel(),
                           _stream(stream))
    _check("tri_calibrate", rc)


def tri_prune_fallbacks(ws, stream=None):
    """Segments the last tri_prune_window on `ws` redid over all keys (synchronising)."""
    n = ctypes.c_int32(0)
    _check("tri_prune_fallbacks", load().tri_prune_fallbacks(_p(ws), ws.numel(), ctypes.byref(n), _stream(stream)))
    return n.value


def tri_append(desc, k_new, v_new, pos_new, stream=None):
    rc = load().tri_append(ctypes.byref(desc), _p(k_new), _p(v_new), _p(pos_new), _stream(stream))
    _check("tri_append", rc)


def tri_decode_attn(desc, n_q_heads, q, scale, out, stream=None):
    rc = load().tri_decode_attn(ctypes.byref(desc), int(n_q_heads), _p(q), float(scale), _p(out),
                                _stream(stream))
    _check("tri_decode_attn", rc)


def tri_strerror(code):
    return load().tri_strerror(int(code)).decode()


def tri_last_error():
    return load().tri_last_error().decode()


def tri_timing_enable(on=True, only=None):
    """Time every kernel, or only the kernels named in `only` (each timed
    launch costs two event records of GPU time)."""
    lib = load()
    mask = 0xFFFFFFFF
    if only is not None:
        names = []
        i = 0
        while lib.tri_timing_name(i) is not None:
            names.append(lib.tri_timing_name(i).decode())
            i += 1
        unknown = set(only) - set(names)
        if unknown:
            raise ValueError(f"unknown kernel names {sorted(unknown)}")
        mask = sum(1 << names.index(n) for n in set(only))
    _check("tri_timing_mask", lib.tri_timing_mask(mask))
    _check("tri_timing_enable", lib.tri_timing_enable(1 if on else 0))


def tri_timing_reset():
    _check("tri_timing_reset", load().tri_timing_reset())


def tri_timing_read():
    """{kernel name: (launches, total ms)} for every instrumented kernel."""
    lib = load()
    out = {}
    i = 0
    while True:
        name = lib.tri_timing_name(i)
        if name is None:
            break
        n = ctypes.c_int64(0)
        ms = ctypes.c_double(0.0)
        _check("tri_timing_read", lib.tri_timing_read(i, ctypes.byref(n), ctypes.byref(ms)))
        out[name.decode()] = (n.value, ms.value)
        i += 1
    return out
