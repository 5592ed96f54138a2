"""TriAttention KV-cache pruning oracle (TEST INFRASTRUCTURE ONLY).

A plain, slow fp64 CPU implementation of the pruning path, written from the
pages' description (see ``triattn_oracle.c`` for each step and its source).
Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline may import this package; the product library never does, and the two
share no code.  This module is argument marshalling (numpy <-> C) plus a
thread pool that runs independent segments side by side.

Sources: the yeyulingfeng.com page "实现单卡4090跑通OpenClaw!...TriAttention"
(section 主要方法) and the zingnex.cn page "TriAttention：用三角级数压缩KV缓存..."
(sections 预RoPE空间的发现, TriAttention的核心机制).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "triattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
# score variants (orc_score_segment_variant): the ablated components and the R-weighted centre reading
VAR_TRIG_ONLY = 1
VAR_NORM_ONLY = 2
VAR_FIXED_WEIGHT = 4
VAR_R_WEIGHTED_TRIG = 8

_lib = None


def build() -> str:
    """Compile the oracle with the host C compiler (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    dbl = ctypes.c_double
    lib.orc_score_segment.argtypes = [P, i32, P, i64, i32, dbl, i64, P, P, P, i32, P, i32, P, P, P]
    lib.orc_score_segment_variant.argtypes = [P, i32, P, i64, i32, dbl, i64, P, P, P, i32, P, i32, i32, P, P, P]
    lib.orc_zscore_max.argtypes = [P, i32, i64, P, P, P]
    lib.orc_select_topb.argtypes = [P, P, i64, i64, P, P]
    lib.orc_select_topb_f32.argtypes = [P, P, i64, i64, P, P]
    lib.orc_gather_rows.argtypes = [P, i64, P, i64, P]
    lib.orc_paged_rows.argtypes = [P, i64, P, i32, i64, P]
    lib.orc_fill_freed_layout.argtypes = [P, i64, i64, P]
    lib.orc_decode_attn.argtypes = [P, i32, P, P, i32, i64, i32, i32, dbl, P]
    lib.orc_calibrate.argtypes = [P, i32, i64, i32, P, P, P]
    for fn in (lib.orc_score_segment, lib.orc_zscore_max, lib.orc_select_topb,
               lib.orc_select_topb_f32, lib.orc_gather_rows, lib.orc_paged_rows,
               lib.orc_decode_attn, lib.orc_calibrate, lib.orc_score_segment_variant,
               lib.orc_fill_freed_layout):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stored(rows: np.ndarray) -> tuple[np.ndarray, int]:
    """Stored rows as (contiguous array, dtype code): float32, or bf16 bit patterns (uint16)."""
    rows = np.ascontiguousarray(rows)
    if rows.dtype == np.float32:
        return rows, F32
    if rows.dtype == np.uint16:
        return rows, BF16
    raise TypeError(f"stored rows must be float32 or bf16 bits (uint16), got {rows.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def score_segment(K, pos, t, theta, M, phi, R, offsets, parts=False, variant=0):
    """S [G][N] (fp64) for one segment.  K: [N][d] stored rows; M, phi, R: [G][F];
    variant: VAR_* flags (0 = the method as read)."""
    lib = _load()
    K, dt = _stored(K)
    N, d = K.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    M = np.ascontiguousarray(M, dtype=np.float32)
    phi = np.ascontiguousarray(phi, dtype=np.float32)
    R = np.ascontiguousarray(R, dtype=np.float32)
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    G = M.shape[0]
    assert M.shape == (G, d // 2) and phi.shape == M.shape and R.shape == M.shape
    assert pos.shape == (N,)
    S = np.empty((G, N), dtype=np.float64)
    trig = np.empty((G, N), dtype=np.float64) if parts else None
    norm = np.empty((G, N), dtype=np.float64) if parts else None
    rc = lib.orc_score_segment_variant(_ptr(K), dt, _ptr(pos), N, d, float(theta), int(t), _ptr(M),
                                       _ptr(phi), _ptr(R), G, _ptr(offs), len(offs), int(variant), _ptr(S),
                                       _ptr(trig) if parts else None, _ptr(norm) if parts else None)
    _check(rc, "score_segment")
    return (S, trig, norm) if parts else S


def zscore_max(S):
    """(mu [G], sigma [G], A [N]) from S [G][N]."""
    lib = _load()
    S = np.ascontiguousarray(S, dtype=np.float64)
    G, N = S.shape
    mu = np.empty(G)
    sigma = np.empty(G)
    A = np.empty(N)
    _check(lib.orc_zscore_max(_ptr(S), G, N, _ptr(mu), _ptr(sigma), _ptr(A)), "zscore_max")
    return mu, sigma, A


def select_topb(A, B, pos=None):
    """Ascending kept slots.  A: fp64 or fp32 aggregated scores [N]; pos: the
    slots' positions [N] (ties at the cut go to the earlier position), or None
    when slot order is position order."""
    lib = _load()
    A = np.ascontiguousarray(A)
    N = A.shape[0]
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        assert pos.shape == (N,)
    idx = np.empty(max(min(N, B), 1), dtype=np.int32)
    nk = ctypes.c_int64(0)
    pp = _ptr(pos) if pos is not None else None
    if A.dtype == np.float32:
        rc = lib.orc_select_topb_f32(_ptr(A), pp, N, int(B), _ptr(idx), ctypes.byref(nk))
    else:
        A = A.astype(np.float64, copy=False)
        rc = lib.orc_select_topb(_ptr(A), pp, N, int(B), _ptr(idx), ctypes.byref(nk))
    _check(rc, "select_topb")
    return idx[: nk.value].copy()


def gather_rows(src, idx):
    """dst[j] = src[idx[j]], byte for byte."""
    lib = _load()
    src = np.ascontiguousarray(src)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    row_bytes = src[0:1].nbytes if src.shape[0] else src.itemsize * int(np.prod(src.shape[1:]))
    dst = np.empty((len(idx),) + src.shape[1:], dtype=src.dtype)
    _check(lib.orc_gather_rows(_ptr(src), row_bytes, _ptr(idx), len(idx), _ptr(dst)), "gather_rows")
    return dst


def fill_freed_layout(kept, N):
    """Slot arrangement of a segment pruned in place in the fill-freed-slots
    mode: entry j is the pre-prune slot of the key now in slot j (kept slots
    below len(kept) stay put; the kept slots above fill the freed ones in
    ascending order)."""
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    out = np.empty(len(kept), dtype=np.int32)
    _check(_load().orc_fill_freed_layout(_ptr(kept), len(kept), int(N), _ptr(out)), "fill_freed_layout")
    return out


def paged_rows(pool, page_table, page_size, n):
    """Rows 0..n-1 of a paged segment, in slot order.  pool: [P][page_size][...]."""
    lib = _load()
    pool = np.ascontiguousarray(pool)
    flat = pool.reshape((pool.shape[0] * pool.shape[1],) + pool.shape[2:])
    row_bytes = flat[0:1].nbytes
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    dst = np.empty((n,) + flat.shape[1:], dtype=flat.dtype)
    _check(lib.orc_paged_rows(_ptr(flat), row_bytes, _ptr(pt), int(page_size), int(n), _ptr(dst)),
           "paged_rows")
    return dst


def decode_attn(q, K, V, scale):
    """out [G][d] (fp64) = softmax(scale q K^T) V for the G heads sharing K/V."""
    lib = _load()
    q, qdt = _stored(q)
    K, kdt = _stored(K)
    V, vdt = _stored(V)
    assert kdt == vdt
    G, d = q.shape
    N = K.shape[0]
    out = np.empty((G, d), dtype=np.float64)
    _check(lib.orc_decode_attn(_ptr(q), qdt, _ptr(K), _ptr(V), kdt, N, d, G, float(scale),
                               _ptr(out)), "decode_attn")
    return out


def calibrate(q):
    """Centre magnitude, phase and concentration per band of one query head
    from sampled pre-RoPE rows q [n][d] (fp32 or bf16-as-uint16): fp64 [F] x 3."""
    qs, dt = _stored(q)
    n, d = qs.shape
    M = np.zeros(d // 2)
    phi = np.zeros(d // 2)
    R = np.zeros(d // 2)
    _check(_load().orc_calibrate(_ptr(qs), dt, n, d, _ptr(M), _ptr(phi), _ptr(R)), "orc_calibrate")
    return M, phi, R


def prune_segment(K, V, pos, t, theta, M, phi, R, offsets, B, variant=0):
    """The whole path for one segment: scores, z/max, top-B, compaction."""
    S = score_segment(K, pos, t, theta, M, phi, R, offsets, variant=variant)
    mu, sigma, A = zscore_max(S)
    idx = select_topb(A, B, pos)
    return {
        "S": S, "mu": mu, "sigma": sigma, "A": A, "idx": idx,
        "K": gather_rows(K, idx), "V": gather_rows(V, idx),
        "pos": np.asarray(pos, dtype=np.int32)[idx],
    }


def host_threads() -> int:
    """Threads the oracle runs on: the process's CPU share, which is
    OMP_NUM_THREADS where the host sets one (the cores a job is given on a
    shared machine), else every core the process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def run_parallel(fn, items, threads=None):
    """Map fn over independent items on a thread pool (the C calls release the GIL)."""
    items = list(items)
    if threads is None:
        threads = min(len(items), host_threads()) or 1
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
