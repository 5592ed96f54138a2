"""Shared test plumbing: building caches from the seeded generators, running the
HIP path through the C ABI, running the oracle on the same bytes, and the
tolerance checks.

Tolerances (from the arithmetic: fp32 accumulation of exact bf16 products and
an fp32 aggregate, against the oracle's fp64):
  scores S_h : |gpu - ref| <= 1e-4 * max(|ref|, rms of the head's ref scores).
               The fp32 error is bounded relative to the sum of the terms'
               magnitudes, not to |S|: scores near zero (the trig term
               cancelling the norm term) measured up to 8e-3 of |S| against
               the fp64 oracle at head_dim 64, so a bare relative bound cannot
               hold there
  mu, sigma  : |gpu - ref| <= 1e-4 * max(|ref mu|, ref sigma)
  A          : |gpu - ref| <= 1e-4 * max(|ref|, 1)
  top-B      : same count, ascending; a slot may differ from the oracle's set
               only if |A_ref - T| <= 1e-4 * |T|, T = oracle's B-th largest
               aggregated score (ties at the cut: the earlier position)
  K', V', p' : bit-exact copies of the rows the GPU kept
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W

RTOL = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def calib_for(T, cfg, variant=0):
    cal = W.calibration(cfg)
    c = T.tri_calib_load(cal["mag"], cal["phase"], cal["conc"], cal["offsets"],
                         n_kv_heads=cfg.n_kv_heads, rope_theta=cfg.theta, variant=variant)
    return c, cal


def dense_desc(T, cfg, cache, layers=None):
    n_layers = cfg.n_layers if layers is None else layers
    return T.cache_desc(cache["k"], cache["v"], cache["pos"], cache["lengths"], n_layers=n_layers,
                        n_seq=cfg.n_seq, n_kv_heads=cfg.n_kv_heads)


def empty_like_dense(cache, capacity):
    n_seg, _, d = cache["k"].shape
    dev = cache["k"].device
    return {
        "k": torch.zeros((n_seg, capacity, d), dtype=cache["k"].dtype, device=dev),
        "v": torch.zeros((n_seg, capacity, d), dtype=cache["k"].dtype, device=dev),
        "pos": torch.full((n_seg, capacity), -1, dtype=torch.int32, device=dev),
        "lengths": torch.zeros((n_seg,), dtype=torch.int32, device=dev),
    }


def seg_calib(cal, cfg, s, layer0=0):
    """(M, phi, R) [G][F] numpy arrays of segment s's query heads."""
    per_l = cfg.n_seq * cfg.n_kv_heads
    l = s // per_l + layer0
    h = s % cfg.n_kv_heads
    G = cfg.group
    sl = slice(h * G, (h + 1) * G)
    return (cal["mag"][l, sl].numpy(), cal["phase"][l, sl].numpy(), cal["conc"][l, sl].numpy())


def seg_seq(cfg, s):
    return (s // cfg.n_kv_heads) % cfg.n_seq


def oracle_segment(cfg, cal, K, V, pos, t, s, B, layer0=0, variant=0):
    """Oracle prune of one segment from its stored rows (numpy, already CPU)."""
    M, phi, R = seg_calib(cal, cfg, s, layer0)
    return oracle.prune_segment(K, V, pos, t, cfg.theta, M, phi, R, cfg.offsets, B, variant=variant)


def oracle_select(cfg, cal, K, pos, t, s, B, layer0=0):
    """Oracle scores, statistics, aggregate and top-B of one segment (no gather)."""
    M, phi, R = seg_calib(cal, cfg, s, layer0)
    S = oracle.score_segment(K, pos, t, cfg.theta, M, phi, R, cfg.offsets)
    mu, sigma, A = oracle.zscore_max(S)
    return {"S": S, "mu": mu, "sigma": sigma, "A": A, "idx": oracle.select_topb(A, B, pos)}


def check_scores(S_gpu, S_ref, what=""):
    """Error per score relative to max(|S|, the head's rms score)."""
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    rms = np.sqrt(np.mean(S_ref ** 2, axis=1, keepdims=True))
    scale = np.maximum(np.abs(S_ref), rms)
    err = np.abs(S_gpu - S_ref) / scale
    assert err.max() <= RTOL, f"{what} score mismatch: max scaled err {err.max():.3e}"
    return err.max()


def check_mu_sigma(ms_gpu, mu, sigma, what=""):
    ms_gpu = np.asarray(ms_gpu, dtype=np.float64)
    scale = np.maximum(np.abs(mu), sigma)
    assert np.all(np.abs(ms_gpu[:, 0] - mu) <= RTOL * scale), f"{what} mu {ms_gpu[:, 0]} vs {mu}"
    assert np.all(np.abs(ms_gpu[:, 1] - sigma) <= RTOL * scale), f"{what} sigma {ms_gpu[:, 1]} vs {sigma}"


def check_agg(A_gpu, A_ref, what=""):
    A_gpu = np.asarray(A_gpu, dtype=np.float64)
    err = np.abs(A_gpu - A_ref) / np.maximum(np.abs(A_ref), 1.0)
    assert err.max() <= RTOL, f"{what} aggregate mismatch: max err {err.max():.3e}"


def check_selection(idx_gpu, A_ref, B, what="", pos=None):
    """idx_gpu against the oracle's top-B of A_ref (ties at the cut to the
    earlier of the slots' positions pos; None: slot order) under the tie band."""
    idx_gpu = np.asarray(idx_gpu)
    N = len(A_ref)
    if N <= B:
        assert np.array_equal(idx_gpu, np.arange(N)), f"{what}: N <= B must keep every slot"
        return 0
    assert len(idx_gpu) == B, f"{what}: kept {len(idx_gpu)} != {B}"
    assert np.all(np.diff(idx_gpu) > 0), f"{what}: kept slots not strictly ascending"
    assert idx_gpu.min() >= 0 and idx_gpu.max() < N
    ref = oracle.select_topb(A_ref, B, pos)
    thr = np.sort(A_ref)[-B]
    diff = np.setxor1d(ref, idx_gpu)
    band = RTOL * abs(thr)
    bad = [int(i) for i in diff if abs(A_ref[i] - thr) > band]
    assert not bad, f"{what}: {len(bad)} slots differ away from the cut (e.g. {bad[:5]}, thr {thr})"
    return len(diff)


def kept_slots_from_positions(pos_src, pos_dst):
    """Slots the GPU kept, recovered from the compacted positions (positions of
    a segment are distinct)."""
    order = np.argsort(pos_src, kind="stable")
    where = np.searchsorted(pos_src[order], pos_dst)
    assert np.all(pos_src[order][where] == pos_dst), "compacted position not present in the source"
    return order[where]


def check_compaction(Ks, Vs, Ps, Kd, Vd, Pd, idx, what=""):
    assert np.array_equal(Kd, Ks[idx]), f"{what}: K rows not bit-exact"
    assert np.array_equal(Vd, Vs[idx]), f"{what}: V rows not bit-exact"
    assert np.array_equal(Pd, Ps[idx]), f"{what}: positions not bit-exact"


def stored(x):
    return W.to_stored_numpy(x)


def check_in_place(cfg, cal, Kb, Vb, Pb, Ka, Va, Pa, N, nk, t, s, B, tag, oop_kept=None, fill=False):
    """One segment pruned in place.  b: its rows before the prune (all slots);
    a: after.  The kept set against the oracle's top-B (and, when given, the
    out-of-place pass's set); the arrangement: slot order, as out of place, or
    with fill the oracle's fill-freed-slots layout of that set; rows
    bit-exact, rows at or above the kept count untouched."""
    nks = min(N, B)
    assert nk == nks, f"{tag}: kept count {nk} != {nks}"
    if N == 0:
        return
    K, V, P = Kb[:N], Vb[:N], Pb[:N]
    ix = kept_slots_from_positions(P, Pa[:nks])
    kept = np.sort(ix)
    ref = oracle_segment(cfg, cal, K, V, P, t, s, B)
    check_selection(kept, ref["A"], B, tag, pos=P)
    if oop_kept is not None:
        assert np.array_equal(kept, oop_kept), f"{tag}: kept set differs from the out-of-place pass"
    layout = oracle.fill_freed_layout(kept, N) if fill else kept
    assert np.array_equal(ix, layout), f"{tag}: arrangement is not the {'fill-freed' if fill else 'slot-order'} layout"
    check_compaction(K, V, P, Ka[:nks], Va[:nks], Pa[:nks], ix, tag)
    assert np.array_equal(Ka[nks:], Kb[nks:]) and np.array_equal(Va[nks:], Vb[nks:]) and \
        np.array_equal(Pa[nks:], Pb[nks:]), f"{tag}: rows at or above the kept count were written"
