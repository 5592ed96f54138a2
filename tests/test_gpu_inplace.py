"""In-place pruning: tri_prune_window with dst naming src's storage.  Per
segment, against the oracle:
* the kept set (oracle top-B under the tie band), and byte for byte the set the
  out-of-place pass keeps on the same input;
* the arrangement: slot order, so the pruned rows equal the out-of-place
  pass's output byte for byte; or, with TRI_INPLACE_FILL_FREED, the oracle's
  fill-freed-slots layout of that kept set, exactly;
* K/V rows and positions bit-exact, rows at or above the kept count untouched;
* lengths updated through n_kept aliasing them.
Dense bf16 and fp32, the candidate pass (including more moved rows than one
batch holds), ragged lengths around the budget, paged pools, ties broken by
position on a cache whose slots are not in position order, and the argument
checks."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (calib_for, check_in_place, check_selection, dense_desc, empty_like_dense,
                     kept_slots_from_positions, log, seg_seq, stored)

pytestmark = pytest.mark.gpu


def _dense_in_place(T, cfg, cpu, B, what, fill=False):
    """Out-of-place pass on one copy, in-place pass on another; check both."""
    calib, cal = calib_for(T, cfg)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cpu.items()}
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, B)
    out = empty_like_dense(g, B)
    nk_oop = torch.full_like(g["lengths"], -1)
    # (the candidate pass wherever the cache allows it: these batches are too
    # small for the automatic path to take it)
    T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), nk_oop, ws, path=T.TRI_PATH_CANDIDATES)
    torch.cuda.synchronize()
    fb_oop = T.tri_prune_fallbacks(ws)
    # in place, n_kept = the cache's own lengths
    path = T.TRI_PATH_CANDIDATES | (T.TRI_INPLACE_FILL_FREED if fill else 0)
    T.tri_prune_window(calib, desc, g["t"], B, desc, g["lengths"], ws, path=path)
    torch.cuda.synchronize()
    fb = T.tri_prune_fallbacks(ws)
    log(f"  fallbacks: out of place {fb_oop}, in place {fb}")
    lengths = cpu["lengths"].numpy()
    Kb, Vb, Pb = stored(cpu["k"]), stored(cpu["v"]), cpu["pos"].numpy()
    Ka, Va, Pa = stored(g["k"].cpu()), stored(g["v"].cpu()), g["pos"].cpu().numpy()
    nk = g["lengths"].cpu().numpy()
    assert np.array_equal(nk, nk_oop.cpu().numpy())
    P_oop = out["pos"].cpu().numpy()
    K_oop, V_oop = stored(out["k"].cpu()), stored(out["v"].cpu())
    for s in range(len(lengths)):
        N = int(lengths[s])
        nks = min(N, B)
        oop = kept_slots_from_positions(Pb[s, :N], P_oop[s, :nks]) if N else None
        check_in_place(cfg, cal, Kb[s], Vb[s], Pb[s], Ka[s], Va[s], Pa[s], N, int(nk[s]),
                       int(cpu["t"][seg_seq(cfg, s)]), s, B, f"{what} seg {s} N={N}", oop, fill=fill)
        if not fill:                                   # the same bytes as out of place
            assert np.array_equal(Ka[s, :nks], K_oop[s, :nks]) and np.array_equal(Va[s, :nks], V_oop[s, :nks]) \
                and np.array_equal(Pa[s, :nks], P_oop[s, :nks]), f"{what} seg {s}: in place differs from out of place"


@pytest.mark.parametrize("fill", [False, True])
@pytest.mark.parametrize("d,G,dtype", [(128, 4, torch.bfloat16), (64, 8, torch.bfloat16), (64, 2, torch.float32)])
def test_in_place_ragged_lengths(gpu_lib, d, G, dtype, fill):
    """Segments of length 0, 1, B-1, B, B+1, chunk-straddling and full (full-score path)."""
    B, cap = 200, 2600
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=dtype, theta=1e6, n_kv_heads=3, n_seq=3,
                                    n_keys=cap, t=cap + 5, budget=B, sigma=None, seed=21)
    log(f"case in place ragged d={d} G={G} {dtype} fill={fill}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([0, 1, B - 1, B, B + 1, 513, 1024, 2047, cap], dtype=torch.int32)
    _dense_in_place(gpu_lib, cfg, cpu, B, f"in place d{d} G{G}", fill=fill)


@pytest.mark.parametrize("d,G", [(128, 4), (64, 8), (128, 1), (64, 2), (128, 2), (64, 4)])
def test_in_place_candidate_pass(gpu_lib, d, G):
    """Lengths around the candidate-mode boundaries (4096 and 8B)."""
    B, cap = 600, 12000
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=torch.bfloat16, theta=1e6, n_kv_heads=3, n_seq=3,
                                    n_keys=cap, t=cap + 3, budget=B, sigma=None, seed=23)
    log(f"case in place candidate d={d} G={G}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 4095, 4096, 8 * B - 1, 8 * B, 8 * B + 1, 9001, B + 1, cap - 17],
                                  dtype=torch.int32)
    _dense_in_place(gpu_lib, cfg, cpu, B, f"in place candidate d{d} G{G}")


@pytest.mark.parametrize("fill", [False, True])
def test_in_place_many_moved_rows(gpu_lib, fill):
    """Many moved rows: in slot order up to 4096 rows in 256-row batches; in the
    fill mode more than 2048 kept rows above the kept count, whose freed slots
    are found in two batches.  One candidate-mode segment (N = 65536, B = 4096)
    and one on the full-score path (N = 12000, B = 4096 < N < 8B)."""
    B, cap = 4096, 65536
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=1, n_seq=2,
                                    n_keys=cap, t=cap + 1, budget=B, sigma=None, seed=25)
    log(f"case in place, many moved rows, fill={fill}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 12000], dtype=torch.int32)
    _dense_in_place(gpu_lib, cfg, cpu, B, "in place many moves", fill=fill)


def test_in_place_maximum_sizes(gpu_lib):
    """The largest segment and budget: 65536 keys, B = 8192 (candidate pass, up
    to four batches of freed slots), and a 30000-key segment on the full-score
    path."""
    B, cap = 8192, 65536
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=1, n_seq=2,
                                    n_keys=cap, t=cap + 1, budget=B, sigma=None, seed=33)
    log("case in place, maximum sizes")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 30000], dtype=torch.int32)
    _dense_in_place(gpu_lib, cfg, cpu, B, "in place maximum")


def test_candidate_select_36_keys_per_thread(gpu_lib):
    """B = 4500: segments below 8 B = 36000 keys list every key, so the
    candidate select holds up to 36000 entries (36 per thread).  Candidate and
    full-score segments, in place and out of place, against the oracle."""
    B, cap = 4500, 40000
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=1, n_seq=5,
                                    n_keys=cap, t=cap + 1, budget=B, sigma=None, seed=37)
    log("case candidate select, 36 keys per thread")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 36000, 35999, 20000, B + 1], dtype=torch.int32)
    _dense_in_place(gpu_lib, cfg, cpu, B, "in place J36")


@pytest.mark.parametrize("fill", [False, True])
@pytest.mark.parametrize("page_size", [16, 24])
def test_in_place_paged(gpu_lib, page_size, fill):
    """A ragged paged pool (random page tables) pruned where it is; in slot
    order its pages then hold exactly what the out-of-place pass writes to
    fresh pages."""
    T = gpu_lib
    cfg = W.CONFIGS["ragged"].replace(n_seq=3, len_range=(100, 3000), budget=256, seed=27, page_size=page_size)
    log(f"case in place paged, {page_size}-token pages, fill={fill}")
    pc = W.paged_cache(cfg, "cpu")
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in pc.items()}
    calib, cal = calib_for(T, cfg)
    B = cfg.budget
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                       max_pages=g["max_pages"])
    ws = T.workspace(calib, src, B)
    # out of place into a dense cache of B rows, first
    oop = empty_like_dense({"k": torch.empty((cfg.n_seg, 1, cfg.head_dim), dtype=cfg.dtype, device="cuda")}, B)
    T.tri_prune_window(calib, src, g["t"], B, dense_desc(T, cfg, oop), oop["lengths"], ws)
    T.tri_prune_window(calib, src, g["t"], B, src, g["lengths"], ws,
                       path=T.TRI_PATH_AUTO | (T.TRI_INPLACE_FILL_FREED if fill else 0))
    torch.cuda.synchronize()
    pt = pc["page_table"].numpy()
    ps = cfg.page_size
    Kp0, Vp0, Pp0 = stored(pc["k"]), stored(pc["v"]), pc["pos"].numpy()
    Kp1, Vp1, Pp1 = stored(g["k"].cpu()), stored(g["v"].cpu()), g["pos"].cpu().numpy()
    Ko, Vo, Po = stored(oop["k"].cpu()), stored(oop["v"].cpu()), oop["pos"].cpu().numpy()
    nk = g["lengths"].cpu().numpy()
    for s in range(cfg.n_seg):
        N = int(pc["lengths"][s])
        n_rows = (N + ps - 1) // ps * ps                     # the segment's own pages only
        rows = lambda pool: oracle.paged_rows(pool, pt[s], ps, n_rows)
        check_in_place(cfg, cal, rows(Kp0), rows(Vp0), rows(Pp0), rows(Kp1), rows(Vp1), rows(Pp1), N,
                       int(nk[s]), int(pc["t"][seg_seq(cfg, s)]), s, B, f"in place paged seg {s} N={N}", fill=fill)
        if not fill:
            nks = min(N, B)
            assert np.array_equal(rows(Kp1)[:nks], Ko[s, :nks]) and np.array_equal(rows(Vp1)[:nks], Vo[s, :nks]) \
                and np.array_equal(rows(Pp1)[:nks], Po[s, :nks]), f"paged seg {s}: in place differs from out of place"


@pytest.mark.parametrize("path", ["full", "candidates"])
def test_ties_keep_the_earliest_positions(gpu_lib, path):
    """A cache whose slots are not in position order (positions a random
    permutation), with twice the best key's row written into 1001 scattered
    slots: the copies score identically on the GPU (the score reads the stored
    row only), the cut falls inside them (B = 512), and the 512 copies at the
    earliest positions must be kept, whatever their slots.  Out of place, in
    place and in place filling freed slots all keep that set.  The oracle
    un-rotates each copy by its own position, so its copies differ at the
    rounding level of fp64 and it keeps some other 512 of them: the GPU's set
    is checked against it under the tie band."""
    T = gpu_lib
    B, N = 512, 8192
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=1, n_seq=1,
                                    n_keys=N, t=N + 1, budget=B, sigma=None, seed=41)
    log(f"case ties by position ({path})")
    cpu = W.dense_cache(cfg, "cpu")
    gen = torch.Generator().manual_seed(4141)
    cpu["pos"][0] = torch.randperm(N, generator=gen).to(torch.int32)
    calib, cal = calib_for(T, cfg)
    Kb, Vb, Pb = stored(cpu["k"][0]), stored(cpu["v"][0]), cpu["pos"][0].numpy()
    ref0 = oracle.prune_segment(Kb, Vb, Pb, cfg.t, cfg.theta, *[x[0, :4].numpy() for x in
                                (cal["mag"], cal["phase"], cal["conc"])], cfg.offsets, B)
    best = int(np.argmax(ref0["A"]))
    dup = np.union1d(torch.randperm(N, generator=gen)[:1000].numpy(), [best])
    cpu["k"][0, dup] = (cpu["k"][0, best] * 2).clone()       # twice the best key: far above the rest
    K2 = stored(cpu["k"][0])
    ref = oracle.prune_segment(K2, Vb, Pb, cfg.t, cfg.theta, *[x[0, :4].numpy() for x in
                               (cal["mag"], cal["phase"], cal["conc"])], cfg.offsets, B)
    rest = np.setdiff1d(np.arange(N), dup)
    assert ref["A"][rest].max() < ref["A"][dup].min() - 1e-3, "the copies are not the top keys"
    want = np.sort(dup[np.argsort(Pb[dup], kind="stable")[:B]])   # the copies at the earliest positions
    p = T.TRI_PATH_FULL if path == "full" else T.TRI_PATH_CANDIDATES
    results = {}
    for mode in ("out", "in", "fill"):
        g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cpu.items()}
        desc = dense_desc(T, cfg, g)
        ws = T.workspace(calib, desc, B)
        if mode == "out":
            out = empty_like_dense(g, B)
            T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws, path=p)
            Pd = out["pos"][0].cpu().numpy()
        else:
            T.tri_prune_window(calib, desc, g["t"], B, desc, g["lengths"], ws,
                               path=p | (T.TRI_INPLACE_FILL_FREED if mode == "fill" else 0))
            Pd = g["pos"][0, :B].cpu().numpy()
        torch.cuda.synchronize()
        kept = np.sort(kept_slots_from_positions(Pb, Pd))
        results[mode] = kept
        assert np.array_equal(kept, want), f"{mode}: kept {len(np.setxor1d(kept, want))} slots off the earliest positions"
    # the oracle's top-B of the modified cache, under the tie band
    check_selection(results["out"], ref["A"], B, f"ties {path}", pos=Pb)


def test_in_place_argument_checks(gpu_lib):
    """Sharing that is not the same storage is refused before any launch."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(head_dim=64, group=2, dtype=torch.bfloat16, n_kv_heads=1, n_seq=1,
                                    n_keys=600, t=600, budget=100)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in W.dense_cache(cfg, "cpu").items()}
    calib, _ = calib_for(T, cfg)
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, 100)
    other_v = torch.empty_like(g["v"])
    half = T.cache_desc(g["k"], other_v, g["pos"], g["lengths"], n_layers=1, n_seq=1, n_kv_heads=1)
    with pytest.raises(T.TriError) as e:
        T.tri_prune_window(calib, desc, g["t"], 100, half, g["lengths"], ws)
    assert e.value.code == T.TRI_ERR_INVALID_ARG
    shifted = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=1, n_kv_heads=1, layer0=0)
    shifted.capacity = desc.capacity - 1
    with pytest.raises(T.TriError) as e:
        T.tri_prune_window(calib, desc, g["t"], 100, shifted, g["lengths"], ws)
    assert e.value.code == T.TRI_ERR_INVALID_ARG
    out = empty_like_dense(g, 100)
    for path in (3, -1, 32, T.TRI_INPLACE_FILL_FREED | 3):   # no such path
        with pytest.raises(T.TriError) as e:
            T.tri_prune_window(calib, desc, g["t"], 100, dense_desc(T, cfg, out), out["lengths"], ws, path=path)
        assert e.value.code == T.TRI_ERR_INVALID_ARG
    with pytest.raises(T.TriError) as e:                      # compaction alone stays out of place
        idx = torch.zeros((1, 100), dtype=torch.int32, device="cuda")
        T.tri_compact(desc, idx, g["lengths"], 100, desc)
    assert e.value.code == T.TRI_ERR_INVALID_ARG
