"""GPU parity at sizes the oracle finishes in seconds: every step of the HIP path
(through the C ABI) against the oracle on the same seeded inputs, plus the edge
cases (empty, single-key, under/at/over budget, ragged chunk tails, equal
scores, every supported GQA group and head size, fp32 and bf16, paged)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (calib_for, check_agg, check_compaction, check_in_place, check_mu_sigma, check_scores,
                     check_selection, dense_desc, empty_like_dense, kept_slots_from_positions, log,
                     oracle_segment, seg_calib, seg_seq, stored)

pytestmark = pytest.mark.gpu


def _to(cache, device):
    return {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in cache.items()}


def _run_unfused(T, cfg, g, calib, B, path=None):
    """The unfused chain, then the fused pass on the same cache.  These batches
    are too small for the automatic path to take the candidate pass, so the
    fused pass asks for it (it applies wherever the cache allows it) unless a
    path is given."""
    path = T.TRI_PATH_CANDIDATES if path is None else path
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, B)
    n_seg, cap = g["k"].shape[0], g["k"].shape[1]
    G = cfg.group
    scores = torch.full((n_seg, G, cap), float("nan"), device="cuda")
    agg = torch.full((n_seg, cap), float("nan"), device="cuda")
    ms = torch.zeros((n_seg, G, 2), device="cuda")
    T.tri_score(calib, desc, g["t"], agg, ws, scores=scores, mu_sigma=ms)
    idx = torch.full((n_seg, B), -1, dtype=torch.int32, device="cuda")
    nk = torch.full((n_seg,), -1, dtype=torch.int32, device="cuda")
    T.tri_select_topb(agg, g["lengths"], B, idx, nk)
    out = empty_like_dense(g, B)
    T.tri_compact(desc, idx, nk, B, dense_desc(T, cfg, out))
    # the same cache through the fused entry point
    out2 = empty_like_dense(g, B)
    nk2 = torch.full((n_seg,), -1, dtype=torch.int32, device="cuda")
    T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out2), nk2, ws, path=path)
    fallbacks = T.tri_prune_fallbacks(ws)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu(), agg=agg.cpu(), ms=ms.cpu(), idx=idx.cpu(), nk=nk.cpu(), out=_to(out, "cpu"),
                out2=_to(out2, "cpu"), nk2=nk2.cpu(), fallbacks=fallbacks)


def _check_all(cfg, cal, cpu, r, B, lengths, what, variant=0):
    """Oracle on every segment of a small dense cache, all steps."""
    n_seg = cpu["k"].shape[0]
    for s in range(n_seg):
        N = int(lengths[s])
        t = int(cpu["t"][seg_seq(cfg, s)])
        tag = f"{what} seg {s} N={N}"
        assert int(r["nk"][s]) == min(N, B) and int(r["nk2"][s]) == min(N, B), tag
        if N == 0:
            continue
        K, V = stored(cpu["k"][s, :N]), stored(cpu["v"][s, :N])
        P = cpu["pos"][s, :N].numpy()
        ref = oracle_segment(cfg, cal, K, V, P, t, s, B, variant=variant)
        check_scores(r["scores"][s, :, :N].numpy(), ref["S"], tag)
        check_mu_sigma(r["ms"][s].numpy(), ref["mu"], ref["sigma"], tag)
        check_agg(r["agg"][s, :N].numpy(), ref["A"], tag)
        nk = min(N, B)
        idx = r["idx"][s, :nk].numpy()
        check_selection(idx, ref["A"], B, tag)
        o = r["out"]
        check_compaction(K, V, P, stored(o["k"][s, :nk]), stored(o["v"][s, :nk]), o["pos"][s, :nk].numpy(), idx, tag)
        # fused pass: byte-identical to the unfused chain
        o2 = r["out2"]
        for key in ("k", "v", "pos"):
            assert torch.equal(o2[key][s, :nk], o[key][s, :nk]), f"{tag}: fused {key} differs from unfused"


def test_tiny_config_every_step(gpu_lib):
    T = gpu_lib
    cfg = W.CONFIGS["tiny"]
    log(f"case tiny: N={cfg.n_keys} B={cfg.budget} d={cfg.head_dim} fp32")
    cpu = W.dense_cache(cfg, "cpu")
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, cfg.budget)
    _check_all(cfg, cal, cpu, r, cfg.budget, cpu["lengths"].numpy(), "tiny")


@pytest.mark.parametrize("d,G,dtype,theta", [
    (128, 4, torch.bfloat16, 1e6), (64, 8, torch.bfloat16, 150000.0), (128, 1, torch.bfloat16, 1e6),
    (64, 2, torch.float32, 1e4), (128, 8, torch.float32, 1e6), (64, 4, torch.bfloat16, 1e4)])
def test_ragged_lengths_every_step(gpu_lib, d, G, dtype, theta):
    """Segments of length 0, 1, B-1, B, B+1, chunk-straddling and full."""
    T = gpu_lib
    B = 200
    cap = 2600
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=dtype, theta=theta, n_kv_heads=3, n_seq=3,
                                    n_keys=cap, t=cap + 5, budget=B, sigma=None, seed=7)
    log(f"case ragged d={d} G={G} {dtype}")
    cpu = W.dense_cache(cfg, "cpu")
    lengths = torch.tensor([0, 1, B - 1, B, B + 1, 513, 1024, 2047, cap], dtype=torch.int32)
    cpu["lengths"] = lengths
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    _check_all(cfg, cal, cpu, r, B, lengths.numpy(), f"ragged d{d} G{G}")


def test_equal_scores_keep_lowest_slots(gpu_lib):
    """Identical keys: zero spread, z = 0 everywhere, the cut takes the lowest slots."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, dtype=torch.bfloat16, theta=1e6, n_keys=3000, t=3000, budget=700)
    log("case equal scores")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["k"][0, :] = cpu["k"][0, 5]
    cpu["pos"][0, :] = 5            # same position too, so every score is bit-identical
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, cfg.budget)
    assert torch.all(r["ms"][0, :, 1] == 0.0)
    assert torch.all(r["agg"][0, :3000] == 0.0)
    assert torch.equal(r["idx"][0], torch.arange(700, dtype=torch.int32))
    _check_all(cfg, cal, cpu, r, cfg.budget, cpu["lengths"].numpy(), "equal")


@pytest.mark.parametrize("with_pos", [False, True])
@pytest.mark.parametrize("cap", [700, 2048, 4096, 8192, 32768, 32896, 40000, 65536])
def test_select_kernel_bit_exact(gpu_lib, cap, with_pos):
    """tri_select_topb on seeded score arrays (ties, signed zeros, all-equal)
    equals the oracle's selection exactly; with positions (tri_select_topb_ex:
    a random permutation in even segments, a few hundred repeated values in odd
    ones), ties at the cut go to the earliest position, then the lower slot."""
    T = gpu_lib
    n_seg = 8
    A = W.synthetic_scores(n_seg, cap, seed=cap)
    B = min(4096, cap // 3)
    lengths = torch.tensor([cap, 0, 1, B, B + 1, cap - 1, cap // 2 + 7, cap], dtype=torch.int32)
    log(f"case select cap={cap} B={B} positions={with_pos}")
    pos = None
    if with_pos:
        gen = torch.Generator().manual_seed(cap + 1)
        pos = torch.stack([torch.randperm(cap, generator=gen) if s % 2 == 0 else
                           torch.randint(-300, 300, (cap,), generator=gen) for s in range(n_seg)]).to(torch.int32)
    idx = torch.full((n_seg, B), -1, dtype=torch.int32, device="cuda")
    nk = torch.full((n_seg,), -1, dtype=torch.int32, device="cuda")
    T.tri_select_topb(A.cuda(), lengths.cuda(), B, idx, nk, pos=None if pos is None else pos.cuda())
    torch.cuda.synchronize()
    idx, nk = idx.cpu(), nk.cpu()
    for s in range(n_seg):
        N = int(lengths[s])
        ref = oracle.select_topb(A[s, :N].numpy(), B, None if pos is None else pos[s, :N].numpy())
        assert int(nk[s]) == len(ref), f"seg {s}"
        assert np.array_equal(idx[s, :len(ref)].numpy(), ref), f"cap {cap} seg {s} N {N}"


@pytest.mark.parametrize("page_size,dtype", [(16, torch.bfloat16), (8, torch.bfloat16), (24, torch.bfloat16),
                                             (64, torch.bfloat16), (16, torch.float32), (24, torch.float32)])
def test_paged_small_every_step(gpu_lib, page_size, dtype):
    """Ragged paged pool, every step against the oracle; page sizes other than
    the 16 tokens of the workloads (one of them not a power of two), bf16 and
    fp32 pools."""
    T = gpu_lib
    cfg = W.CONFIGS["ragged"].replace(n_seq=3, len_range=(100, 3000), budget=256, seed=3, page_size=page_size,
                                      dtype=dtype)
    log(f"case paged small, {page_size}-token pages, {dtype}")
    pc = W.paged_cache(cfg, "cpu")
    g = _to(pc, "cuda")
    calib, cal = calib_for(T, cfg)
    B, G, n_seg = cfg.budget, cfg.group, cfg.n_seg
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                       max_pages=g["max_pages"])
    cap = cfg.page_size * g["max_pages"]
    ws = T.workspace(calib, src, B)
    scores = torch.zeros((n_seg, G, cap), device="cuda")
    agg = torch.zeros((n_seg, cap), device="cuda")
    ms = torch.zeros((n_seg, G, 2), device="cuda")
    T.tri_score(calib, src, g["t"], agg, ws, scores=scores, mu_sigma=ms)
    idx = torch.full((n_seg, B), -1, dtype=torch.int32, device="cuda")
    nk = torch.zeros((n_seg,), dtype=torch.int32, device="cuda")
    T.tri_select_topb(agg, g["lengths"], B, idx, nk)
    dst = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                       max_pages=g["out_max_pages"])
    T.tri_compact(src, idx, nk, B, dst)
    torch.cuda.synchronize()
    first = {k: g[k].clone() for k in ("out_k", "out_v", "out_pos")}
    for k in ("out_k", "out_v", "out_pos"):
        g[k].zero_()
    nk2 = torch.zeros_like(nk)
    dst2 = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk2, n_layers=1, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                        max_pages=g["out_max_pages"])
    T.tri_prune_window(calib, src, g["t"], B, dst2, nk2, ws)
    torch.cuda.synchronize()
    for k in ("out_k", "out_v", "out_pos"):
        assert torch.equal(g[k], first[k]), f"fused paged {k} differs from unfused"
    lengths = pc["lengths"].numpy()
    for s in range(n_seg):
        N = int(lengths[s])
        t = int(pc["t"][seg_seq(cfg, s)])
        pt = pc["page_table"][s].numpy()
        K = oracle.paged_rows(stored(pc["k"]), pt, cfg.page_size, N)
        V = oracle.paged_rows(stored(pc["v"]), pt, cfg.page_size, N)
        P = oracle.paged_rows(pc["pos"].numpy(), pt, cfg.page_size, N)
        ref = oracle_segment(cfg, cal, K, V, P, t, s, B)
        tag = f"paged seg {s} N={N}"
        check_scores(scores[s, :, :N].cpu().numpy(), ref["S"], tag)
        check_agg(agg[s, :N].cpu().numpy(), ref["A"], tag)
        nks = min(N, B)
        assert int(nk[s]) == nks
        ix = idx[s, :nks].cpu().numpy()
        check_selection(ix, ref["A"], B, tag)
        opt = pc["out_page_table"][s].numpy()
        Kd = oracle.paged_rows(stored(first["out_k"].cpu()), opt, cfg.page_size, nks)
        Vd = oracle.paged_rows(stored(first["out_v"].cpu()), opt, cfg.page_size, nks)
        Pd = oracle.paged_rows(first["out_pos"].cpu().numpy(), opt, cfg.page_size, nks)
        check_compaction(K, V, P, Kd, Vd, Pd, ix, tag)


@pytest.mark.parametrize("d,G,dtype", [(128, 4, torch.bfloat16), (64, 8, torch.bfloat16), (128, 1, torch.bfloat16),
                                       (64, 2, torch.float32)])
@pytest.mark.parametrize("path", ["full", "candidates"])
def test_split_select_matches_the_single_workgroup_select(gpu_lib, d, G, dtype, path):
    """Fewer than 256 segments of at least 8192 slots, out of place: the split
    select (one workgroup per segment and chunk) and the many-workgroup
    gather.  In place the same cache goes through the one-workgroup select and
    gather, which leaves the same bytes; both are compared on lengths at and
    around the budget, chunk boundaries and the capacity, and against the
    oracle's selection."""
    T = gpu_lib
    B, cap = 600, 9000
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=dtype, theta=1e6, n_kv_heads=2, n_seq=7,
                                    n_keys=cap, t=cap + 3, budget=B, sigma=None, seed=61)
    log(f"case split select d={d} G={G} {dtype} {path}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([0, 1, B - 1, B, B + 1, 511, 512, 513, 2047, 2049, 4096, 4801, cap - 1, cap],
                                  dtype=torch.int32)
    calib, cal = calib_for(T, cfg)
    p = T.TRI_PATH_FULL if path == "full" else T.TRI_PATH_CANDIDATES
    g = _to(cpu, "cuda")
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, B)
    out = empty_like_dense(g, B)
    T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws, path=p)
    fb = T.tri_prune_fallbacks(ws)
    T.tri_prune_window(calib, desc, g["t"], B, desc, g["lengths"], ws, path=p)
    torch.cuda.synchronize()
    log(f"  split select fallbacks: {fb}")
    lengths = cpu["lengths"].numpy()
    assert torch.equal(out["lengths"], g["lengths"])
    for s in range(cfg.n_seg):
        nk = min(int(lengths[s]), B)
        for key in ("k", "v", "pos"):
            assert torch.equal(out[key][s, :nk], g[key][s, :nk]), f"seg {s} N={lengths[s]}: {key} differs"
        N = int(lengths[s])
        if N > B:
            P = cpu["pos"][s, :N].numpy()
            ref = oracle_segment(cfg, cal, stored(cpu["k"][s, :N]), stored(cpu["v"][s, :N]), P,
                                 int(cpu["t"][seg_seq(cfg, s)]), s, B)
            check_selection(out["pos"][s, :nk].cpu().numpy(), ref["A"], B, f"split seg {s} N={N}", pos=P)


def test_paged_prune_into_fresh_pages_of_the_same_pool(gpu_lib):
    """Out of place into pages of the source's own pool (a second page table
    over pages the source does not use): the same pages' contents as pruning
    into a separate pool, and the source pages untouched."""
    T = gpu_lib
    cfg = W.CONFIGS["ragged"].replace(n_seq=3, len_range=(100, 3000), budget=256, seed=5)
    log("case paged prune into the source pool")
    pc = W.paged_cache(cfg, "cpu")
    g = _to(pc, "cuda")
    calib, _ = calib_for(T, cfg)
    B = cfg.budget
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                       max_pages=g["max_pages"])
    ws = T.workspace(calib, src, B)
    nk = torch.zeros((cfg.n_seg,), dtype=torch.int32, device="cuda")
    sep = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                       max_pages=g["out_max_pages"])
    T.tri_prune_window(calib, src, g["t"], B, sep, nk, ws)
    # one pool holding the source pages and, after them, the fresh pages
    n_src = g["k"].shape[0]
    pool = {key: torch.cat([g[key], torch.zeros_like(g["out_" + key])]) for key in ("k", "v", "pos")}
    src2 = T.cache_desc(pool["k"], pool["v"], pool["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                        max_pages=g["max_pages"])
    pt2 = (g["out_page_table"] + n_src).contiguous()
    nk2 = torch.zeros_like(nk)
    dst2 = T.cache_desc(pool["k"], pool["v"], pool["pos"], nk2, n_layers=1, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, page_table=pt2, page_size=cfg.page_size,
                        max_pages=g["out_max_pages"])
    T.tri_prune_window(calib, src2, g["t"], B, dst2, nk2, ws)
    torch.cuda.synchronize()
    assert torch.equal(nk2, nk)
    for key in ("k", "v", "pos"):
        assert torch.equal(pool[key][n_src:], g["out_" + key]), f"{key}: fresh pages differ from the separate pool"
        assert torch.equal(pool[key][:n_src], g[key]), f"{key}: source pages were written"


@pytest.mark.parametrize("page_size", [16, 24])
def test_paged_split_select_into_fresh_pages(gpu_lib, page_size):
    """Few paged segments of at least 8192 slots, out of place: the split
    select, whose emission copies each chunk's kept rows into the fresh pages.
    Byte for byte the unfused chain's result (tri_compact's gather) on every
    segment, and the oracle's selection and compaction on a sample."""
    T = gpu_lib
    cfg = W.CONFIGS["ragged"].replace(n_seq=2, len_range=(7000, 12000), budget=1024, seed=17, page_size=page_size)
    log(f"case paged split select, {page_size}-token pages")
    pc = W.paged_cache(cfg, "cpu")
    g = _to(pc, "cuda")
    calib, cal = calib_for(T, cfg)
    B, n_seg = cfg.budget, cfg.n_seg
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                       max_pages=g["max_pages"])
    cap = cfg.page_size * g["max_pages"]
    assert n_seg < 256 and cap >= 8192, "the case must take the split select"
    ws = T.workspace(calib, src, B)
    agg = torch.zeros((n_seg, cap), device="cuda")
    T.tri_score(calib, src, g["t"], agg, ws)
    idx = torch.full((n_seg, B), -1, dtype=torch.int32, device="cuda")
    nk = torch.zeros((n_seg,), dtype=torch.int32, device="cuda")
    T.tri_select_topb(agg, g["lengths"], B, idx, nk)
    dst = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                       max_pages=g["out_max_pages"])
    T.tri_compact(src, idx, nk, B, dst)
    torch.cuda.synchronize()
    first = {k: g[k].clone() for k in ("out_k", "out_v", "out_pos")}
    for k in ("out_k", "out_v", "out_pos"):
        g[k].fill_(-1)
    nk2 = torch.zeros_like(nk)
    dst2 = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk2, n_layers=1, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                        max_pages=g["out_max_pages"])
    T.tri_prune_window(calib, src, g["t"], B, dst2, nk2, ws)
    torch.cuda.synchronize()
    assert torch.equal(nk2, nk)
    lengths = pc["lengths"].numpy()
    for s in range(n_seg):
        nks = min(int(lengths[s]), B)
        opt = pc["out_page_table"][s].numpy()
        for k in ("out_k", "out_v", "out_pos"):
            a = oracle.paged_rows(stored_t(g[k].cpu()).numpy() if k != "out_pos" else g[k].cpu().numpy(),
                                  opt, cfg.page_size, nks)
            b = oracle.paged_rows(stored_t(first[k].cpu()).numpy() if k != "out_pos" else first[k].cpu().numpy(),
                                  opt, cfg.page_size, nks)
            assert np.array_equal(a, b), f"seg {s}: {k} differs from the unfused chain"
    for s in (0, n_seg // 2, n_seg - 1):
        N = int(lengths[s])
        t = int(pc["t"][seg_seq(cfg, s)])
        pt = pc["page_table"][s].numpy()
        K = oracle.paged_rows(stored(pc["k"]), pt, cfg.page_size, N)
        V = oracle.paged_rows(stored(pc["v"]), pt, cfg.page_size, N)
        P = oracle.paged_rows(pc["pos"].numpy(), pt, cfg.page_size, N)
        ref = oracle_segment(cfg, cal, K, V, P, t, s, B)
        tag = f"paged split seg {s} N={N}"
        nks = min(N, B)
        ix = idx[s, :nks].cpu().numpy()
        check_selection(ix, ref["A"], B, tag)
        opt = pc["out_page_table"][s].numpy()
        Kd = oracle.paged_rows(stored(g["out_k"].cpu()), opt, cfg.page_size, nks)
        Vd = oracle.paged_rows(stored(g["out_v"].cpu()), opt, cfg.page_size, nks)
        Pd = oracle.paged_rows(g["out_pos"].cpu().numpy(), opt, cfg.page_size, nks)
        check_compaction(K, V, P, Kd, Vd, Pd, ix, tag)


@pytest.mark.parametrize("in_place", [False, True, "fill"])
def test_decode_loop_small(gpu_lib, in_place):
    """Append + decode attention each step, prune after each window (into the
    other buffer, or in place, or in place filling freed slots), on a
    GPT-OSS-shaped but small cache.  In place, the same window state is also
    pruned out of place first: slot order gives the same bytes, the fill mode
    the same kept set."""
    T = gpu_lib
    cfg = W.CONFIGS["gptoss"].replace(n_layers=2, n_seq=3, budget=64, window=8, windows=3, start_pos_range=512)
    log(f"case decode small, in place {in_place}")
    st = _to(W.decode_start(cfg, "cpu"), "cuda")
    km = W.key_model(cfg)
    calib, cal = calib_for(T, cfg)
    cap = st["capacity"]
    caches = [st, {**empty_like_dense(st, cap), "t": st["t"]}]
    cur = 0
    t = cfg.start_pos_range
    scale = 1.0 / math.sqrt(cfg.head_dim)
    for w in range(cfg.windows):
        for j in range(cfg.window):
            c = caches[cur]
            desc = dense_desc(T, cfg, c)
            k_new, v_new, q = W.decode_token(cfg, km, w * cfg.window + j, t, "cpu")
            pos_new = torch.full((cfg.n_seq,), t, dtype=torch.int32, device="cuda")
            T.tri_append(desc, k_new.cuda(), v_new.cuda(), pos_new)
            out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
            T.tri_decode_attn(desc, cfg.n_q_heads, q.cuda(), scale, out)
            torch.cuda.synchronize()
            if j in (0, cfg.window - 1):
                for s in range(cfg.n_seg):
                    N = int(c["lengths"][s])
                    l, b, h = s // (cfg.n_seq * cfg.n_kv_heads), seg_seq(cfg, s), s % cfg.n_kv_heads
                    qs = q[l, b, h * cfg.group:(h + 1) * cfg.group]
                    ref = oracle.decode_attn(stored(qs), stored(c["k"][s, :N].cpu()), stored(c["v"][s, :N].cpu()),
                                             scale)
                    got = out[l, b, h * cfg.group:(h + 1) * cfg.group].cpu().numpy()
                    err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
                    assert err.max() <= 1e-4, f"attention w{w} step {j} seg {s}: {err.max():.2e}"
            t += 1
        c = caches[cur]
        c["t"] = torch.full((cfg.n_seq,), t, dtype=torch.int32, device="cuda")
        desc = dense_desc(T, cfg, c)
        ws = T.workspace(calib, desc, cfg.budget)
        if in_place:
            fill = in_place == "fill"
            before = {k: c[k].cpu() for k in ("k", "v", "pos", "lengths")}
            oop = empty_like_dense(c, cfg.budget)
            T.tri_prune_window(calib, desc, c["t"], cfg.budget, dense_desc(T, cfg, oop), oop["lengths"], ws)
            T.tri_prune_window(calib, desc, c["t"], cfg.budget, desc, c["lengths"], ws,
                               path=T.TRI_INPLACE_FILL_FREED if fill else T.TRI_PATH_AUTO)
            torch.cuda.synchronize()
            Ka, Va, Pa = stored(c["k"].cpu()), stored(c["v"].cpu()), c["pos"].cpu().numpy()
            Kb, Vb, Pb = stored(before["k"]), stored(before["v"]), before["pos"].numpy()
            Po = oop["pos"].cpu().numpy()
            for s in range(cfg.n_seg):
                N, nks = int(before["lengths"][s]), int(c["lengths"][s])
                oop_kept = np.sort(kept_slots_from_positions(Pb[s, :N], Po[s, :nks]))
                check_in_place(cfg, cal, Kb[s], Vb[s], Pb[s], Ka[s], Va[s], Pa[s], N, nks, t, s, cfg.budget,
                               f"decode window {w} seg {s} in place", oop_kept, fill=fill)
                if not fill:
                    assert np.array_equal(Pa[s, :nks], Po[s, :nks]) and \
                        np.array_equal(Ka[s, :nks], stored(oop["k"][s, :nks].cpu())), \
                        f"decode window {w} seg {s}: in place differs from out of place"
            continue
        nxt = caches[1 - cur]
        nk = nxt["lengths"]
        T.tri_prune_window(calib, desc, c["t"], cfg.budget, dense_desc(T, cfg, nxt), nk, ws)
        torch.cuda.synchronize()
        for s in range(cfg.n_seg):
            N = int(c["lengths"][s])
            K, V, P = stored(c["k"][s, :N].cpu()), stored(c["v"][s, :N].cpu()), c["pos"][s, :N].cpu().numpy()
            ref = oracle_segment(cfg, cal, K, V, P, t, s, cfg.budget)
            nks = int(nk[s])
            assert nks == min(N, cfg.budget)
            Pd = nxt["pos"][s, :nks].cpu().numpy()
            ix = kept_slots_from_positions(P, Pd)
            check_selection(ix, ref["A"], cfg.budget, f"decode window {w} seg {s}")
            check_compaction(K, V, P, stored(nxt["k"][s, :nks].cpu()), stored(nxt["v"][s, :nks].cpu()), Pd, ix)
        nxt["t"] = c["t"]
        cur = 1 - cur


# ---------------------------------------------------------------- candidate pass
# bf16 segments with N >= 4096 and N >= 8B run the fused pass on candidate lists
# (keys reaching a sampled per-head threshold) with a certificate and a full
# fallback; the result must equal the unfused chain byte for byte.

@pytest.mark.parametrize("d,G", [(128, 4), (64, 8), (128, 1), (64, 2)])
def test_candidate_pass_every_step(gpu_lib, d, G):
    """Lengths around the candidate-mode boundaries (4096 and 8B), ragged tails."""
    T = gpu_lib
    B = 600
    cap = 12000
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=torch.bfloat16, theta=1e6, n_kv_heads=3, n_seq=3,
                                    n_keys=cap, t=cap + 3, budget=B, sigma=None, seed=11)
    log(f"case candidate pass d={d} G={G}")
    cpu = W.dense_cache(cfg, "cpu")
    lengths = torch.tensor([cap, 4095, 4096, 8 * B - 1, 8 * B, 8 * B + 1, 9001, B + 1, cap - 17], dtype=torch.int32)
    cpu["lengths"] = lengths
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    log(f"  fallbacks: {r['fallbacks']}")
    assert r["fallbacks"] == 0
    _check_all(cfg, cal, cpu, r, B, lengths.numpy(), f"candidate d{d} G{G}")


def _sampled_slots(N, s, n_sample=256):
    """Slots the threshold sample of segment s reads: one per stratum of
    N // n_sample keys, at a hashed offset (the kernel's stratified rule)."""
    stride = N // n_sample
    return [j * stride + (((j * 2654435761 + s * 40503) & 0xFFFFFFFF) >> 8) % stride for j in range(n_sample)]


def test_candidate_pass_fallback_redoes_segment(gpu_lib):
    """Segment 0's sampled keys are scaled up 4x, so its thresholds sit far
    above the rest of its keys: too few candidates, the certificate fails and
    the segment is redone over every key.  Segment 1 is ordinary."""
    T = gpu_lib
    B = 300
    cap = 8192
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=2, n_seq=1,
                                    n_keys=cap, t=cap, budget=B, sigma=None, seed=5)
    log("case candidate fallback")
    cpu = W.dense_cache(cfg, "cpu")
    sampled = torch.tensor(_sampled_slots(cap, 0))
    cpu["k"][0, sampled] = cpu["k"][0, sampled] * 4           # exact in bf16
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    log(f"  fallbacks: {r['fallbacks']}")
    assert r["fallbacks"] == 1
    _check_all(cfg, cal, cpu, r, B, cpu["lengths"].numpy(), "fallback")


def test_candidate_pass_equal_scores(gpu_lib):
    """All keys identical in candidate mode (N = 8B): the sample has no spread,
    so every key is a candidate (N of them, which the select step can hold),
    and the kept set is the lowest B slots.  (This one-segment batch takes the
    split select, which hands ties at the cut beyond the budget, here every
    key, to the single-workgroup select: one fallback.)"""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, dtype=torch.bfloat16, theta=1e6, n_keys=9000, t=9000, budget=1125)
    log("case candidate equal scores")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["k"][0, :] = cpu["k"][0, 5]
    cpu["v"][0, :] = torch.arange(9000, dtype=torch.float32)[:, None].to(torch.bfloat16)
    cpu["pos"][0, :] = 5
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, cfg.budget)
    assert r["fallbacks"] == 1
    assert torch.equal(r["out2"]["v"][0], cpu["v"][0, :1125])
    _check_all(cfg, cal, cpu, r, cfg.budget, cpu["lengths"].numpy(), "candidate equal")


def test_candidate_pass_overflow_falls_back(gpu_lib):
    """All keys identical with N > 8B: every key is a candidate, more than the
    select step holds for this budget (max(N/2, 8B) = 7200 < 9000), so the
    segment is redone in full; the kept set is the lowest B slots."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, dtype=torch.bfloat16, theta=1e6, n_keys=9000, t=9000, budget=900)
    log("case candidate overflow")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["k"][0, :] = cpu["k"][0, 5]
    cpu["v"][0, :] = torch.arange(9000, dtype=torch.float32)[:, None].to(torch.bfloat16)
    cpu["pos"][0, :] = 5
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, cfg.budget)
    assert r["fallbacks"] == 1
    assert torch.equal(r["out2"]["v"][0], cpu["v"][0, :900])
    _check_all(cfg, cal, cpu, r, cfg.budget, cpu["lengths"].numpy(), "candidate overflow")


# ---------------------------------------------------------------- score variants
VARIANTS = {
    "trig_only": (1, 1), "norm_only": (2, 2), "fixed_weight": (4, 4), "r_weighted_trig": (8, 8),
    "trig_only_r_weighted": (9, 9),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_score_variants_every_step(gpu_lib, name):
    """Each variant through the unfused chain and the fused pass (candidate mode
    included: N = 9000 >= 8B) against the oracle with the same flags; the
    linear-offset ablation is a different offset set."""
    T = gpu_lib
    lib_flag, orc_flag = VARIANTS[name]
    B = 800
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, dtype=torch.bfloat16, theta=1e6, n_kv_heads=2, n_seq=1,
                                    n_keys=9000, t=9000, budget=B, sigma=None, seed=21,
                                    offsets=tuple(range(1, 17)) if name == "r_weighted_trig" else W.geometric(16))
    log(f"case variant {name}")
    cpu = W.dense_cache(cfg, "cpu")
    calib, cal = calib_for(T, cfg, variant=lib_flag)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    log(f"  fallbacks: {r['fallbacks']}")
    _check_all(cfg, cal, cpu, r, B, cpu["lengths"].numpy(), f"variant {name}", variant=orc_flag)


@pytest.mark.parametrize("page_size", [16, 24, 8])
def test_paged_decode_attention_over_pruned_pages(gpu_lib, page_size):
    """Decode attention reading a pruned paged cache in place (fresh pages with
    random page tables, per-KV-head kept counts) against the oracle."""
    import math
    T = gpu_lib
    cfg = W.CONFIGS["ragged"].replace(n_seq=3, len_range=(100, 3000), budget=256, seed=4, page_size=page_size)
    log(f"case paged decode attention, {page_size}-token pages")
    pc = W.paged_cache(cfg, "cpu")
    g = _to(pc, "cuda")
    calib, cal = calib_for(T, cfg)
    B = cfg.budget
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["page_table"], page_size=cfg.page_size,
                       max_pages=g["max_pages"])
    nk = torch.zeros((cfg.n_seg,), dtype=torch.int32, device="cuda")
    dst = T.cache_desc(g["out_k"], g["out_v"], g["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=g["out_page_table"], page_size=cfg.page_size,
                       max_pages=g["out_max_pages"])
    T.tri_prune_window(calib, src, g["t"], B, dst, nk, T.workspace(calib, src, B))
    gq = torch.Generator().manual_seed(77)
    q = torch.randn((1, cfg.n_seq, cfg.n_q_heads, cfg.head_dim), generator=gq).to(cfg.dtype)
    out = torch.full(q.shape, float("nan"), device="cuda")
    scale = 1.0 / math.sqrt(cfg.head_dim)
    T.tri_decode_attn(dst, cfg.n_q_heads, q.cuda(), scale, out)
    torch.cuda.synchronize()
    OK, OV = stored(g["out_k"].cpu()), stored(g["out_v"].cpu())
    opt = pc["out_page_table"].numpy()
    kept = nk.cpu().numpy()
    for s in range(cfg.n_seg):
        b, h = seg_seq(cfg, s), s % cfg.n_kv_heads
        hs = slice(h * cfg.group, (h + 1) * cfg.group)
        K = oracle.paged_rows(OK, opt[s], cfg.page_size, int(kept[s]))
        V = oracle.paged_rows(OV, opt[s], cfg.page_size, int(kept[s]))
        ref = oracle.decode_attn(stored(q[0, b, hs]), K, V, scale)
        got = out[0, b, hs].cpu().numpy()
        err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
        assert err.max() <= 1e-4, f"paged attention seg {s} (kept {kept[s]}): {err.max():.2e}"


def test_many_segments_mixed_lengths(gpu_lib):
    """At least 256 segments, so the fused pass copies inside the select kernel
    (fewer segments go through the separate gather), with lengths from 0 to the
    capacity: copy-through below the budget, pruning above it."""
    T = gpu_lib
    B, cap = 200, 600
    cfg = W.CONFIGS["tiny"].replace(head_dim=64, group=4, dtype=torch.bfloat16, theta=1e4, n_kv_heads=8, n_seq=36,
                                    n_keys=cap, t=cap + 2, budget=B, sigma=None, seed=31)
    assert cfg.n_seg >= 256
    log(f"case many segments: {cfg.n_seg} segments, N in [0, {cap}], B={B}")
    cpu = W.dense_cache(cfg, "cpu")
    gl = torch.Generator().manual_seed(31)
    cpu["lengths"] = torch.randint(0, cap + 1, (cfg.n_seg,), generator=gl, dtype=torch.int32)
    cpu["lengths"][:4] = torch.tensor([0, 1, B, B + 1], dtype=torch.int32)
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    _check_all(cfg, cal, cpu, r, B, cpu["lengths"].numpy(), "many segments")


@pytest.mark.parametrize("d,G,dtype,lengths", [
    (128, 4, torch.bfloat16, [65536, 65535, 8193]), (64, 8, torch.float32, [65536, 8192])])
def test_maximum_sizes(gpu_lib, d, G, dtype, lengths):
    """The largest segment (65536 keys) and budget (8192) the library takes,
    every step against the oracle.  bf16 at N = 8 B runs the candidate pass,
    one key fewer the full-score path."""
    T = gpu_lib
    B, cap = 8192, 65536
    cfg = W.CONFIGS["tiny"].replace(head_dim=d, group=G, dtype=dtype, theta=1e6, n_kv_heads=1, n_seq=len(lengths),
                                    n_keys=cap, t=cap + 1, budget=B, sigma=None, seed=29)
    log(f"case maximum sizes d={d} G={G} {dtype} lengths={lengths}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor(lengths, dtype=torch.int32)
    calib, cal = calib_for(T, cfg)
    r = _run_unfused(T, cfg, _to(cpu, "cuda"), calib, B)
    _check_all(cfg, cal, cpu, r, B, cpu["lengths"].numpy(), f"maximum d{d}")


@pytest.mark.parametrize("d,G,dtype,paged,n_seq", [
    (64, 1, torch.bfloat16, False, 2), (64, 8, torch.bfloat16, True, 2), (128, 8, torch.bfloat16, False, 2),
    (128, 2, torch.bfloat16, True, 2), (64, 2, torch.float32, False, 2), (128, 4, torch.float32, True, 2),
    (64, 8, torch.float32, False, 2), (128, 1, torch.bfloat16, False, 2),
    (64, 8, torch.bfloat16, False, 1), (128, 2, torch.bfloat16, True, 1)])
def test_decode_attention_shapes(gpu_lib, d, G, dtype, paged, n_seq):
    """Decode attention for every head size, group size and storage type, dense
    and paged (16-token pages, random page table), at lengths that end inside a
    tile, against the oracle; n_seq = 1 gives an odd segment count."""
    import math
    T = gpu_lib
    hkv, ps = 3, 16
    n_seg, hq = n_seq * hkv, hkv * G
    lengths = [1, 17, 33, 100, 511, 1000] if n_seq == 2 else [1000, 1, 511]
    cap = 1008
    gen = torch.Generator().manual_seed(41 + d + G)
    K = torch.randn((n_seg, cap, d), generator=gen).to(dtype)
    V = torch.randn((n_seg, cap, d), generator=gen).to(dtype)
    q = torch.randn((1, n_seq, hq, d), generator=gen).to(dtype)
    ln = torch.tensor(lengths, dtype=torch.int32)
    log(f"case attention d={d} G={G} {dtype} paged={paged}")
    if paged:
        mp = cap // ps
        perm = torch.randperm(n_seg * mp, generator=gen).to(torch.int32).view(n_seg, mp)
        pool_k = torch.empty((n_seg * mp, ps, d), dtype=dtype)
        pool_v = torch.empty_like(pool_k)
        pool_k[perm.reshape(-1).long()] = K.view(n_seg * mp, ps, d)
        pool_v[perm.reshape(-1).long()] = V.view(n_seg * mp, ps, d)
        pos = torch.zeros((n_seg * mp, ps), dtype=torch.int32)
        desc = T.cache_desc(pool_k.cuda(), pool_v.cuda(), pos.cuda(), ln.cuda(), n_layers=1, n_seq=n_seq,
                            n_kv_heads=hkv, page_table=perm.cuda(), page_size=ps, max_pages=mp)
        keep = (pool_k, pool_v, pos, perm)
    else:
        pos = torch.zeros((n_seg, cap), dtype=torch.int32)
        desc = T.cache_desc(K.cuda(), V.cuda(), pos.cuda(), ln.cuda(), n_layers=1, n_seq=n_seq, n_kv_heads=hkv)
        keep = None
    out = torch.full(q.shape, float("nan"), device="cuda")
    scale = 1.0 / math.sqrt(d)
    T.tri_decode_attn(desc, hq, q.cuda(), scale, out)
    torch.cuda.synchronize()
    for s in range(n_seg):
        N = lengths[s]
        b, h = s // hkv, s % hkv
        hs = slice(h * G, (h + 1) * G)
        ref = oracle.decode_attn(stored(q[0, b, hs]), stored(K[s, :N]), stored(V[s, :N]), scale)
        got = out[0, b, hs].cpu().numpy()
        err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
        assert err.max() <= 1e-4, f"attention d={d} G={G} {dtype} paged={paged} seg {s} N={N}: {err.max():.2e}"


@pytest.mark.parametrize("d,G,n_seq", [(64, 8, 320), (128, 4, 320), (64, 2, 320), (128, 4, 20), (64, 8, 20),
                                       (128, 2, 10)])
def test_decode_attention_batch_sizes(gpu_lib, d, G, n_seq):
    """Dense bf16 caches at ragged lengths, every segment against the oracle:
    more segments (2560) than the GPU holds workgroups at once, and batches
    of 160 and 80 segments (fewer than CUs: 8 and 16 waves per segment)."""
    T = gpu_lib
    hkv, cap = 8, 160
    n_seg, hq = n_seq * hkv, hkv * G
    gen = torch.Generator().manual_seed(47 + d + G)
    K = torch.randn((n_seg, cap, d), generator=gen).to(torch.bfloat16)
    V = torch.randn((n_seg, cap, d), generator=gen).to(torch.bfloat16)
    q = torch.randn((1, n_seq, hq, d), generator=gen).to(torch.bfloat16)
    ln = torch.randint(1, cap + 1, (n_seg,), generator=gen, dtype=torch.int32)
    ln[:6] = torch.tensor([1, cap, 2, cap - 1, 17, 64], dtype=torch.int32)
    log(f"case attention, {n_seg} segments, d={d} G={G}")
    pos = torch.zeros((n_seg, cap), dtype=torch.int32)
    desc = T.cache_desc(K.cuda(), V.cuda(), pos.cuda(), ln.cuda(), n_layers=1, n_seq=n_seq, n_kv_heads=hkv)
    out = torch.full(q.shape, float("nan"), device="cuda")
    scale = 1.0 / math.sqrt(d)
    T.tri_decode_attn(desc, hq, q.cuda(), scale, out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qs, Ks, Vs = stored(q), stored(K), stored(V)
    for s in range(n_seg):
        N = int(ln[s])
        b, h = s // hkv, s % hkv
        hs = slice(h * G, (h + 1) * G)
        ref = oracle.decode_attn(qs[0, b, hs], Ks[s, :N], Vs[s, :N], scale)
        got = out[0, b, hs]
        err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
        assert err.max() <= 1e-4, f"attention d={d} G={G} seg {s} N={N}: {err.max():.2e}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d,n_seq,hkv", [(64, 2, 3), (128, 7, 5), (64, 9, 4)])
def test_append_rows_and_full_segments(gpu_lib, dtype, d, n_seq, hkv):
    """tri_append writes row lengths[s] of each segment (K, V bit-exact, the
    sequence's position) and grows the length; a full segment is unchanged.
    Workgroups hold several segments (16, 8 or 4 per 256 threads): batches of
    up to 36 segments span several of them and end part-way through one."""
    T = gpu_lib
    cap = 40
    n_seg = n_seq * hkv
    gen = torch.Generator().manual_seed(43 + d + n_seg)
    K = torch.randn((n_seg, cap, d), generator=gen).to(dtype)
    V = torch.randn((n_seg, cap, d), generator=gen).to(dtype)
    pos = torch.randint(0, 1000, (n_seg, cap), generator=gen, dtype=torch.int32)
    ln = torch.randint(0, cap + 1, (n_seg,), generator=gen, dtype=torch.int32)
    ln[:6] = torch.tensor([0, 5, cap - 1, cap, 17, 39], dtype=torch.int32)
    ln[-1] = cap
    kn = torch.randn((n_seg, d), generator=gen).to(dtype)
    vn = torch.randn((n_seg, d), generator=gen).to(dtype)
    pn = 7001 + torch.arange(n_seq, dtype=torch.int32)
    g = {"k": K.cuda(), "v": V.cuda(), "pos": pos.cuda(), "lengths": ln.cuda()}
    desc = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=1, n_seq=n_seq, n_kv_heads=hkv)
    T.tri_append(desc, kn.cuda(), vn.cuda(), pn.cuda())
    torch.cuda.synchronize()
    Ka, Va, Pa, La = g["k"].cpu(), g["v"].cpu(), g["pos"].cpu(), g["lengths"].cpu()
    for s in range(n_seg):
        N = int(ln[s])
        if N >= cap:
            assert int(La[s]) == cap
            assert torch.equal(Ka[s], K[s]) and torch.equal(Va[s], V[s]) and torch.equal(Pa[s], pos[s]), f"seg {s}"
            continue
        assert int(La[s]) == N + 1, f"seg {s}"
        assert torch.equal(stored_t(Ka[s, N]), stored_t(kn[s])) and torch.equal(stored_t(Va[s, N]), stored_t(vn[s]))
        assert int(Pa[s, N]) == int(pn[s // hkv])
        other = torch.ones(cap, dtype=torch.bool)
        other[N] = False                                       # every other row untouched
        assert torch.equal(Ka[s][other], K[s][other]) and torch.equal(Va[s][other], V[s][other])
        assert torch.equal(Pa[s][other], pos[s][other])


def stored_t(x):
    """Bit pattern of a row (bf16 or fp32) as an integer tensor, for exact compares."""
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def test_prune_paths_give_the_same_cache(gpu_lib):
    """On a bf16 batch whose capacity allows the candidate pass, the three
    paths of tri_prune_window_ex (automatic: the full path for 9 segments;
    full; candidates) write byte-identical caches and kept counts, out of
    place and in place.  Neither the automatic nor the full path falls back."""
    T = gpu_lib
    B, cap = 600, 12000
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=3, n_seq=3,
                                    n_keys=cap, t=cap + 3, budget=B, sigma=None, seed=53)
    log("case prune paths")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 4095, 4096, 8 * B - 1, 8 * B, 8 * B + 1, 9001, B + 1, 0], dtype=torch.int32)
    calib, _ = calib_for(T, cfg)
    outs, fbs = {}, {}
    for path in (T.TRI_PATH_AUTO, T.TRI_PATH_FULL, T.TRI_PATH_CANDIDATES):
        g = _to(cpu, "cuda")
        desc = dense_desc(T, cfg, g)
        ws = T.workspace(calib, desc, B)
        out = empty_like_dense(g, B)
        T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws, path=path)
        fbs[path] = T.tri_prune_fallbacks(ws)
        T.tri_prune_window(calib, desc, g["t"], B, desc, g["lengths"], ws, path=path)      # in place
        torch.cuda.synchronize()
        outs[path] = (_to(out, "cpu"), _to(g, "cpu"))
    log(f"  fallbacks per path: {fbs}")
    assert fbs[T.TRI_PATH_AUTO] == 0 and fbs[T.TRI_PATH_FULL] == 0
    ref_out, ref_in = outs[T.TRI_PATH_FULL]
    for path, (out, inp) in outs.items():
        for key in ("k", "v", "pos", "lengths"):
            assert torch.equal(out[key], ref_out[key]), f"path {path}: out of place {key} differs"
            assert torch.equal(inp[key], ref_in[key]), f"path {path}: in place {key} differs"


@pytest.mark.parametrize("n_seq,n_keys", [(3, 12000), (1, 3000)])
def test_prune_with_exactly_the_reported_workspace(gpu_lib, n_seq, n_keys):
    """tri_prune_window runs in exactly tri_workspace_size bytes (candidate
    pass and full path; the candidate-capable cache and a small one), and
    refuses one byte less or a start off the 256-byte grid, before any launch
    (the destination stays untouched)."""
    T = gpu_lib
    B = 600
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=3, n_seq=n_seq,
                                    n_keys=n_keys, t=n_keys + 1, budget=B, sigma=None, seed=59)
    log(f"case exact workspace: {cfg.n_seg} segments x {n_keys} keys")
    g = _to(W.dense_cache(cfg, "cpu"), "cuda")
    calib, _ = calib_for(T, cfg)
    desc = dense_desc(T, cfg, g)
    need = T.tri_workspace_size(calib, desc, B)
    assert need > 0
    buf = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    off = (-buf.data_ptr()) % 256
    ws = buf[off:off + need]
    outs = []
    for path in (T.TRI_PATH_FULL, T.TRI_PATH_CANDIDATES):
        out = empty_like_dense(g, B)
        T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws, path=path)
        outs.append(out)
    torch.cuda.synchronize()
    for key in ("k", "v", "pos", "lengths"):
        assert torch.equal(outs[0][key], outs[1][key]), f"exact workspace: {key} differs between paths"
    untouched = empty_like_dense(g, B)
    for bad in (buf[off:off + need - 1], buf[off + 1:off + 1 + need]):
        with pytest.raises(T.TriError) as e:
            T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, untouched), untouched["lengths"], bad)
        assert e.value.code == T.TRI_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(untouched["lengths"].abs().sum()) == 0 and int((untouched["pos"] != -1).sum()) == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_budget_above_capacity_copies_through(gpu_lib, dtype):
    """A cache whose capacity (64) is below the budget (128): every segment is
    copied through unchanged out of place (n_kept = lengths), and an in-place
    pass leaves the cache as it was."""
    T = gpu_lib
    B, cap = 128, 64
    cfg = W.CONFIGS["tiny"].replace(head_dim=64, group=2, dtype=dtype, n_kv_heads=2, n_seq=2, n_keys=cap, t=cap,
                                    budget=B, seed=61)
    log(f"case budget above capacity {dtype}")
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([0, 1, 63, 64], dtype=torch.int32)
    g = _to(cpu, "cuda")
    calib, _ = calib_for(T, cfg)
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, B)
    out = empty_like_dense(g, B)
    T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws)
    T.tri_prune_window(calib, desc, g["t"], B, desc, g["lengths"], ws)       # in place: nothing to do
    torch.cuda.synchronize()
    assert torch.equal(out["lengths"].cpu(), cpu["lengths"])
    for s in range(cfg.n_seg):
        N = int(cpu["lengths"][s])
        for key in ("k", "v", "pos"):
            assert torch.equal(out[key][s, :N].cpu(), cpu[key][s, :N]), f"seg {s} {key} not copied through"
    for key in ("k", "v", "pos", "lengths"):
        assert torch.equal(g[key].cpu(), cpu[key]), f"in place: {key} changed"


def test_two_streams_two_workspaces(gpu_lib):
    """Two caches pruned and attended on two streams at once, each call with
    its own workspace, give the bytes the same calls give one after another on
    the default stream."""
    import math
    T = gpu_lib
    B, cap = 600, 12000
    cfgs = [W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=3, n_seq=3,
                                      n_keys=cap, t=cap + 1, budget=B, sigma=None, seed=seed) for seed in (71, 72)]
    log("case two streams")
    cpus = [W.dense_cache(c, "cpu") for c in cfgs]
    calib, _ = calib_for(T, cfgs[0])
    q = torch.randn((1, 3, 12, 128), generator=torch.Generator().manual_seed(73)).to(torch.bfloat16).cuda()
    scale = 1.0 / math.sqrt(128)

    def run(streams):
        res = []
        for cfg, cpu, st in zip(cfgs, cpus, streams):
            g = _to(cpu, "cuda")
            desc = dense_desc(T, cfg, g)
            ws = T.workspace(calib, desc, B)
            out = empty_like_dense(g, B)
            att = torch.empty((1, 3, 12, 128), device="cuda")
            torch.cuda.synchronize()
            T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), out["lengths"], ws, stream=st,
                               path=T.TRI_PATH_CANDIDATES)
            T.tri_decode_attn(dense_desc(T, cfg, out), 12, q, scale, att, stream=st)
            res.append((out, att, g, ws))
        torch.cuda.synchronize()
        return [({k: v.cpu() for k, v in out.items()}, att.cpu()) for out, att, _, _ in res]

    serial = run([None, None])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    concurrent = run([s1, s2])
    for (o_a, a_a), (o_b, a_b) in zip(serial, concurrent):
        for key in ("k", "v", "pos", "lengths"):
            assert torch.equal(o_a[key], o_b[key]), f"two streams: {key} differs"
        assert torch.equal(a_a, a_b), "two streams: attention differs"


def test_fallback_count_zero_without_candidate_mode(gpu_lib):
    """A pass that never enters candidate mode (fp32 here) reports zero
    fallbacks even on a workspace holding stale bytes."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"]
    g = _to(W.dense_cache(cfg, "cpu"), "cuda")
    calib, _ = calib_for(T, cfg)
    desc = dense_desc(T, cfg, g)
    out = empty_like_dense(g, cfg.budget)
    nk = torch.zeros_like(g["lengths"])
    ws = T.workspace(calib, desc, cfg.budget)
    ws.fill_(0x5A)
    T.tri_prune_window(calib, desc, g["t"], cfg.budget, dense_desc(T, cfg, out), nk, ws)
    assert T.tri_prune_fallbacks(ws) == 0


def test_cache_at_a_later_calibration_layer(gpu_lib):
    """A two-layer cache whose layer 0 is calibration layer 1 of three
    (layer0 = 1): every step of the pass, candidate mode included, must use
    layers 1 and 2 of the calibration."""
    T = gpu_lib
    B, cap = 600, 12000
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_layers=2, n_kv_heads=2,
                                    n_seq=2, n_keys=cap, t=cap + 3, budget=B, sigma=None, seed=47)
    log(f"case layer0 = 1: {cfg.n_seg} segments over calibration layers 1-2")
    cal = W.calibration(cfg.replace(n_layers=3))
    calib = T.tri_calib_load(cal["mag"], cal["phase"], cal["conc"], cal["offsets"], n_kv_heads=cfg.n_kv_heads,
                             rope_theta=cfg.theta)
    cpu = W.dense_cache(cfg, "cpu")
    cpu["lengths"] = torch.tensor([cap, 9001, 4095, 700, cap, 5000, B, 8000], dtype=torch.int32)
    g = _to(cpu, "cuda")
    desc = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=2, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, layer0=1)
    out = empty_like_dense(g, B)
    nk = torch.full_like(g["lengths"], -1)
    odesc = T.cache_desc(out["k"], out["v"], out["pos"], out["lengths"], n_layers=2, n_seq=cfg.n_seq,
                         n_kv_heads=cfg.n_kv_heads, layer0=1)
    ws = T.workspace(calib, desc, B)
    T.tri_prune_window(calib, desc, g["t"], B, odesc, nk, ws, path=T.TRI_PATH_CANDIDATES)
    agg = torch.full((cfg.n_seg, cap), float("nan"), device="cuda")
    T.tri_score(calib, desc, g["t"], agg, ws)
    torch.cuda.synchronize()
    A = agg.cpu()
    for s in range(cfg.n_seg):
        N = int(cpu["lengths"][s])
        tag = f"layer0=1 seg {s} N={N}"
        K, V, P = stored(cpu["k"][s, :N]), stored(cpu["v"][s, :N]), cpu["pos"][s, :N].numpy()
        ref = oracle_segment(cfg, cal, K, V, P, int(cpu["t"][seg_seq(cfg, s)]), s, B, layer0=1)
        check_agg(A[s, :N].numpy(), ref["A"], tag)
        nks = int(nk[s])
        assert nks == min(N, B), tag
        Pd = out["pos"][s, :nks].cpu().numpy()
        ix = kept_slots_from_positions(P, Pd)
        check_selection(ix, ref["A"], B, tag)
        check_compaction(K, V, P, stored(out["k"][s, :nks].cpu()), stored(out["v"][s, :nks].cpu()), Pd, ix, tag)
