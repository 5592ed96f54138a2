"""GPU parity at the five workload configurations' full sizes, in the launch
configuration the benchmark times (tri_prune_window over the whole cache).

Where the oracle cannot cover a whole configuration in seconds, sampled
segments are checked exhaustively (scores, aggregates, selection, compaction)
and properties that hold at any size are checked on every segment: kept count,
strictly ascending positions, and kept rows bit-equal to the source rows they
came from."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (check_in_place, calib_for, check_agg, check_compaction, check_scores, check_selection, dense_desc,
                     empty_like_dense, kept_slots_from_positions, log, oracle_segment, seg_seq, stored)

pytestmark = pytest.mark.gpu


def _dense_prune(T, cfg, g, calib, B, path=None):
    desc = dense_desc(T, cfg, g)
    ws = T.workspace(calib, desc, B)
    out = empty_like_dense(g, B)
    nk = out["lengths"]
    T.tri_prune_window(calib, desc, g["t"], B, dense_desc(T, cfg, out), nk, ws, path=path)
    return desc, ws, out


def _dense_properties(g, out, B, what):
    """Every segment: count, ascending positions (= source slots here), rows equal."""
    N = g["lengths"].long()
    nk = out["lengths"].long()
    assert torch.equal(nk, torch.clamp(N, max=B)), f"{what}: kept counts"
    pos = out["pos"].long()
    ar = torch.arange(B, device=pos.device)[None, :]
    valid = ar < nk[:, None]
    assert bool(torch.all(torch.where(valid[:, 1:], pos[:, 1:] > pos[:, :-1], True))), f"{what}: positions"
    assert bool(torch.all(torch.where(valid, (pos >= 0) & (pos < N[:, None]), True))), f"{what}: position range"
    src = torch.where(valid, pos, 0)
    for key in ("k", "v"):
        for a in range(0, g[key].shape[0], 256):      # bounded temporaries
            sl = slice(a, a + 256)
            gathered = torch.gather(g[key][sl], 1, src[sl, :, None].expand(-1, -1, g[key].shape[2]))
            same = (gathered.view(torch.int16) == out[key][sl].view(torch.int16)).all(dim=2)
            assert bool(torch.all(same | ~valid[sl])), f"{what}: {key} rows"


def test_qwen_single_layer_full(gpu_lib):
    T = gpu_lib
    cfg = W.CONFIGS["qwen1l"]
    B = cfg.budget
    log(f"case qwen1l full: 8 segments x {cfg.n_keys}")
    g = W.dense_cache(cfg, "cuda")
    calib, cal = calib_for(T, cfg)
    desc, ws, out = _dense_prune(T, cfg, g, calib, B)          # 8 segments: the full-score path
    # the candidate pass, asked for, keeps the same rows in the same order
    _, ws_c, out_c = _dense_prune(T, cfg, g, calib, B, path=T.TRI_PATH_CANDIDATES)
    fb = T.tri_prune_fallbacks(ws_c)
    log(f"  candidate pass: {fb} fallbacks")
    for key in ("k", "v", "pos", "lengths"):
        assert torch.equal(out_c[key], out[key]), f"qwen1l: candidate pass {key} differs from the full path"
    assert T.tri_prune_fallbacks(ws) == 0
    del out_c, ws_c
    n_seg, cap, G = cfg.n_seg, g["capacity"], cfg.group
    scores = torch.empty((n_seg, G, cap), device="cuda")
    agg = torch.empty((n_seg, cap), device="cuda")
    T.tri_score(calib, desc, g["t"], agg, ws, scores=scores)
    torch.cuda.synchronize()
    _dense_properties(g, out, B, "qwen1l")
    K, V, P = stored(g["k"].cpu()), stored(g["v"].cpu()), g["pos"].cpu().numpy()
    t = int(g["t"][0])
    refs = oracle.run_parallel(lambda s: oracle_segment(cfg, cal, K[s], V[s], P[s], t, s, B), range(n_seg))
    S, A = scores.cpu().numpy(), agg.cpu().numpy()
    Kd, Vd, Pd = stored(out["k"].cpu()), stored(out["v"].cpu()), out["pos"].cpu().numpy()
    for s, ref in enumerate(refs):
        tag = f"qwen1l seg {s}"
        check_scores(S[s], ref["S"], tag)
        check_agg(A[s], ref["A"], tag)
        ix = Pd[s]                      # positions are slots here
        nd = check_selection(ix, ref["A"], B, tag)
        check_compaction(K[s], V[s], P[s], Kd[s], Vd[s], Pd[s], ix, tag)
        log(f"  {tag}: {nd} slots differ inside the tie band")


def test_qwen_full_model_cache(gpu_lib):
    T = gpu_lib
    cfg = W.CONFIGS["qwen36l"]
    B = cfg.budget
    log(f"case qwen36l: {cfg.n_seg} segments x {cfg.n_keys}")
    g = W.dense_cache(cfg, "cuda")
    calib, cal = calib_for(T, cfg)
    desc, ws, out = _dense_prune(T, cfg, g, calib, B)
    torch.cuda.synchronize()
    _dense_properties(g, out, B, "qwen36l")
    n_seg, cap, G = cfg.n_seg, g["capacity"], cfg.group
    per_l = cfg.n_seq * cfg.n_kv_heads
    sample = [0, 18 * per_l + 7 * cfg.n_kv_heads + 3, n_seg - 1]
    agg = torch.empty((n_seg, cap), device="cuda")
    scores = torch.empty((n_seg, G, cap), device="cuda")
    T.tri_score(calib, desc, g["t"], agg, ws, scores=scores)
    torch.cuda.synchronize()
    t = int(g["t"][0])
    data = {s: (stored(g["k"][s].cpu()), stored(g["v"][s].cpu()), g["pos"][s].cpu().numpy()) for s in sample}
    refs = oracle.run_parallel(lambda s: oracle_segment(cfg, cal, *data[s], t, s, B), sample)
    for s, ref in zip(sample, refs):
        tag = f"qwen36l seg {s}"
        K, V, P = data[s]
        check_scores(scores[s].cpu().numpy(), ref["S"], tag)
        check_agg(agg[s].cpu().numpy(), ref["A"], tag)
        Pd = out["pos"][s].cpu().numpy()
        check_selection(Pd, ref["A"], B, tag)
        check_compaction(K, V, P, stored(out["k"][s].cpu()), stored(out["v"][s].cpu()), Pd, Pd, tag)
        log(f"  {tag} ok")


def test_ragged_paged_full(gpu_lib):
    T = gpu_lib
    cfg = W.CONFIGS["ragged"]
    B = cfg.budget
    log("case ragged paged: 64 sequences")
    pc = W.paged_cache(cfg, "cuda")
    calib, cal = calib_for(T, cfg)
    src = T.cache_desc(pc["k"], pc["v"], pc["pos"], pc["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=pc["page_table"], page_size=cfg.page_size,
                       max_pages=pc["max_pages"])
    nk = torch.zeros((cfg.n_seg,), dtype=torch.int32, device="cuda")
    dst = T.cache_desc(pc["out_k"], pc["out_v"], pc["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=pc["out_page_table"], page_size=cfg.page_size,
                       max_pages=pc["out_max_pages"])
    ws = T.workspace(calib, src, B)
    T.tri_prune_window(calib, src, pc["t"], B, dst, nk, ws)
    torch.cuda.synchronize()
    lengths = pc["lengths"].cpu().numpy()
    assert np.array_equal(nk.cpu().numpy(), np.minimum(lengths, B))
    order = np.argsort(lengths)
    sample = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 101})
    cap = cfg.page_size * pc["max_pages"]
    agg = torch.empty((cfg.n_seg, cap), device="cuda")
    scores = torch.empty((cfg.n_seg, cfg.group, cap), device="cuda")
    T.tri_score(calib, src, pc["t"], agg, ws, scores=scores)
    torch.cuda.synchronize()
    Kp, Vp, Pp = stored(pc["k"].cpu()), stored(pc["v"].cpu()), pc["pos"].cpu().numpy()
    OKp, OVp, OPp = stored(pc["out_k"].cpu()), stored(pc["out_v"].cpu()), pc["out_pos"].cpu().numpy()
    pt, opt = pc["page_table"].cpu().numpy(), pc["out_page_table"].cpu().numpy()

    # properties on every segment: ascending positions, rows equal to their source
    for s in range(cfg.n_seg):
        N, nks = int(lengths[s]), min(int(lengths[s]), B)
        Pd = oracle.paged_rows(OPp, opt[s], cfg.page_size, nks)
        assert np.all(np.diff(Pd) > 0) and Pd.min() >= 0 and Pd.max() < N, f"seg {s} positions"
        if s % 16 == 0:
            K = oracle.paged_rows(Kp, pt[s], cfg.page_size, N)
            Kd = oracle.paged_rows(OKp, opt[s], cfg.page_size, nks)
            assert np.array_equal(Kd, K[Pd]), f"seg {s} rows"

    def one(s):
        N = int(lengths[s])
        K = oracle.paged_rows(Kp, pt[s], cfg.page_size, N)
        V = oracle.paged_rows(Vp, pt[s], cfg.page_size, N)
        P = oracle.paged_rows(Pp, pt[s], cfg.page_size, N)
        return K, V, P, oracle_segment(cfg, cal, K, V, P, int(pc["t"][seg_seq(cfg, s)]), s, B)

    for s, (K, V, P, ref) in zip(sample, oracle.run_parallel(one, sample)):
        N, nks = int(lengths[s]), min(int(lengths[s]), B)
        tag = f"ragged seg {s} N={N}"
        check_scores(scores[s, :, :N].cpu().numpy(), ref["S"], tag)
        check_agg(agg[s, :N].cpu().numpy(), ref["A"], tag)
        Pd = oracle.paged_rows(OPp, opt[s], cfg.page_size, nks)
        check_selection(Pd, ref["A"], B, tag)
        check_compaction(K, V, P, oracle.paged_rows(OKp, opt[s], cfg.page_size, nks),
                         oracle.paged_rows(OVp, opt[s], cfg.page_size, nks), Pd, Pd, tag)
        log(f"  {tag} ok")

    # decode attention reading the pruned pages in place
    gq = torch.Generator().manual_seed(5)
    q = torch.randn((1, cfg.n_seq, cfg.n_q_heads, cfg.head_dim), generator=gq).to(cfg.dtype)
    out = torch.full(q.shape, float("nan"), device="cuda")
    scale = 1.0 / math.sqrt(cfg.head_dim)
    T.tri_decode_attn(dst, cfg.n_q_heads, q.cuda(), scale, out)
    torch.cuda.synchronize()
    for s in sample:
        nks = min(int(lengths[s]), B)
        b, h = seg_seq(cfg, s), s % cfg.n_kv_heads
        hs = slice(h * cfg.group, (h + 1) * cfg.group)
        ref = oracle.decode_attn(stored(q[0, b, hs]), oracle.paged_rows(OKp, opt[s], cfg.page_size, nks),
                                 oracle.paged_rows(OVp, opt[s], cfg.page_size, nks), scale)
        got = out[0, b, hs].cpu().numpy()
        err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
        assert err.max() <= 1e-4, f"ragged paged attention seg {s}: {err.max():.2e}"
    log("  paged decode attention over the pruned pages ok")


@pytest.mark.parametrize("in_place", [False, True])
def test_gptoss_decode_loop_full(gpu_lib, in_place):
    T = gpu_lib
    cfg = W.CONFIGS["gptoss"]
    B = cfg.budget
    log(f"case gptoss decode loop: {cfg.windows} windows x {cfg.window} steps, {cfg.n_seg} segments, "
        f"in place {in_place}")
    st = W.decode_start(cfg, "cuda")
    km = st.pop("key_model")
    calib, cal = calib_for(T, cfg)
    cap = st["capacity"]
    caches = [st, {**empty_like_dense(st, cap), "t": st["t"]}]
    cur = 0
    t = cfg.start_pos_range
    scale = 1.0 / math.sqrt(cfg.head_dim)
    sample = [0, 2333, cfg.n_seg - 1]
    for w in range(cfg.windows):
        c = caches[cur]
        desc = dense_desc(T, cfg, c)
        for j in range(cfg.window):
            k_new, v_new, q = W.decode_token(cfg, km, w * cfg.window + j, t, "cuda")
            pos_new = torch.full((cfg.n_seq,), t, dtype=torch.int32, device="cuda")
            T.tri_append(desc, k_new, v_new, pos_new)
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            T.tri_decode_attn(desc, cfg.n_q_heads, q, scale, out)
            if w in (0, cfg.windows - 1) and j in (0, cfg.window - 1):
                torch.cuda.synchronize()
                for s in sample:
                    N = int(c["lengths"][s])
                    l, b, h = s // (cfg.n_seq * cfg.n_kv_heads), seg_seq(cfg, s), s % cfg.n_kv_heads
                    hs = slice(h * cfg.group, (h + 1) * cfg.group)
                    ref = oracle.decode_attn(stored(q[l, b, hs].cpu()), stored(c["k"][s, :N].cpu()),
                                             stored(c["v"][s, :N].cpu()), scale)
                    got = out[l, b, hs].cpu().numpy()
                    err = np.abs(got - ref) / np.maximum(np.abs(ref), np.abs(ref).max(axis=1, keepdims=True))
                    assert err.max() <= 1e-4, f"attention window {w} step {j} seg {s}: {err.max():.2e}"
            t += 1
        c["t"] = torch.full((cfg.n_seq,), t, dtype=torch.int32, device="cuda")
        ws = T.workspace(calib, desc, B)
        if in_place:
            checked = w in (0, cfg.windows - 1)
            if checked:
                before = {k: c[k][sample].cpu() for k in ("k", "v", "pos", "lengths")}
            T.tri_prune_window(calib, desc, c["t"], B, desc, c["lengths"], ws)
            torch.cuda.synchronize()
            assert bool(torch.all(c["lengths"] == B)), f"window {w}: kept counts"
            if checked:
                Ka, Va, Pa = (stored(c["k"][sample].cpu()), stored(c["v"][sample].cpu()),
                              c["pos"][sample].cpu().numpy())
                Kb, Vb, Pb = stored(before["k"]), stored(before["v"]), before["pos"].numpy()
                for i, s in enumerate(sample):
                    check_in_place(cfg, cal, Kb[i], Vb[i], Pb[i], Ka[i], Va[i], Pa[i], int(before["lengths"][i]),
                                   B, t, s, B, f"gptoss window {w} seg {s} in place")
                log(f"  window {w} checked")
            continue
        nxt = caches[1 - cur]
        T.tri_prune_window(calib, desc, c["t"], B, dense_desc(T, cfg, nxt), nxt["lengths"], ws)
        torch.cuda.synchronize()
        assert bool(torch.all(nxt["lengths"] == B)), f"window {w}: kept counts"
        if w in (0, cfg.windows - 1):
            for s in sample:
                N = int(c["lengths"][s])
                K, V, P = stored(c["k"][s, :N].cpu()), stored(c["v"][s, :N].cpu()), c["pos"][s, :N].cpu().numpy()
                ref = oracle_segment(cfg, cal, K, V, P, t, s, B)
                Pd = nxt["pos"][s, :B].cpu().numpy()
                ix = kept_slots_from_positions(P, Pd)
                tag = f"gptoss window {w} seg {s}"
                check_selection(ix, ref["A"], B, tag)
                check_compaction(K, V, P, stored(nxt["k"][s, :B].cpu()), stored(nxt["v"][s, :B].cpu()), Pd, ix, tag)
            log(f"  window {w} checked")
        nxt["t"] = c["t"]
        cur = 1 - cur
