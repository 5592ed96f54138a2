"""GPU parity at the five workload configurations' full sizes, in the launch
configuration the benchmark times (tri_prune_window over the whole cache).

The oracle checks every segment where it finishes in a minute: the single
layer, all 512 segments of the ragged batch, every segment of one layer of
the GPT-OSS-shaped loop at its first and last window.  On the 36-layer cache
it checks layers 0, 18 and 35 (384 segments; the whole cache is about 1.3e4
core-seconds of oracle), and on every segment the candidate pass must write
byte for byte what the full-score path writes, and the properties that hold
at any size are checked: kept count, strictly ascending positions, kept rows
bit-equal to the source rows they came from."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (check_in_place, calib_for, check_agg, check_mu_sigma, check_compaction, check_scores, check_selection, dense_desc,
                     empty_like_dense, kept_slots_from_positions, log, oracle_segment, oracle_select, seg_seq,
                     stored)

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


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_candidate_pass_equals_full_path_on_other_draws(gpu_lib, seed):
    """32 segments of the main workload's shape (32,768 bf16 keys, d = 128,
    GQA 4, B = 2048) drawn with other seeds: the candidate pass (threshold at
    sample rank 2.5B/N, certified or redone) writes the same cache byte for
    byte as the full-score path; the fallback count is logged."""
    T = gpu_lib
    cfg = W.CONFIGS["qwen1l"].replace(n_seq=4, n_keys=32768, seed=seed)
    B = cfg.budget
    log(f"case candidate pass vs full path, seed {seed}: {cfg.n_seg} segments x {cfg.n_keys}")
    g = W.dense_cache(cfg, "cuda")
    calib, _ = calib_for(T, cfg)
    _, _, full = _dense_prune(T, cfg, g, calib, B, path=T.TRI_PATH_FULL)
    _, ws, cand = _dense_prune(T, cfg, g, calib, B, path=T.TRI_PATH_CANDIDATES)
    torch.cuda.synchronize()
    log(f"  candidate pass: {T.tri_prune_fallbacks(ws)} fallbacks")
    for key in ("k", "v", "pos", "lengths"):
        a, b = full[key], cand[key]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), f"seed {seed}: {key} differs between the paths"
    _dense_properties(g, full, B, f"seed {seed}")


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
    """The bench workload: 4608 segments of 32768 keys.  The automatic path
    (the candidate pass) against the full-score path on every segment, byte
    for byte, with no segment falling back; every step against the oracle on
    layers 0, 18 and 35 (all 16 sequences x 8 KV heads of each)."""
    T = gpu_lib
    cfg = W.CONFIGS["qwen36l"]
    B = cfg.budget
    log(f"case qwen36l: {cfg.n_seg} segments x {cfg.n_keys}")
    g = W.dense_cache(cfg, "cuda")
    calib, cal = calib_for(T, cfg)
    desc, ws, out = _dense_prune(T, cfg, g, calib, B)
    fb = T.tri_prune_fallbacks(ws)
    log(f"  automatic path: {fb} fallbacks")
    assert fb == 0, f"{fb} segments fell back to the full path"
    _dense_properties(g, out, B, "qwen36l")
    _, ws_f, out_f = _dense_prune(T, cfg, g, calib, B, path=T.TRI_PATH_FULL)
    torch.cuda.synchronize()
    for key in ("k", "v", "pos", "lengths"):
        assert torch.equal(out_f[key], out[key]), f"qwen36l: full-score path {key} differs from the candidate pass"
    log("  candidate pass == full-score path on every segment")
    del out_f, ws_f
    n_seg, cap, G = cfg.n_seg, g["capacity"], cfg.group
    agg = torch.empty((n_seg, cap), device="cuda")
    scores = torch.empty((n_seg, G, cap), device="cuda")
    ms = torch.empty((n_seg, G, 2), device="cuda")
    T.tri_score(calib, desc, g["t"], agg, ws, scores=scores, mu_sigma=ms)
    torch.cuda.synchronize()
    t = int(g["t"][0])
    per_l = cfg.n_seq * cfg.n_kv_heads
    for layer in (0, 18, 35):
        segs = list(range(layer * per_l, (layer + 1) * per_l))
        K = stored(g["k"][segs].cpu())
        P = g["pos"][segs].cpu().numpy()
        refs = oracle.run_parallel(lambda i: oracle_select(cfg, cal, K[i], P[i], t, segs[i], B), range(len(segs)))
        S, A, MS = scores[segs].cpu().numpy(), agg[segs].cpu().numpy(), ms[segs].cpu().numpy()
        Pd = out["pos"][segs].cpu().numpy()
        n_diff = 0
        for i, (s, ref) in enumerate(zip(segs, refs)):
            tag = f"qwen36l seg {s}"
            check_scores(S[i], ref["S"], tag)
            check_mu_sigma(MS[i], ref["mu"], ref["sigma"], tag)
            check_agg(A[i], ref["A"], tag)
            n_diff += check_selection(Pd[i], ref["A"], B, tag, pos=P[i])     # positions are slots here
        log(f"  layer {layer}: {len(segs)} segments match the oracle ({n_diff} slots differ inside the tie band)")


@pytest.mark.parametrize("part", range(4))
def test_ragged_paged_full(gpu_lib, part):
    """The ragged paged batch (64 sequences x 8 KV heads, 4096..65536 keys,
    fresh output pages).  Every step of every segment against the oracle, a
    quarter of the 512 segments per part; part 0 also runs decode attention
    over the pruned pages."""
    T = gpu_lib
    cfg = W.CONFIGS["ragged"]
    B = cfg.budget
    log(f"case ragged paged: 64 sequences, part {part}")
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
    log(f"  fallbacks: {T.tri_prune_fallbacks(ws)}")
    lengths = pc["lengths"].cpu().numpy()
    assert np.array_equal(nk.cpu().numpy(), np.minimum(lengths, B))
    cap = cfg.page_size * pc["max_pages"]
    agg = torch.empty((cfg.n_seg, cap), device="cuda")
    scores = torch.empty((cfg.n_seg, cfg.group, cap), device="cuda")
    T.tri_score(calib, src, pc["t"], agg, ws, scores=scores)
    torch.cuda.synchronize()
    Kp, Vp, Pp = stored(pc["k"].cpu()), stored(pc["v"].cpu()), pc["pos"].cpu().numpy()
    OKp, OVp, OPp = stored(pc["out_k"].cpu()), stored(pc["out_v"].cpu()), pc["out_pos"].cpu().numpy()
    pt, opt = pc["page_table"].cpu().numpy(), pc["out_page_table"].cpu().numpy()
    segs = list(range(part, cfg.n_seg, 4))

    def one(s):
        N = int(lengths[s])
        K = oracle.paged_rows(Kp, pt[s], cfg.page_size, N)
        P = oracle.paged_rows(Pp, pt[s], cfg.page_size, N)
        return oracle_select(cfg, cal, K, P, int(pc["t"][seg_seq(cfg, s)]), s, B)

    n_diff = 0
    for s, ref in zip(segs, oracle.run_parallel(one, segs)):
        N, nks = int(lengths[s]), min(int(lengths[s]), B)
        tag = f"ragged seg {s} N={N}"
        check_scores(scores[s, :, :N].cpu().numpy(), ref["S"], tag)
        check_agg(agg[s, :N].cpu().numpy(), ref["A"], tag)
        K = oracle.paged_rows(Kp, pt[s], cfg.page_size, N)
        V = oracle.paged_rows(Vp, pt[s], cfg.page_size, N)
        P = oracle.paged_rows(Pp, pt[s], cfg.page_size, N)
        Pd = oracle.paged_rows(OPp, opt[s], cfg.page_size, nks)
        ix = kept_slots_from_positions(P, Pd)
        n_diff += check_selection(ix, ref["A"], B, tag, pos=P)
        check_compaction(K, V, P, oracle.paged_rows(OKp, opt[s], cfg.page_size, nks),
                         oracle.paged_rows(OVp, opt[s], cfg.page_size, nks), Pd, ix, tag)
    log(f"  {len(segs)} segments match the oracle ({n_diff} slots differ inside the tie band)")
    if part:
        return

    # the candidate pass (which the automatic path leaves out on this batch:
    # its lists of up to 32K entries need one select workgroup per CU) writes
    # the same pages on every segment
    cand = {k: torch.zeros_like(pc["out_" + k]) for k in ("k", "v", "pos")}
    nkc = torch.zeros_like(nk)
    dstc = T.cache_desc(cand["k"], cand["v"], cand["pos"], nkc, n_layers=1, n_seq=cfg.n_seq,
                        n_kv_heads=cfg.n_kv_heads, page_table=pc["out_page_table"], page_size=cfg.page_size,
                        max_pages=pc["out_max_pages"])
    T.tri_prune_window(calib, src, pc["t"], B, dstc, nkc, ws, path=T.TRI_PATH_CANDIDATES)
    torch.cuda.synchronize()
    log(f"  candidate pass: {T.tri_prune_fallbacks(ws)} fallbacks")
    assert torch.equal(nkc, nk)
    CK, CV, CP = stored(cand["k"].cpu()), stored(cand["v"].cpu()), cand["pos"].cpu().numpy()
    for s in range(cfg.n_seg):
        nks = min(int(lengths[s]), B)
        for a, b, key in ((CK, OKp, "k"), (CV, OVp, "v"), (CP, OPp, "pos")):
            assert np.array_equal(oracle.paged_rows(a, opt[s], cfg.page_size, nks),
                                  oracle.paged_rows(b, opt[s], cfg.page_size, nks)), f"seg {s}: candidate pass {key}"

    # decode attention reading the pruned pages in place
    sample = [0, 101, 257, cfg.n_seg - 1]
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


def _layer_against_oracle(cfg, cal, before, res, layer_segs, t, B, w, slot_order=True):
    """The pruned segments layer_segs of cache `res` against the oracle's prune
    of their rows before the prune (`before`: lengths, K, V, positions on the
    host) at position t."""
    N0, Kb, Vb, Pb = before
    refs = oracle.run_parallel(lambda i: oracle_select(cfg, cal, Kb[i, :N0[i]], Pb[i, :N0[i]], t,
                                                       layer_segs[i], B), range(len(layer_segs)))
    Kd, Vd = stored(res["k"][layer_segs, :B].cpu()), stored(res["v"][layer_segs, :B].cpu())
    Pd = res["pos"][layer_segs, :B].cpu().numpy()
    n_diff = 0
    for i, (s, ref) in enumerate(zip(layer_segs, refs)):
        tag = f"gptoss window {w} seg {s}"
        N = int(N0[i])
        ix = kept_slots_from_positions(Pb[i, :N], Pd[i])
        n_diff += check_selection(np.sort(ix), ref["A"], B, tag, pos=Pb[i, :N])
        check_compaction(Kb[i, :N], Vb[i, :N], Pb[i, :N], Kd[i], Vd[i], Pd[i], ix, tag)
        if slot_order:
            assert np.all(np.diff(ix) > 0), f"{tag}: not in slot order"
    log(f"  window {w}: {len(layer_segs)} segments of layer 11 match the oracle "
        f"({n_diff} slots differ inside the tie band)")


@pytest.mark.parametrize("in_place", [False, True, "fill"])
def test_gptoss_decode_loop_full(gpu_lib, in_place):
    """16 windows of 128 steps (append + decode attention each step), a prune
    after each window: into the other buffer, or in place (slot order, or
    filling freed slots).  In place, each window's state is first pruned out of
    place too, and the in-place cache must hold the same bytes on every
    segment (slot order) or the same kept set (fill).  At the first and last
    window, every segment of layer 11 against the oracle, and attention on
    sampled segments."""
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
    per_l = cfg.n_seq * cfg.n_kv_heads
    layer_segs = list(range(11 * per_l, 12 * per_l))
    fill = in_place == "fill"
    oop = empty_like_dense(st, B) if in_place else None
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
        checked = w in (0, cfg.windows - 1)
        if checked:
            N0 = c["lengths"][layer_segs].cpu().numpy()
            Kb = stored(c["k"][layer_segs].cpu())
            Vb = stored(c["v"][layer_segs].cpu())
            Pb = c["pos"][layer_segs].cpu().numpy()
        if in_place:
            T.tri_prune_window(calib, desc, c["t"], B, dense_desc(T, cfg, oop), oop["lengths"], ws)
            T.tri_prune_window(calib, desc, c["t"], B, desc, c["lengths"], ws,
                               path=T.TRI_INPLACE_FILL_FREED if fill else T.TRI_PATH_AUTO)
            torch.cuda.synchronize()
            assert bool(torch.all(c["lengths"] == B)), f"window {w}: kept counts"
            if not fill:
                for key in ("k", "v", "pos"):
                    assert torch.equal(c[key][:, :B], oop[key]), f"window {w}: in place {key} differs from out of place"
            else:                                       # the same kept set, arranged otherwise
                assert torch.equal(torch.sort(c["pos"][:, :B], dim=1).values, torch.sort(oop["pos"], dim=1).values), \
                    f"window {w}: fill mode kept another set"
            res = c
        else:
            nxt = caches[1 - cur]
            T.tri_prune_window(calib, desc, c["t"], B, dense_desc(T, cfg, nxt), nxt["lengths"], ws)
            torch.cuda.synchronize()
            assert bool(torch.all(nxt["lengths"] == B)), f"window {w}: kept counts"
            res = nxt
        if checked:
            _layer_against_oracle(cfg, cal, (N0, Kb, Vb, Pb), res, layer_segs, t, B, w, slot_order=not fill)
        if not in_place:
            nxt["t"] = c["t"]
            cur = 1 - cur


def test_gptoss_decode_loop_overlapped(gpu_lib):
    """The GPT-OSS-shaped loop with each window's prune overlapped: out of
    place on a second stream in four layer groups, beside the window's last
    attention and the next window's first step (appended and attended group by
    group).  Run in lockstep with the same loop pruned serially on the decode
    stream: the attention outputs of every window's first, second and last
    step and both caches after every window's second step are byte for byte
    the serial loop's; at the first and last window every segment of layer 11
    of the overlapped prune's result against the oracle."""
    from long_reasoning_decode_amd.decode_loop import LayerGroups, OverlappedPrune, first_step
    T = gpu_lib
    cfg = W.CONFIGS["gptoss"]
    B, win, Hq = cfg.budget, cfg.window, cfg.n_q_heads
    n_groups = 4
    log(f"case gptoss decode loop overlapped: {cfg.windows} windows x {win} steps, {n_groups} layer groups")
    D = torch.cuda.Stream()
    with torch.cuda.stream(D):
        st = W.decode_start(cfg, "cuda")
        km = st.pop("key_model")
        calib, cal = calib_for(T, cfg)
        cap = st["capacity"]
        keys = ("k", "v", "pos", "lengths")
        ser = [st, empty_like_dense(st, cap)]
        ovl = [{k: st[k].clone() for k in keys}, empty_like_dense(st, cap)]
        dser = [dense_desc(T, cfg, c) for c in ser]
        dovl = [dense_desc(T, cfg, c) for c in ovl]
        groups = [LayerGroups(c, n_layers=cfg.n_layers, n_seq=cfg.n_seq, n_kv_heads=cfg.n_kv_heads,
                              n_groups=n_groups) for c in ovl]
        ws_s, ws_o = T.workspace(calib, dser[0], B), T.workspace(calib, dovl[0], B)
        P = torch.cuda.Stream()
        pruners = [OverlappedPrune(calib, groups[i], groups[1 - i], B, ws_o, D, P) for i in (0, 1)]
        tv_s = torch.empty((cfg.n_seq,), dtype=torch.int32, device="cuda")
        tv_o = torch.empty_like(tv_s)
        q_shape = (cfg.n_layers, cfg.n_seq, Hq, cfg.head_dim)
        out_s = torch.empty(q_shape, dtype=torch.float32, device="cuda")
        out_o = torch.empty_like(out_s)
        per_l = cfg.n_seq * cfg.n_kv_heads
        layer_segs = list(range(11 * per_l, 12 * per_l))
        scale = 1.0 / math.sqrt(cfg.head_dim)
        pending, cur, t = None, 0, cfg.start_pos_range
        for w in range(cfg.windows):
            for j in range(win):
                k_new, v_new, q = W.decode_token(cfg, km, w * win + j, t, "cuda")
                pos_new = torch.full((cfg.n_seq,), t, dtype=torch.int32, device="cuda")
                T.tri_append(dser[cur], k_new, v_new, pos_new, stream=D)
                T.tri_decode_attn(dser[cur], Hq, q, scale, out_s, stream=D)
                if j == 0 and pending is not None:
                    first_step(pending, groups[cur], Hq, k_new, v_new, pos_new, q, scale, out_o, D)
                    pending = None
                else:
                    T.tri_append(dovl[cur], k_new, v_new, pos_new, stream=D)
                    if j == win - 1:
                        tv_o.fill_(t + 1)
                        pruners[cur].launch(tv_o)
                        pending = pruners[cur]
                    T.tri_decode_attn(dovl[cur], Hq, q, scale, out_o, stream=D)
                if j in (0, 1, win - 1):
                    assert torch.equal(out_o, out_s), f"window {w} step {j}: attention differs from the serial loop"
                if j == 1:
                    for k in keys:
                        assert torch.equal(ovl[cur][k], ser[cur][k]), f"window {w} step 1: cache {k} differs"
                t += 1
            tv_s.fill_(t)
            T.tri_prune_window(calib, dser[cur], tv_s, B, dser[1 - cur], ser[1 - cur]["lengths"], ws_s, stream=D)
            if w in (0, cfg.windows - 1):
                for g in range(n_groups):
                    pending.wait(g)
                D.synchronize()
                for k in keys:
                    assert torch.equal(ovl[1 - cur][k], ser[1 - cur][k]), f"window {w}: pruned cache {k} differs"
                src = ser[cur]
                before = (src["lengths"][layer_segs].cpu().numpy(), stored(src["k"][layer_segs].cpu()),
                          stored(src["v"][layer_segs].cpu()), src["pos"][layer_segs].cpu().numpy())
                _layer_against_oracle(cfg, cal, before, ovl[1 - cur], layer_segs, t, B, w)
            cur = 1 - cur
        D.synchronize()
    calib.free()
