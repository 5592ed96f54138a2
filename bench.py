"""Benchmark of the TriAttention pruning pass on one MI355X.

A step is one tri_prune_window call over the whole synthetic cache (score every
key, z-score/max per GQA group, select the top-B per KV head, compact K/V and
positions into a second cache).  Default workload: a Qwen3-8B-shaped full-model
cache, 36 layers x 16 sequences x 8 KV heads x 32768 keys, head_dim 128, bf16,
GQA 4, B = 2048, 16 geometric offsets.  Inputs are generated on the GPU before
timing and stay resident in HBM.

Prints one JSON line.  Per-kernel durations come from HIP events recorded by
the library on the launch stream over the timed steps (tri_timing_*).
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "keys scored+pruned/sec (G keys/s) and % of HBM roofline, 32K cache, B=2048"
HBM_PEAK_GBS = 8000.0


# The source file each timed kernel is defined in; every kernel also depends
# on the shared headers and on the C ABI's launch choices (api.hip).
KERNEL_SOURCE = {"score": "score.hip", "select_gather": "select.hip", "gather": "select.hip", "decode_attn": "decode.hip",
                 "calibrate": "calib.hip"}
SHARED_SOURCES = ["api.hip", "common.h", "launch.h", "stats.h"]


def kernel_source_sha(kernel=None):
    """Hash of the sources a kernel's counters depend on (None: every kernel source)."""
    csrc = os.path.join(ROOT, "long_reasoning_decode_amd", "csrc")
    if kernel is None:
        files = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        files = [os.path.join(csrc, f) for f in sorted(SHARED_SOURCES + [KERNEL_SOURCE[kernel]])]
    h = hashlib.sha256()
    for p in files:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if kernel not in KERNEL_SOURCE or vals.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(n_keys_total, n_seg, n_kept_total, d, es):
    """Bytes the method must move: every key read once for scoring, kept K and
    V rows read and written, kept positions read and written."""
    score = n_keys_total * d * es
    gather = n_kept_total * (4 * d * es + 8)
    return score, gather


# The pages' own figures for the method, end to end (decode throughput and KV
# memory at full-attention accuracy, Qwen3-8B on AIME25; hardware not named):
# context for the result line, not this kernel's metric.
PAGES_CONTEXT = {
    "decode_throughput_vs_full_attention": 2.5,
    "kv_memory_reduction": 10.7,
    "source": "zingnex.cn TriAttention page, section 实验验证; yeyulingfeng.com TriAttention page, "
              "section (二)主实验结果",
    "note": "end-to-end serving figures on hardware the pages do not name; they measure the whole decode, "
            "not the pruning pass timed here",
}


def cpu_baseline(W, cfg, g, cal, B, n_sample):
    import numpy as np

    import oracle
    threads = oracle.host_threads()
    n_sample = max(n_sample, threads)                   # every thread gets a segment
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    per_l = cfg.n_seq * cfg.n_kv_heads
    segs = [int(s) for s in np.linspace(0, cfg.n_seg - 1, n_sample).round()]
    data = {s: (W.to_stored_numpy(g["k"][s]), W.to_stored_numpy(g["v"][s]), g["pos"][s].cpu().numpy())
            for s in segs}
    t = int(g["t"][0])
    G = cfg.group

    def one(s):
        l, h = s // per_l, s % cfg.n_kv_heads
        sl = slice(h * G, (h + 1) * G)
        K, V, P = data[s]
        return oracle.prune_segment(K, V, P, t, cfg.theta, cal["mag"][l, sl].numpy(), cal["phase"][l, sl].numpy(),
                                    cal["conc"][l, sl].numpy(), cfg.offsets, B)

    t0 = time.perf_counter()
    oracle.run_parallel(one, segs, threads=threads)
    dt = time.perf_counter() - t0
    keys = len(segs) * cfg.n_keys
    return {"value": keys / dt / 1e9, "unit": "G keys/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{len(segs)} whole segments ({cfg.n_keys} keys each, full prune chain) spread over "
                      f"layers/sequences/heads; {dt:.1f} s wall on {threads} threads (the process's CPU "
                      f"share: OMP_NUM_THREADS, else its affinity set)"}


def kernel_breakdown(T, step, steps):
    """{kernel: (launches, total ms)} over `steps` steps with every kernel
    bracketed by events (untimed: each event record costs GPU time)."""
    import torch
    T.tri_timing_reset()
    T.tri_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    T.tri_timing_enable(False)
    return T.tri_timing_read()


def timed_steps(T, step, steps, stream, kernels, finish=None):
    """The timed region: `steps` steps between two events, with only the named
    kernels' launches bracketed by library events; `finish` (optional) orders
    `stream` after work the last step left on other streams.  Returns (ms per
    step, {kernel: (launches, total ms)})."""
    import torch
    T.tri_timing_reset()
    T.tri_timing_enable(True, only=kernels)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        step()
    if finish is not None:
        finish()
    ev1.record(stream)
    torch.cuda.synchronize()
    T.tri_timing_enable(False)
    return ev0.elapsed_time(ev1) / steps, T.tri_timing_read()


def flushed_steps(step, steps, stream, flush_mib):
    """Each step timed alone (events on its stream) right after writing a
    flush_mib buffer, so the step starts with nothing of its inputs in the
    last-level cache; the flush itself is outside every timed interval.
    Returns the mean ms per step."""
    import torch
    buf = torch.empty(flush_mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        buf.fill_(float(i))
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    del buf
    torch.cuda.empty_cache()
    return ms


def copy_bandwidth(mib=4096, reps=5):
    """Read + write bytes per second of a plain device-to-device copy."""
    import torch
    n = mib * 1024 * 1024
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def copy_probe(mib):
    """Plain device-to-device copies of a known size, for scaling counters."""
    import torch
    torch.cuda.set_device(0)
    n = mib * 1024 * 1024
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "copy_GBs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def bench_decode_loop(args, T, W):
    """GPT-OSS-shaped decode loop: a step is one 128-token window, i.e. 128 x
    (append one token to every segment, single-query attention of every query
    head over its cache) followed by the window's prune back to B.  Tokens are
    generated before timing and reused window after window.  The prune runs in
    place unless --out-of-place is given, in
    which case it compacts into a second cache and the two alternate.  In place
    the cache stays in slot order (every kept row after the first dropped slot
    moves), or with --fill-freed only the kept rows above B move, into the freed
    slots.  Then the same windows are timed with the prune overlapped
    (out of place, on a second stream in --overlap-groups layer groups, beside
    the window's last attention and the next window's first step), reported
    under "overlapped"."""
    import math

    import torch

    from long_reasoning_decode_amd.decode_loop import LayerGroups, OverlappedPrune, first_step
    cfg = W.CONFIGS["gptoss"]
    B, win = cfg.budget, cfg.window
    st = W.decode_start(cfg, "cuda")
    km = st.pop("key_model")
    cal = W.calibration(cfg)
    calib = T.tri_calib_load(cal["mag"], cal["phase"], cal["conc"], cal["offsets"], n_kv_heads=cfg.n_kv_heads,
                             rope_theta=cfg.theta)
    cap = st["capacity"]
    caches = [st, {"k": torch.empty_like(st["k"]), "v": torch.empty_like(st["v"]),
                   "pos": torch.empty_like(st["pos"]), "lengths": torch.zeros_like(st["lengths"])}]
    descs = [T.cache_desc(c["k"], c["v"], c["pos"], c["lengths"], n_layers=cfg.n_layers, n_seq=cfg.n_seq,
                          n_kv_heads=cfg.n_kv_heads) for c in caches]
    ws = T.workspace(calib, descs[0], B)
    t0 = cfg.start_pos_range
    toks = [W.decode_token(cfg, km, j, t0 + j, "cuda") for j in range(win)]
    out = torch.empty(toks[0][2].shape, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(cfg.head_dim)
    # positions of every window run: warmup, the per-kernel breakdown and the timed steps
    # (twice: the serial schedule, then the overlapped one)
    pos = torch.arange(t0, t0 + 2 * (args.warmup + 2 * args.steps + 1) * win, dtype=torch.int32,
                       device="cuda")[:, None].expand(-1, cfg.n_seq).contiguous()      # [token][seq]
    tvec = torch.empty((cfg.n_seq,), dtype=torch.int32, device="cuda")
    state = {"cur": 0, "w": 0}
    stream = torch.cuda.current_stream()
    in_place = not args.out_of_place
    moved = {}

    # timed region: events around every 8th decode-attention launch of a window only
    sampled = list(range(0, win, 8))
    state["sample"] = False

    def window(count_moves=False):
        cur = state["cur"]
        d = descs[cur]
        for j in range(win):
            k_new, v_new, q = toks[j]
            T.tri_append(d, k_new, v_new, pos[state["w"] * win + j], stream=stream)
            if state["sample"]:
                T.tri_timing_enable(j % 8 == 0, only=["decode_attn"])
            T.tri_decode_attn(d, cfg.n_q_heads, q, scale, out, stream=stream)
        if state["sample"]:
            T.tri_timing_enable(False)
        tvec.fill_(t0 + (state["w"] + 1) * win)
        if in_place:
            before = caches[cur]["pos"][:, :B].clone() if count_moves else None
            T.tri_prune_window(calib, d, tvec, B, d, caches[cur]["lengths"], ws, stream=stream,
                               path=T.TRI_INPLACE_FILL_FREED if args.fill_freed else T.TRI_PATH_AUTO)
            if count_moves:             # rows the prune wrote: slots below B whose key changed
                moved["rows"] = int((caches[cur]["pos"][:, :B] != before).sum())
        else:
            nxt = caches[1 - cur]
            T.tri_prune_window(calib, d, tvec, B, descs[1 - cur], nxt["lengths"], ws, stream=stream)
            state["cur"] = 1 - cur
        state["w"] += 1

    # the overlapped schedule: window w's prune on a second stream, group by group
    groups = [LayerGroups(c, n_layers=cfg.n_layers, n_seq=cfg.n_seq, n_kv_heads=cfg.n_kv_heads,
                          n_groups=args.overlap_groups) for c in caches]
    prune_stream = torch.cuda.Stream()
    pruners = [OverlappedPrune(calib, groups[i], groups[1 - i], B, ws, stream, prune_stream) for i in (0, 1)]

    def window_overlapped():
        cur = state["cur"]
        d = descs[cur]
        for j in range(win):
            k_new, v_new, q = toks[j]
            p = pos[state["w"] * win + j]
            if state["sample"]:                 # every 8th whole-cache launch (step 0 runs in groups)
                T.tri_timing_enable(j % 8 == 1, only=["decode_attn"])
            if j == 0 and state["pending"] is not None:
                first_step(state["pending"], groups[cur], cfg.n_q_heads, k_new, v_new, p, q, scale, out, stream)
                state["pending"] = None
                continue
            T.tri_append(d, k_new, v_new, p, stream=stream)
            if j == win - 1:                    # the window's tokens are in: prune beside this step's attention
                tvec.fill_(t0 + (state["w"] + 1) * win)
                pruners[cur].launch(tvec)
                state["pending"] = pruners[cur]
            T.tri_decode_attn(d, cfg.n_q_heads, q, scale, out, stream=stream)
        if state["sample"]:
            T.tri_timing_enable(False)
        state["cur"] = 1 - cur
        state["w"] += 1

    def drain():                                # the last window's prune, inside the timed region
        if state["pending"] is not None:
            for g in range(args.overlap_groups):
                state["pending"].wait(g)
            state["pending"] = None

    for i in range(args.warmup):
        window(count_moves=in_place and i == args.warmup - 1)
    torch.cuda.synchronize()
    kt = kernel_breakdown(T, window, args.steps)          # every kernel, untimed
    state["sample"] = True
    ms, kt_timed = timed_steps(T, window, args.steps, stream, ["decode_attn"])
    state["sample"] = False
    state["pending"] = None
    for i in range(args.warmup):
        window_overlapped()
    drain()
    torch.cuda.synchronize()
    ms_ov, _ = timed_steps(T, window_overlapped, args.steps, stream, [], finish=drain)
    es = 2
    # decode attention reads every valid K and V row once per step (lengths B+1 .. B+win over a
    # window); the timed region brackets the launches j = 0, 8, ..., so their bytes are counted
    attn_bytes = (cfg.n_seg * sum(B + j + 1 for j in range(win)) * cfg.head_dim * es * 2
                  + win * (out.numel() * (es + 4)))
    sampled_bytes = (cfg.n_seg * sum(B + j + 1 for j in sampled) * cfg.head_dim * es * 2
                     + len(sampled) * (out.numel() * (es + 4)))
    attn_launches, attn_ms = kt_timed["decode_attn"]
    attn_avg = attn_ms / attn_launches
    attn_gbs = sampled_bytes / len(sampled) / (attn_avg * 1e-3) / 1e9
    # score reads every key; compaction reads and writes K, V and position of each copied row
    # (all B kept rows out of place; in place, the rows moved, counted on the last warmup window)
    copied = moved.get("rows", cfg.n_seg * B) if in_place else cfg.n_seg * B
    prune_bytes = cfg.n_seg * (B + win) * cfg.head_dim * es + copied * (4 * cfg.head_dim * es + 8)
    kernels = {k: {"avg_ms": round(v[1] / v[0], 4), "launches": v[0]} for k, v in kt.items() if v[0]}
    kernels["decode_attn"]["algorithmic_bytes"] = round(attn_bytes / win)        # per launch, window average
    kernels["decode_attn"]["timed_region_avg_ms"] = round(attn_avg, 4)           # the sampled launches
    prune_ms = sum(v["avg_ms"] for k, v in kernels.items() if k not in ("append", "decode_attn"))
    tokens = win * cfg.n_seq
    result = {
        "metric": "decode tokens/sec over the pruned cache (GPT-OSS-shaped loop, prune every 128 tokens)",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": (f"gptoss: {cfg.n_layers} layers x {cfg.n_seq} sequences x {cfg.n_kv_heads} KV heads, "
                                f"GQA {cfg.group}, head_dim {cfg.head_dim}, bf16, B={B}; a step is one {win}-token "
                                f"window (append + decode attention per token, then the prune "
                                f"{'in place' if in_place else 'into a second cache'})"),
                   "tokens_per_step": tokens,
                   "in_place_layout": (("fill freed slots" if args.fill_freed else "slot order") if in_place
                                       else None)},
        "pages_context": PAGES_CONTEXT,
        "roofline": {"bound": "hbm", "kernel": "decode_attn", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("decode_attn", "gptoss")},
        "prune": {"algorithmic_bytes": prune_bytes, "ms": round(prune_ms, 4),
                  "achieved_GBs": round(prune_bytes / (prune_ms * 1e-3) / 1e9, 1),
                  "in_place": in_place, "rows_copied": copied},
        "overlapped": {"schedule": (f"prune out of place on a second stream in {args.overlap_groups} layer groups, "
                                    "beside the window's last attention and the next window's first step"),
                       "ms_per_step": round(ms_ov, 4), "tokens_per_s": round(tokens / (ms_ov * 1e-3), 1),
                       "vs_serial": round(ms / ms_ov, 4)},
        "kernels": kernels,
    }
    calib.free()
    print(json.dumps(result), flush=True)


def bench_calibrate(args, T, W):
    """Offline calibration from sampled pre-RoPE queries, Qwen3-8B-shaped: 36
    layers x 4096 samples x 32 query heads x 128 dims, bf16.  A step is one
    tri_calibrate over all of them (the samples are resident in HBM)."""
    import torch
    cfg = W.CONFIGS["qwen36l"]
    n = 4096
    q = W.query_samples(cfg, n, device="cuda")
    L, _, Hq, d = q.shape
    mag = torch.empty((L, Hq, d // 2), device="cuda")
    phase, conc = torch.empty_like(mag), torch.empty_like(mag)
    import ctypes
    sz = ctypes.c_size_t(0)
    T.load().tri_calibrate_workspace_size(L, n, Hq, d, ctypes.byref(sz))
    ws = torch.empty(sz.value, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    def step():
        T.tri_calibrate(q, mag, phase, conc, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kt = kernel_breakdown(T, step, args.steps)
    ms, kt_timed = timed_steps(T, step, args.steps, stream, ["calibrate"])
    kernels = {k: {"avg_ms": round(v[1] / v[0], 4), "launches": v[0]} for k, v in kt.items() if v[0]}
    alg = q.numel() * q.element_size() + 3 * mag.numel() * 4
    kernels["calibrate"]["algorithmic_bytes"] = q.numel() * q.element_size()
    part = kt_timed["calibrate"][1] / kt_timed["calibrate"][0]
    kernels["calibrate"]["timed_region_avg_ms"] = round(part, 4)
    gbs = q.numel() * q.element_size() / (part * 1e-3) / 1e9
    result = {
        "metric": "query samples calibrated/sec (offline centre magnitude, phase and concentration)",
        "value": round(L * n * Hq / (ms * 1e-3) / 1e9, 3), "unit": "G (sample, head) rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"calib: {L} layers x {n} samples x {Hq} query heads x {d} dims, bf16 pre-RoPE queries",
                   "algorithmic_bytes": alg},
        "roofline": {"bound": "hbm", "kernel": "calibrate", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("calibrate", "calib")},
        "kernels": kernels,
    }
    print(json.dumps(result), flush=True)


def bench_ragged(args, T, W):
    """Ragged paged batch: 64 sequences x 8 KV heads, N ~ U{4096..65536} in
    16-token pages of a shared pool, B = 4096, pruned into fresh pages; then
    one decode-attention step reading the pruned pages in place.  A step is the
    prune plus that attention step."""
    import math

    import torch
    cfg = W.CONFIGS["ragged"]
    B = cfg.budget
    pc = W.paged_cache(cfg, "cuda")
    cal = W.calibration(cfg)
    calib = T.tri_calib_load(cal["mag"], cal["phase"], cal["conc"], cal["offsets"], n_kv_heads=cfg.n_kv_heads,
                             rope_theta=cfg.theta)
    src = T.cache_desc(pc["k"], pc["v"], pc["pos"], pc["lengths"], n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=pc["page_table"], page_size=cfg.page_size,
                       max_pages=pc["max_pages"])
    nk = torch.zeros((cfg.n_seg,), dtype=torch.int32, device="cuda")
    dst = T.cache_desc(pc["out_k"], pc["out_v"], pc["out_pos"], nk, n_layers=1, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads, page_table=pc["out_page_table"], page_size=cfg.page_size,
                       max_pages=pc["out_max_pages"])
    ws = T.workspace(calib, src, B)
    q = torch.randn((1, cfg.n_seq, cfg.n_q_heads, cfg.head_dim), device="cuda").to(cfg.dtype)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(cfg.head_dim)
    stream = torch.cuda.current_stream()

    def step():
        T.tri_prune_window(calib, src, pc["t"], B, dst, nk, ws, stream=stream)
        T.tri_decode_attn(dst, cfg.n_q_heads, q, scale, out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kt = kernel_breakdown(T, step, args.steps)
    ms, kt_timed = timed_steps(T, step, args.steps, stream, ["decode_attn"])
    kernels = {k: {"avg_ms": round(v[1] / v[0], 4), "launches": v[0]} for k, v in kt.items() if v[0]}
    lens = pc["lengths"].long()
    kept = torch.clamp(lens, max=B)
    es = 2
    n_keys = int(lens.sum())
    prune_bytes = n_keys * cfg.head_dim * es + int(kept.sum()) * (4 * cfg.head_dim * es + 8)
    prune_ms = sum(v["avg_ms"] for k, v in kernels.items() if k != "decode_attn")
    attn_bytes = int(kept.sum()) * cfg.head_dim * es * 2
    attn_avg = kt_timed["decode_attn"][1] / kt_timed["decode_attn"][0]
    attn_gbs = attn_bytes / (attn_avg * 1e-3) / 1e9
    kernels["decode_attn"]["timed_region_avg_ms"] = round(attn_avg, 4)
    kernels["decode_attn"]["algorithmic_bytes"] = attn_bytes
    kernels["score"]["algorithmic_bytes"] = n_keys * cfg.head_dim * es
    result = {
        "metric": "keys scored+pruned/sec on the ragged paged batch (G keys/s)",
        "value": round(n_keys / (prune_ms * 1e-3) / 1e9, 3), "unit": "G keys/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": (f"ragged: {cfg.n_seq} sequences x {cfg.n_kv_heads} KV heads, N ~ U{{4096..65536}} "
                                f"({n_keys} keys), {cfg.page_size}-token pages, B={B}, bf16; a step is the prune "
                                "into fresh pages plus one decode-attention step over them")},
        "pass_hbm": {"algorithmic_bytes": prune_bytes, "ms": round(prune_ms, 4),
                     "achieved_GBs": round(prune_bytes / (prune_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "kernel": "decode_attn (paged)", "achieved": round(attn_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("decode_attn", "ragged")},
        "kernels": kernels, "fallback_segments": T.tri_prune_fallbacks(ws),
    }
    calib.free()
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen36l", choices=["qwen36l", "qwen1l", "tiny", "gptoss", "calib", "ragged"],
                    help="qwen36l (default): the pruning pass; gptoss: decode-loop windows; "
                         "calib: offline calibration from query samples; ragged: paged batch prune + attention")
    ap.add_argument("--unfused-steps", type=int, default=3,
                    help="qwen workloads: also time the unfused tri_score -> tri_select_topb -> tri_compact chain")
    ap.add_argument("--copy-ref", type=int, default=1,
                    help="qwen workloads: measure a 4 GiB device copy as a reference bandwidth (0: skip)")
    ap.add_argument("--out-of-place", action="store_true",
                    help="gptoss: prune into a second cache instead of in place")
    ap.add_argument("--cpu-sample", type=int, default=16,
                    help="oracle segments for the CPU baseline (at least one per host thread; 0: skip)")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="qwen workloads: MiB written before each timed pass to flush the last-level cache "
                         "(default: 1024 for caches under 16M keys, else 0)")
    ap.add_argument("--fill-freed", action="store_true",
                    help="gptoss: in-place prune in the fill-freed-slots arrangement instead of slot order")
    ap.add_argument("--overlap-groups", type=int, default=1,
                    help="gptoss: layer groups of the overlapped prune, timed after the serial schedule")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device-to-device copy of this many MiB "
                         "(known-size reference for hardware byte counters)")
    args = ap.parse_args()
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); the pruning "
              "path has no cross-GPU step: each GPU would run the same kernels on its own share of the segments",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    from long_reasoning_decode_amd import triattn as T

    T.load()
    torch.cuda.set_device(0)
    if args.workload == "gptoss":
        bench_decode_loop(args, T, W)
        return
    if args.workload == "calib":
        bench_calibrate(args, T, W)
        return
    if args.workload == "ragged":
        bench_ragged(args, T, W)
        return
    cfg = W.CONFIGS[args.workload]
    B = cfg.budget
    t_gen = time.perf_counter()
    g = W.dense_cache(cfg, "cuda")
    cal = W.calibration(cfg)
    calib = T.tri_calib_load(cal["mag"], cal["phase"], cal["conc"], cal["offsets"], n_kv_heads=cfg.n_kv_heads,
                             rope_theta=cfg.theta)
    src = T.cache_desc(g["k"], g["v"], g["pos"], g["lengths"], n_layers=cfg.n_layers, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads)
    out = {"k": torch.empty((cfg.n_seg, B, cfg.head_dim), dtype=cfg.dtype, device="cuda"),
           "pos": torch.empty((cfg.n_seg, B), dtype=torch.int32, device="cuda"),
           "lengths": torch.zeros((cfg.n_seg,), dtype=torch.int32, device="cuda")}
    out["v"] = torch.empty_like(out["k"])
    dst = T.cache_desc(out["k"], out["v"], out["pos"], out["lengths"], n_layers=cfg.n_layers, n_seq=cfg.n_seq,
                       n_kv_heads=cfg.n_kv_heads)
    ws = T.workspace(calib, src, B)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"# inputs ready in {t_gen:.1f} s: {cfg.n_seg} segments x {cfg.n_keys} keys", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def step():
        T.tri_prune_window(calib, src, g["t"], B, dst, out["lengths"], ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # every kernel's duration (untimed steps), then the timed region with only
    # the dominant HBM-bound kernel bracketed by events
    kt = kernel_breakdown(T, step, args.steps)
    heavy = ("score", "select_gather", "gather")
    dom = max(heavy, key=lambda k: kt.get(k, (0, 0.0))[1] / max(kt.get(k, (0, 0.0))[0], 1))
    # Small caches fit the 256 MB last-level cache, and back to back each pass
    # would find the last one's inputs there: those workloads are timed pass by
    # pass, each after a 1 GiB flush.  The 36-layer cache (48 GB) needs none.
    flush_mib = args.flush_mib if args.flush_mib >= 0 else (1024 if cfg.n_seg * cfg.n_keys < (1 << 24) else 0)
    if flush_mib:
        T.tri_timing_reset()
        T.tri_timing_enable(True, only=[dom])
        ms = flushed_steps(step, args.steps, stream, flush_mib)
        T.tri_timing_enable(False)
        kt_timed = T.tri_timing_read()
        warm_ms, _ = timed_steps(T, step, args.steps, stream, [])
    else:
        ms, kt_timed = timed_steps(T, step, args.steps, stream, [dom])
        warm_ms = None
    fallbacks = T.tri_prune_fallbacks(ws)
    print(f"# timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # small caches: the same pass captured once in a HIP graph and replayed
    # (no launch gaps between its kernels), timed the same two ways
    graph_replay = None
    if flush_mib:
        def step_current():
            T.tri_prune_window(calib, src, g["t"], B, dst, out["lengths"], ws, stream=torch.cuda.current_stream())
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step_current()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_current()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_ms = flushed_steps(graph.replay, args.steps, stream, flush_mib)
        g_warm, _ = timed_steps(T, graph.replay, args.steps, stream, [])
        graph_replay = {"ms_per_step": round(g_ms, 4), "warm_ms_per_step": round(g_warm, 4),
                        "value": round(cfg.n_seg * cfg.n_keys / (g_ms * 1e-3) / 1e9, 3)}
        del graph

    # the unfused chain on the same cache (tri_score -> tri_select_topb -> tri_compact), after the timed region
    unfused = None
    if args.unfused_steps > 0:
        agg = torch.empty((cfg.n_seg, cfg.n_keys), dtype=torch.float32, device="cuda")
        idx = torch.empty((cfg.n_seg, B), dtype=torch.int32, device="cuda")
        nk2 = torch.empty((cfg.n_seg,), dtype=torch.int32, device="cuda")

        def chain():
            T.tri_score(calib, src, g["t"], agg, ws, stream=stream)
            T.tri_select_topb(agg, g["lengths"], B, idx, nk2, stream=stream)
            T.tri_compact(src, idx, nk2, B, dst, stream=stream)
        chain()
        torch.cuda.synchronize()
        T.tri_timing_reset()
        T.tri_timing_enable(True)
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for _ in range(args.unfused_steps):
            chain()
        u1.record(stream)
        torch.cuda.synchronize()
        T.tri_timing_enable(False)
        ukt = T.tri_timing_read()
        unfused = {"ms_per_step": round(u0.elapsed_time(u1) / args.unfused_steps, 4), "steps": args.unfused_steps,
                   "kernels": {k: round(v[1] / v[0], 4) for k, v in ukt.items() if v[0]}}
        del agg, idx, nk2
        torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth() if args.copy_ref else None

    n_keys = cfg.n_seg * cfg.n_keys
    n_kept = int(out["lengths"].long().sum())
    es = 2 if cfg.dtype == torch.bfloat16 else 4
    b_score, b_gather = algorithmic_bytes(n_keys, cfg.n_seg, n_kept, cfg.head_dim, es)
    kernels = {}
    # select_gather: the fused select + compaction; below 256 segments the pass
    # runs select, then a separate many-workgroup gather, timed as such
    for name, bytes_per_launch in (("score", b_score), ("select_gather", b_gather), ("gather", b_gather)):
        launches, total = kt.get(name, (0, 0.0))
        if launches:
            avg = total / launches
            kernels[name] = {"avg_ms": round(avg, 4), "launches": launches,
                             "algorithmic_bytes": bytes_per_launch,
                             "achieved_GBs": round(bytes_per_launch / (avg * 1e-3) / 1e9, 1)}
    for name in ("phase", "sample", "select", "split_select", "score_fallback", "select_fallback"):
        launches, total = kt.get(name, (0, 0.0))
        if launches:
            kernels[name] = {"avg_ms": round(total / launches, 4), "launches": launches}
    dom_bytes = {"score": b_score, "select_gather": b_gather, "gather": b_gather}[dom]
    dom_avg = kt_timed[dom][1] / kt_timed[dom][0]
    achieved = round(dom_bytes / (dom_avg * 1e-3) / 1e9, 1)
    kernels[dom]["timed_region_avg_ms"] = round(dom_avg, 4)
    traffic = read_traffic(dom, args.workload)
    pass_gbs = (b_score + b_gather) / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(n_keys / (ms * 1e-3) / 1e9, 3),
        "unit": "G keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: Qwen3-8B-shaped cache, {cfg.n_layers} layers x {cfg.n_seq} sequences x "
                         f"{cfg.n_kv_heads} KV heads x {cfg.n_keys} keys, head_dim {cfg.head_dim}, GQA {cfg.group}, "
                         f"B={B}, {len(cfg.offsets)} geometric offsets, one prune pass"),
            "kv_dtype": "bf16" if es == 2 else "f32", "score_dtype": "f32", "keys_per_step": n_keys,
            "kept_per_step": n_kept,
            "timing": (f"each pass timed alone after a {flush_mib} MiB flush of the last-level cache"
                       if flush_mib else "passes back to back between two events"),
        },
        "warm_ms_per_step": round(warm_ms, 4) if warm_ms is not None else None,
        "graph_replay": graph_replay,
        "pages_context": PAGES_CONTEXT,
        "pass_hbm": {"algorithmic_bytes": b_score + b_gather, "achieved_GBs": round(pass_gbs, 1),
                     "frac_of_peak": round(pass_gbs / HBM_PEAK_GBS, 4),
                     "device_copy_GBs": round(copy_gbs, 1) if copy_gbs else None,
                     "frac_of_device_copy": round(pass_gbs / copy_gbs, 4) if copy_gbs else None},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernels": kernels,
        "fallback_segments": fallbacks,
        "unfused_chain": unfused,
    }
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(W, cfg, g, cal, B, args.cpu_sample)
    calib.free()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
