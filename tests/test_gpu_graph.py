"""The pruning pass captured in a HIP graph (torch.cuda.CUDAGraph): every replay
writes what the eager call writes.  The pass issues kernel launches only (what
it must clear it clears with fill kernels, never memset nodes), so a caller can
capture it.  Each case replays the graph several times with eager work in
between (the destination overwritten, in place the source restored) and
checks every replay against the eager result, byte for byte, and the
fallback count."""
import pytest
import torch

import workloads as W
from helpers import calib_for, dense_desc, empty_like_dense, log

pytestmark = pytest.mark.gpu

# name: (cache shape, budget, path, in place); the first takes the split
# select (fewer than 256 segments of at least 8192 slots), the second the
# fused 256-thread select, the third the candidate pass with its sample and
# fallback kernels, the fourth the in-place gather.
CASES = {
    "split select": (dict(n_kv_heads=2, n_seq=7, n_keys=9000), 600, "auto", False),
    "fused select": (dict(n_kv_heads=8, n_seq=40, n_keys=3000), 700, "auto", False),
    "candidate pass": (dict(n_kv_heads=4, n_seq=64, n_keys=8192), 1024, "candidates", False),
    "in place": (dict(n_kv_heads=8, n_seq=40, n_keys=3000), 700, "auto", True),
}
KEYS = ("k", "v", "pos", "lengths")


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_the_eager_pass(gpu_lib, case):
    T = gpu_lib
    shape, B, path, in_place = CASES[case]
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, t=shape["n_keys"] + 5,
                                    budget=B, sigma=None, seed=71, **shape)
    log(f"case graph replay: {case}, {cfg.n_seg} segments x {cfg.n_keys} keys, B={B}")
    T.tri_timing_enable(False)
    p = T.TRI_PATH_CANDIDATES if path == "candidates" else T.TRI_PATH_AUTO
    g = W.dense_cache(cfg, "cuda")
    n = cfg.n_seg
    g["lengths"] = torch.randint(B // 2, cfg.n_keys + 1, (n,), generator=torch.Generator().manual_seed(7),
                                 dtype=torch.int32).to("cuda")
    g["lengths"][0] = cfg.n_keys
    calib, _ = calib_for(T, cfg)
    pristine = {k: g[k].clone() for k in KEYS}
    src = dense_desc(T, cfg, g)
    ws = T.workspace(calib, src, B)

    # eager reference
    if in_place:
        T.tri_prune_window(calib, src, g["t"], B, src, g["lengths"], ws, path=p)
        ref = {k: g[k].clone() for k in KEYS}
    else:
        ref = empty_like_dense(g, B)
        T.tri_prune_window(calib, src, g["t"], B, dense_desc(T, cfg, ref), ref["lengths"], ws, path=p)
    fb_ref = T.tri_prune_fallbacks(ws)
    torch.cuda.synchronize()

    out = g if in_place else empty_like_dense(g, B)
    dst = src if in_place else dense_desc(T, cfg, out)

    def restore():
        if in_place:
            for k in KEYS:
                g[k].copy_(pristine[k])

    def prune():
        T.tri_prune_window(calib, src, g["t"], B, dst, out["lengths"], ws, path=p)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        restore()
        prune()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        prune()
    torch.cuda.synchronize()

    for r in range(3):
        if in_place:
            restore()
        else:
            for k in ("k", "v"):
                out[k].fill_(float(r + 1))
            out["pos"].fill_(-7 - r)
            out["lengths"].fill_(-1)
        ws.fill_(0xA5 if r % 2 else 0x3C)             # the workspace holds nothing a pass relies on
        graph.replay()
        torch.cuda.synchronize()
        assert T.tri_prune_fallbacks(ws) == fb_ref, f"{case} replay {r}: fallback count"
        assert torch.equal(out["lengths"], ref["lengths"]), f"{case} replay {r}: kept counts"
        for s in range(n):
            nk = int(ref["lengths"][s])
            for k in ("k", "v", "pos"):
                assert torch.equal(out[k][s, :nk], ref[k][s, :nk]), f"{case} replay {r} seg {s}: {k}"
        if in_place:
            for k in ("k", "v", "pos"):
                assert torch.equal(out[k], ref[k]), f"{case} replay {r}: {k} beyond the kept rows"
    log(f"  3 replays match the eager pass (fallbacks {fb_ref})")
    del graph
    calib.free()
