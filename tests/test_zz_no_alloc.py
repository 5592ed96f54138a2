"""tri_prune_window_static (the pruning pass on the library's own scratch,
for callers that cannot allocate) against tri_prune_window_ex with a caller
workspace: the same caches byte for byte, on two calls in a row, the second
with a smaller cache (the scratch keeps the first call's contents), out of
place and in place, on both scoring paths; and a cache whose workspace
exceeds the scratch is refused before any launch."""
import pytest
import torch

import workloads as W
from helpers import calib_for, dense_desc, empty_like_dense, log

pytestmark = pytest.mark.gpu


def _cache(cfg):
    return W.dense_cache(cfg, "cuda")


def _both(T, cfg, path, in_place):
    """One pass each way on copies of the same cache; returns both results."""
    calib, _ = calib_for(T, cfg)
    B = cfg.budget
    base = _cache(cfg)
    res = []
    for static in (False, True):
        g = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
        desc = dense_desc(T, cfg, g)
        if in_place:
            dst, out = desc, g
        else:
            out = empty_like_dense(g, B)
            dst = dense_desc(T, cfg, out)
        if static:
            T.tri_prune_window_static(calib, desc, g["t"], B, dst, out["lengths"], path=path)
        else:
            ws = T.workspace(calib, desc, B)
            T.tri_prune_window(calib, desc, g["t"], B, dst, out["lengths"], ws, path=path)
        torch.cuda.synchronize()
        res.append({k: out[k].clone() for k in ("k", "v", "pos", "lengths")})
    calib.free()
    return res


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("path", ["full", "candidates"])
def test_static_scratch_matches_caller_workspace(gpu_lib, path, in_place):
    T = gpu_lib
    p = T.TRI_PATH_FULL if path == "full" else T.TRI_PATH_CANDIDATES
    big = W.CONFIGS["qwen1l"]                                         # 8 x 32896 keys: 4.7 MB of workspace
    small = W.CONFIGS["tiny"].replace(head_dim=64, group=8, dtype=torch.bfloat16, theta=150000.0, n_kv_heads=3,
                                      n_seq=2, n_keys=5000, t=5003, budget=600, sigma=None, seed=9)
    for name, cfg in (("qwen1l", big), ("small", small)):            # the second call is the smaller one
        log(f"case static scratch: {name}, path {path}, in place {in_place}")
        ref, got = _both(T, cfg, p, in_place)
        for key in ("k", "v", "pos", "lengths"):
            assert torch.equal(got[key], ref[key]), f"{name} {path}: {key} differs from the caller-workspace pass"


def test_static_scratch_refuses_a_larger_workspace(gpu_lib):
    """80 segments of 65536 keys need more than the scratch: refused on the
    host, nothing launched, outputs untouched."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(head_dim=128, group=4, dtype=torch.bfloat16, theta=1e6, n_kv_heads=8,
                                    n_seq=10, n_keys=64, t=64, budget=16, sigma=None, seed=3)
    calib, _ = calib_for(T, cfg)
    g = _cache(cfg)
    desc = dense_desc(T, cfg, g)
    need = T.tri_workspace_size(calib, desc, cfg.budget)
    assert need <= T.TRI_STATIC_SCRATCH_BYTES
    desc.capacity = 65536                          # described larger than stored: refused before any launch
    assert T.tri_workspace_size(calib, desc, cfg.budget) > T.TRI_STATIC_SCRATCH_BYTES
    before = {k: g[k].clone() for k in ("k", "pos", "lengths")}
    # in place (dst = src), so no other buffer is checked against the larger extent
    with pytest.raises(T.TriError) as e:
        T.tri_prune_window_static(calib, desc, g["t"], cfg.budget, desc, g["lengths"])
    assert e.value.code == T.TRI_ERR_WORKSPACE
    assert "scratch" in T.tri_last_error()
    torch.cuda.synchronize()
    for k, v in before.items():
        assert torch.equal(g[k], v), f"{k} was written"
    calib.free()
