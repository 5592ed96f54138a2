"""GPU parity of the offline calibration (tri_calibrate) against the oracle:
centre magnitude, phase and concentration per (layer, query head, band) of
sampled pre-RoPE queries.  Tolerances: per-sample arithmetic is fp32 and the
sums fp64, so M is checked to 2e-6 relative, R to 2e-6 absolute, and the
phase through the centre it describes: |e^{i phi} - e^{i phi_ref}| times the
resultant |mean q_f| within 2e-6 * M (the phase of a vanishing resultant is
ill-conditioned and carries no weight)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import log, stored

pytestmark = pytest.mark.gpu


def _check(q_cpu, mag, phase, conc, pairs, what):
    for (l, h) in pairs:
        rows = stored(q_cpu[l, :, h])
        M, phi, R = oracle.calibrate(rows)
        F = M.shape[0]
        x = rows.astype(np.float64) if rows.dtype == np.float32 else \
            (rows.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        res = np.abs(np.mean(x[:, :F] + 1j * x[:, F:], axis=0))
        gm, gp, gr = mag[l, h].numpy(), phase[l, h].numpy(), conc[l, h].numpy()
        tag = f"{what} layer {l} head {h}"
        assert np.all(np.abs(gm - M) <= 2e-6 * np.maximum(M, 1e-30) + 1e-12), f"{tag}: magnitude"
        assert np.all(np.abs(gr - R) <= 2e-6), f"{tag}: concentration {np.abs(gr - R).max():.2e}"
        assert np.all(np.abs(np.exp(1j * gp) - np.exp(1j * phi)) * res <= 2e-6 * M + 1e-12), f"{tag}: phase"


def _run(T, q):
    L, n, Hq, d = q.shape
    mag = torch.full((L, Hq, d // 2), float("nan"), device="cuda")
    phase, conc = torch.full_like(mag, float("nan")), torch.full_like(mag, float("nan"))
    T.tri_calibrate(q, mag, phase, conc)
    torch.cuda.synchronize()
    return mag.cpu(), phase.cpu(), conc.cpu()


@pytest.mark.parametrize("d,dtype,n", [(64, torch.float32, 300), (128, torch.bfloat16, 513), (64, torch.bfloat16, 7),
                                       (128, torch.float32, 1), (128, torch.float32, 64)])
def test_calibrate_small_every_head(gpu_lib, d, dtype, n):
    """Every (layer, head); sample counts spanning chunk tails; a head with a
    zero band, a head of identical samples, a head of antipodal pairs."""
    T = gpu_lib
    cfg = W.CONFIGS["tiny"].replace(n_layers=2, n_kv_heads=2, group=4, head_dim=d, dtype=dtype, seed=3)
    log(f"case calibrate small d={d} {dtype} n={n}")
    q = W.query_samples(cfg, n)
    q[0, :, 1] = q[0, 0, 1].clone()                # identical samples: R = 1
    q[1, :, 2, 0] = 0.0                            # band 0 real part zero ...
    q[1, :, 2, d // 2] = 0.0                       # ... and imaginary part: a zero band
    half = (n // 2) * 2
    q[1, 1:half:2, 3] = -q[1, 0:half - 1:2, 3]     # antipodal pairs
    mag, phase, conc = _run(T, q.cuda())
    pairs = [(l, h) for l in range(cfg.n_layers) for h in range(cfg.n_q_heads)]
    _check(q, mag, phase, conc, pairs, f"small d{d}")
    assert torch.all(conc[0, 1] > 1 - 2e-6)
    assert torch.all(mag[1, 2, 0] == 0) and torch.all(conc[1, 2, 0] == 0) and torch.all(phase[1, 2, 0] == 0)


def test_calibrate_qwen_shaped(gpu_lib):
    """36 layers x 32 query heads x 4096 samples, head_dim 128, bf16 (1.2 GB of
    samples); the oracle checks a spread of (layer, head) pairs."""
    T = gpu_lib
    cfg = W.CONFIGS["qwen36l"]
    n = 4096
    log(f"case calibrate qwen-shaped: {cfg.n_layers} x {n} x {cfg.n_q_heads} x {cfg.head_dim}")
    q = W.query_samples(cfg, n, device="cuda")
    mag, phase, conc = _run(T, q)
    pairs = [(0, 0), (7, 31), (18, 5), (35, 17), (35, 31)]
    qc = torch.stack([q[l, :, h] for l, h in pairs]).cpu()          # only the checked rows to the host
    sub = {p: i for i, p in enumerate(pairs)}
    for p in pairs:
        i = sub[p]
        _check(qc[i:i + 1, :, None], mag[p[0]:p[0] + 1, p[1]:p[1] + 1], phase[p[0]:p[0] + 1, p[1]:p[1] + 1],
               conc[p[0]:p[0] + 1, p[1]:p[1] + 1], [(0, 0)], f"qwen layer {p[0]} head {p[1]}")
