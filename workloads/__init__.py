"""Seeded synthetic inputs for the TriAttention pruning path.

This module only synthesises inputs: offline calibration draws, a synthetic
post-RoPE KV cache (dense or paged), per-step decode tokens and queries.  It
holds none of the scoring, aggregation, selection or compaction arithmetic,
and both the HIP path's tests and the oracle consume what it produces.

Key model (per layer, KV head and rotary band f): a fixed pre-RoPE centre with
magnitude ~ U[0.5, 2] and phase ~ U[0, 2pi); each key is centre + sigma * (n1 +
i n2), n ~ N(0, 1), then rotated by its position (half-split pairing: band f is
elements f and f + d/2, frequency theta^(-2f/d)) in fp64 and rounded once to
the storage dtype.  Query centres: magnitude ~ U[0.5, 2], phase ~ U[0, 2pi),
concentration R ~ U[0.3, 0.99] per (layer, query head, band).  Values ~ N(0,1).

Every tensor is drawn from its own torch.Generator seeded from (seed, tag), on
the device it is generated on; torch's CPU and GPU generators differ, so a test
that needs the same bytes on both sides generates once and copies.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import torch

TWO_PI = 2.0 * math.pi


@dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    n_seq: int
    n_kv_heads: int
    group: int            # query heads per KV head (GQA group size)
    head_dim: int
    theta: float
    dtype: torch.dtype    # storage dtype of K/V (and decode queries)
    budget: int           # B
    offsets: tuple        # future offsets O
    n_keys: int = 0       # N per segment (dense configs)
    t: int | None = None  # next query position; default N
    sigma: float | None = None          # fixed key noise; None = per head ~ U[sig_lo, sig_hi]
    sig_lo: float = 0.1
    sig_hi: float = 0.6
    len_range: tuple | None = None      # ragged: per-sequence N ~ U{lo..hi}
    page_size: int = 0                  # >0: paged layout
    windows: int = 0                    # decode loop: number of windows
    window: int = 128                   # decode loop: tokens per window
    start_pos_range: int = 32768        # decode loop: initial positions drawn from [0, this)
    seed: int = 0

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def n_seg(self) -> int:
        return self.n_layers * self.n_seq * self.n_kv_heads

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def geometric(n: int) -> tuple:
    return tuple(2 ** i for i in range(n))


CONFIGS = {
    # 1 layer, 1 KV head, GQA 4, d 64, fp32, N=2048 at t=2048, B=512, 11 offsets, sigma 0.3
    "tiny": Config("tiny", 1, 1, 1, 4, 64, 1e4, torch.float32, 512, geometric(11),
                   n_keys=2048, t=2048, sigma=0.3),
    # Qwen3-8B-shaped single layer, batch 1: N = 32768 + one pending 128-token window
    "qwen1l": Config("qwen1l", 1, 1, 8, 4, 128, 1e6, torch.bfloat16, 2048, geometric(16),
                     n_keys=32768 + 128),
    # Qwen3-8B-shaped full model cache: 36 layers x 16 sequences x 8 KV heads at 32768 keys
    "qwen36l": Config("qwen36l", 36, 16, 8, 4, 128, 1e6, torch.bfloat16, 2048, geometric(16),
                      n_keys=32768),
    # ragged paged batch: 64 sequences, N ~ U{4096..65536}, 16-token pages, B=4096
    "ragged": Config("ragged", 1, 64, 8, 4, 128, 1e6, torch.bfloat16, 4096, geometric(17),
                     len_range=(4096, 65536), page_size=16),
    # GPT-OSS-20B-like decode loop: 24 layers, 64 q / 8 kv heads, d 64, batch 32
    "gptoss": Config("gptoss", 24, 32, 8, 8, 64, 150000.0, torch.bfloat16, 1024, geometric(16),
                     windows=16, window=128),
}


def _gen(device, seed: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 7919 + 12345) % (2 ** 63))
    return g


def _uniform(shape, lo, hi, g, device, dtype=torch.float64):
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=dtype)


def band_frequencies(cfg: Config, device="cpu") -> torch.Tensor:
    f = torch.arange(cfg.head_dim // 2, device=device, dtype=torch.float64)
    return cfg.theta ** (-2.0 * f / cfg.head_dim)


def calibration(cfg: Config):
    """Offline query-centre statistics, fp32 [L][Hq][F] host tensors."""
    F = cfg.head_dim // 2
    shape = (cfg.n_layers, cfg.n_q_heads, F)
    M = _uniform(shape, 0.5, 2.0, _gen("cpu", cfg.seed, 1), "cpu")
    phi = _uniform(shape, 0.0, TWO_PI, _gen("cpu", cfg.seed, 2), "cpu")
    R = _uniform(shape, 0.3, 0.99, _gen("cpu", cfg.seed, 3), "cpu")
    return {"mag": M.float().contiguous(), "phase": phi.float().contiguous(),
            "conc": R.float().contiguous(), "offsets": torch.tensor(cfg.offsets, dtype=torch.int32)}


def key_model(cfg: Config):
    """Pre-RoPE key centres [L][Hkv][F] (magnitude, phase) and noise sigma [L][Hkv]."""
    F = cfg.head_dim // 2
    shape = (cfg.n_layers, cfg.n_kv_heads, F)
    mag = _uniform(shape, 0.5, 2.0, _gen("cpu", cfg.seed, 11), "cpu")
    ph = _uniform(shape, 0.0, TWO_PI, _gen("cpu", cfg.seed, 12), "cpu")
    if cfg.sigma is not None:
        sig = torch.full((cfg.n_layers, cfg.n_kv_heads), float(cfg.sigma), dtype=torch.float64)
    else:
        sig = _uniform((cfg.n_layers, cfg.n_kv_heads), cfg.sig_lo, cfg.sig_hi,
                       _gen("cpu", cfg.seed, 13), "cpu")
    return {"mag": mag, "phase": ph, "sigma": sig}


def rotate(pre_re, pre_im, positions, cfg: Config):
    """Post-RoPE (re, im) of pre-RoPE bands at integer positions (fp64).

    pre_re/pre_im: [..., n, F]; positions: broadcastable to [..., n]."""
    w = band_frequencies(cfg, pre_re.device)
    ang = positions.to(torch.float64).unsqueeze(-1) * w
    c, s = torch.cos(ang), torch.sin(ang)
    return pre_re * c - pre_im * s, pre_re * s + pre_im * c


def _pack(re, im, dtype):
    return torch.cat([re, im], dim=-1).to(dtype)


def synth_keys(cfg: Config, km, layer, heads, positions: torch.Tensor, g, device):
    """Keys drawn from the centre + noise model.  `layer` and `heads` are ints or
    index tensors broadcast against positions [..., n] (one entry per leading
    index); returns stored rows [..., n, d]."""
    F = cfg.head_dim // 2
    layer = torch.as_tensor(layer, device=device)
    heads = torch.as_tensor(heads, device=device)
    mag = km["mag"].to(device)[layer, heads]        # [..., F]
    ph = km["phase"].to(device)[layer, heads]
    sig = km["sigma"].to(device)[layer, heads]      # [...]
    shape = tuple(positions.shape) + (F,)
    n1 = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    n2 = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    c_re = (mag * torch.cos(ph)).unsqueeze(-2)
    c_im = (mag * torch.sin(ph)).unsqueeze(-2)
    s = sig.reshape(sig.shape + (1, 1))
    re, im = rotate(c_re + s * n1, c_im + s * n2, positions, cfg)
    return _pack(re, im, cfg.dtype)


def dense_cache(cfg: Config, device="cpu", capacity: int | None = None, layers=None):
    """Dense cache [n_seg][cap][d] with segment s = (l * n_seq + b) * Hkv + h.

    Keys at positions 0..N-1 (N = cfg.n_keys), next query at t (default N)."""
    N = cfg.n_keys
    cap = capacity or N
    assert cap >= N
    d = cfg.head_dim
    km = key_model(cfg)
    layers = range(cfg.n_layers) if layers is None else layers
    n_l = len(layers)
    per_l = cfg.n_seq * cfg.n_kv_heads
    K = torch.zeros((n_l * per_l, cap, d), dtype=cfg.dtype, device=device)
    V = torch.zeros_like(K)
    pos = torch.zeros((n_l * per_l, cap), dtype=torch.int32, device=device)
    heads = torch.arange(cfg.n_kv_heads, device=device).repeat(cfg.n_seq)       # [per_l]
    p = torch.arange(N, device=device, dtype=torch.int64)
    for i, l in enumerate(layers):
        g = _gen(device, cfg.seed, 1000 + l)
        rows = synth_keys(cfg, km, l, heads, p.expand(per_l, N), g, device)
        K[i * per_l:(i + 1) * per_l, :N] = rows
        gv = _gen(device, cfg.seed, 5000 + l)
        V[i * per_l:(i + 1) * per_l, :N] = torch.randn((per_l, N, d), generator=gv, device=device,
                                                       dtype=torch.float32).to(cfg.dtype)
        pos[i * per_l:(i + 1) * per_l, :N] = p.to(torch.int32)
    t = cfg.t if cfg.t is not None else N
    return {
        "k": K, "v": V, "pos": pos,
        "lengths": torch.full((n_l * per_l,), N, dtype=torch.int32, device=device),
        "t": torch.full((cfg.n_seq,), t, dtype=torch.int32, device=device),
        "capacity": cap,
    }


def ragged_lengths(cfg: Config):
    lo, hi = cfg.len_range
    g = _gen("cpu", cfg.seed, 21)
    return torch.randint(lo, hi + 1, (cfg.n_seq,), generator=g, dtype=torch.int64)


def paged_cache(cfg: Config, device="cpu"):
    """Ragged paged cache: per-sequence N_b ~ U{lo..hi} (all KV heads of a sequence
    alike), keys at positions 0..N_b-1, next query at t_b = N_b.  Each segment
    owns ceil(N/page) pages of a shared pool in a random order; a second pool
    of fresh pages (also randomly assigned) receives the compacted output."""
    assert cfg.n_layers == 1 and cfg.page_size > 0
    ps, d = cfg.page_size, cfg.head_dim
    lens_b = ragged_lengths(cfg)
    n_seg = cfg.n_seg
    lens = lens_b.repeat_interleave(cfg.n_kv_heads)                 # [n_seg]
    npages = (lens + ps - 1) // ps
    max_pages = int(npages.max())
    total = int(npages.sum())
    perm = torch.randperm(total, generator=_gen("cpu", cfg.seed, 22))
    page_table = torch.zeros((n_seg, max_pages), dtype=torch.int32)
    off = 0
    for s in range(n_seg):
        k = int(npages[s])
        page_table[s, :k] = perm[off:off + k].to(torch.int32)
        off += k
    km = key_model(cfg)
    Kp = torch.zeros((total, ps, d), dtype=cfg.dtype, device=device)
    Vp = torch.zeros_like(Kp)
    Pp = torch.zeros((total, ps), dtype=torch.int32, device=device)
    pt_dev = page_table.to(device)
    g = _gen(device, cfg.seed, 1000)
    gv = _gen(device, cfg.seed, 5000)
    for s in range(n_seg):
        n = int(lens[s])
        k = int(npages[s])
        h = s % cfg.n_kv_heads
        p = torch.arange(k * ps, device=device, dtype=torch.int64)
        rows = synth_keys(cfg, km, 0, torch.tensor(h, device=device), p, g, device)
        vals = torch.randn((k * ps, d), generator=gv, device=device, dtype=torch.float32).to(cfg.dtype)
        rows[n:] = 0
        vals[n:] = 0
        pages = pt_dev[s, :k].long()
        Kp[pages] = rows.view(k, ps, d)
        Vp[pages] = vals.view(k, ps, d)
        pp = p.to(torch.int32)
        pp[n:] = 0
        Pp[pages] = pp.view(k, ps)
    out_pages = (cfg.budget + ps - 1) // ps
    out_total = n_seg * out_pages
    operm = torch.randperm(out_total, generator=_gen("cpu", cfg.seed, 23)).to(torch.int32)
    out_table = operm.view(n_seg, out_pages).contiguous()
    return {
        "k": Kp, "v": Vp, "pos": Pp, "page_table": pt_dev,
        "lengths": lens.to(torch.int32).to(device), "max_pages": max_pages,
        "t": lens_b.to(torch.int32).to(device),
        "out_k": torch.zeros((out_total, ps, d), dtype=cfg.dtype, device=device),
        "out_v": torch.zeros((out_total, ps, d), dtype=cfg.dtype, device=device),
        "out_pos": torch.zeros((out_total, ps), dtype=torch.int32, device=device),
        "out_page_table": out_table.to(device), "out_max_pages": out_pages,
    }


def decode_start(cfg: Config, device="cpu"):
    """Decode-loop start state: B retained keys per segment at distinct sorted
    positions drawn uniformly from [0, start_pos_range), next query at
    t0 = start_pos_range; capacity B + window."""
    B, d = cfg.budget, cfg.head_dim
    cap = B + cfg.window
    per_l = cfg.n_seq * cfg.n_kv_heads
    km = key_model(cfg)
    K = torch.zeros((cfg.n_seg, cap, d), dtype=cfg.dtype, device=device)
    V = torch.zeros_like(K)
    pos = torch.zeros((cfg.n_seg, cap), dtype=torch.int32, device=device)
    heads = torch.arange(cfg.n_kv_heads, device=device).repeat(cfg.n_seq)
    for l in range(cfg.n_layers):
        gp = _gen(device, cfg.seed, 3000 + l)
        r = torch.rand((per_l, cfg.start_pos_range), generator=gp, device=device)
        p = torch.topk(r, B, dim=1).indices.sort(dim=1).values          # [per_l, B]
        g = _gen(device, cfg.seed, 1000 + l)
        sl = slice(l * per_l, (l + 1) * per_l)
        K[sl, :B] = synth_keys(cfg, km, l, heads, p, g, device)
        gv = _gen(device, cfg.seed, 5000 + l)
        V[sl, :B] = torch.randn((per_l, B, d), generator=gv, device=device,
                                dtype=torch.float32).to(cfg.dtype)
        pos[sl, :B] = p.to(torch.int32)
    return {
        "k": K, "v": V, "pos": pos, "capacity": cap, "key_model": km,
        "lengths": torch.full((cfg.n_seg,), B, dtype=torch.int32, device=device),
        "t": torch.full((cfg.n_seq,), cfg.start_pos_range, dtype=torch.int32, device=device),
    }


def decode_token(cfg: Config, km, step: int, t: int, device="cpu"):
    """One generated token for every segment: new key/value rows [n_seg][d] at
    position t (all sequences share t), and post-RoPE queries [L][n_seq][Hq][d]
    whose pre-RoPE bands are the calibrated centre plus N(0, 0.3^2) noise."""
    d = cfg.head_dim
    F = d // 2
    per_l = cfg.n_seq * cfg.n_kv_heads
    g = _gen(device, cfg.seed, 100000 + step)
    seg = torch.arange(cfg.n_seg, device=device)
    pos1 = torch.full((cfg.n_seg, 1), t, device=device, dtype=torch.int64)
    k_new = synth_keys(cfg, km, seg // per_l, seg % cfg.n_kv_heads, pos1, g, device)[:, 0]
    v_new = torch.randn((cfg.n_seg, d), generator=g, device=device,
                        dtype=torch.float32).to(cfg.dtype)
    cal = calibration(cfg)
    M = cal["mag"].to(device, torch.float64)            # [L][Hq][F]
    ph = cal["phase"].to(device, torch.float64)
    shape = (cfg.n_layers, cfg.n_seq, cfg.n_q_heads, F)
    qr = (M * torch.cos(ph)).unsqueeze(1) + 0.3 * torch.randn(shape, generator=g, device=device,
                                                              dtype=torch.float64)
    qi = (M * torch.sin(ph)).unsqueeze(1) + 0.3 * torch.randn(shape, generator=g, device=device,
                                                              dtype=torch.float64)
    re, im = rotate(qr, qi, torch.tensor(t, device=device), cfg)
    q = _pack(re, im, cfg.dtype)
    return k_new, v_new, q


def to_stored_numpy(x: torch.Tensor):
    """CPU numpy view of stored rows: float32 stays float32; bf16 -> raw uint16 bits."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(x.dtype)


def synthetic_scores(n_seg: int, capacity: int, seed: int = 0):
    """Aggregated-score arrays [n_seg][capacity] (fp32) for exercising top-B
    selection on its own: per segment one of several value mixes - Gaussian,
    heavily tied (few distinct levels), signed zeros, all equal."""
    g = _gen("cpu", seed, 31)
    A = torch.randn((n_seg, capacity), generator=g, dtype=torch.float32)
    for s in range(n_seg):
        kind = s % 4
        if kind == 1:
            A[s] = torch.randint(-3, 4, (capacity,), generator=g).float() * 0.25
        elif kind == 2:
            z = torch.randint(0, 3, (capacity,), generator=g)
            A[s] = torch.where(z == 0, torch.tensor(-0.0), torch.where(z == 1, torch.tensor(0.0), A[s]))
        elif kind == 3 and s % 8 == 3:
            A[s] = 1.5
    return A


def query_samples(cfg: Config, n_samples: int, device="cpu", sigma: float = 0.3, seed_tag: int = 7000):
    """Sampled pre-RoPE queries [L][n_samples][Hq][d] in the storage dtype: per
    band, the calibration centre M e^{i phi} plus complex Gaussian noise of
    std sigma per component (half-split layout)."""
    F = cfg.head_dim // 2
    cal = calibration(cfg)
    M = cal["mag"].to(device, torch.float64)[:, None]            # [L][1][Hq][F]
    ph = cal["phase"].to(device, torch.float64)[:, None]
    g = _gen(device, cfg.seed, seed_tag)
    shape = (cfg.n_layers, n_samples, cfg.n_q_heads, F)
    re = M * torch.cos(ph) + sigma * torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    im = M * torch.sin(ph) + sigma * torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    return _pack(re, im, cfg.dtype)
