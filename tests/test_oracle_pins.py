"""Pins for the oracle: checks against what the pages and the mathematics fix,
never against the oracle itself.

* A hand-derived worked example (tests/golden/hand_example.json).
* Closed form at full concentration (R = 1): the score is then the exact
  RoPE logit of the centre query at t + o, averaged over offsets, computed
  here by rotating the centre vector (not by un-rotating the key).
* Invariants: offset averaging is linear, relative-position (shift)
  invariance, monotonicity in R, zero key scores zero.
* z-score / max against numpy's mean/std/max; invariance to per-head affine
  maps; G = 1.
* Top-B against a brute-force rank count on tiny inputs with ties.
* Gather, paged read-out and decode attention against numpy / torch.
* Top-B ties at the cut: the earlier position wins, on caches whose slots
  are not in position order, by the same brute-force rank count.
* Fill-freed-slots layout (the optional in-place arrangement): hand-worked
  cases (tests/golden/fill_freed_layout.json), a brute-force search over
  every arrangement of tiny kept sets for the one that obeys the layout's two
  rules, and invariants on large kept sets.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(**kw):
    return W.CONFIGS["tiny"].replace(**kw)


def _segment(cfg, n=None, seed=0):
    """A small fp32/bf16 segment from the synthetic key model (CPU)."""
    cfg = cfg.replace(seed=seed, n_keys=n or cfg.n_keys)
    c = W.dense_cache(cfg, "cpu")
    cal = W.calibration(cfg)
    K = W.to_stored_numpy(c["k"][0])
    V = W.to_stored_numpy(c["v"][0])
    pos = c["pos"][0].numpy()
    G = cfg.group
    return cfg, K, V, pos, int(c["t"][0]), cal["mag"][0, :G].numpy(), cal["phase"][0, :G].numpy(), \
        cal["conc"][0, :G].numpy()


def _as_float(K):
    if K.dtype == np.uint16:
        return (K.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return K.astype(np.float64)


def _rope_rotate(vec, p, theta):
    """Textbook RoPE (rotate-half pairing) of a real d-vector at position p."""
    d = vec.shape[-1]
    F = d // 2
    w = theta ** (-2.0 * np.arange(F) / d)
    c, s = np.cos(w * p), np.sin(w * p)
    x1, x2 = vec[..., :F], vec[..., F:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


# ---------------------------------------------------------------- worked example
def test_hand_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    env = {"cos": math.cos, "sin": math.sin, "pi": math.pi}
    rows = np.array([[eval(e, env) for e in r] for r in ex["rows_expr"]], dtype=np.float32)
    expect = np.array([[eval(e, env) for e in r] for r in ex["expected_expr"]])
    S = oracle.score_segment(rows, np.array(ex["positions"]), ex["t"], ex["theta"],
                             np.array(ex["mag"]), np.array(ex["phase"]), np.array(ex["conc"]),
                             ex["offsets"])
    np.testing.assert_allclose(S, expect, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- closed form at R = 1
@pytest.mark.parametrize("dtype,d,theta", [(torch.float32, 64, 1e4), (torch.bfloat16, 128, 1e6),
                                           (torch.bfloat16, 64, 150000.0)])
def test_full_concentration_equals_rope_logit(dtype, d, theta):
    cfg, K, _, pos, t, M, phi, _ = _segment(_tiny(dtype=dtype, head_dim=d, theta=theta), n=48)
    R = np.ones_like(M)
    offs = [1, 2, 4, 8, 16, 1024, 32768]
    S = oracle.score_segment(K, pos, t, theta, M, phi, R, offs)
    M64, phi64 = M.astype(np.float64), phi.astype(np.float64)
    centre = np.concatenate([M64 * np.cos(phi64), M64 * np.sin(phi64)], axis=-1)      # [G][d]
    Kf = _as_float(K)
    expect = np.zeros_like(S)
    for o in offs:
        q = _rope_rotate(centre.astype(np.float64), t + o, theta)           # [G][d]
        expect += q @ Kf.T
    expect /= len(offs)
    scale = np.abs(expect).max()
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-10 * scale)


def test_single_offset_is_plain_rope_logit_at_large_positions():
    # Positions near 65536 with w0 = 1: the oracle's fp64 phase must hold there.
    cfg = _tiny(head_dim=128, theta=1e6, dtype=torch.float32)
    rng = np.random.default_rng(3)
    N, d, F, G = 16, 128, 64, 2
    pos = rng.integers(60000, 65536, size=N).astype(np.int32)
    pre = rng.normal(size=(N, d))
    K = np.stack([_rope_rotate(pre[i], pos[i], cfg.theta) for i in range(N)]).astype(np.float32)
    M = rng.uniform(0.5, 2, size=(G, F)).astype(np.float32)
    phi = rng.uniform(0, 2 * np.pi, size=(G, F)).astype(np.float32)
    t, o = 65536, 65536
    S = oracle.score_segment(K, pos, t, cfg.theta, M, phi, np.ones_like(M), [o])
    M64, phi64 = M.astype(np.float64), phi.astype(np.float64)
    centre = np.concatenate([M64 * np.cos(phi64), M64 * np.sin(phi64)], axis=-1)
    expect = _rope_rotate(centre, t + o, cfg.theta) @ K.astype(np.float64).T
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-9 * np.abs(expect).max())


# ---------------------------------------------------------------- invariants
def test_offset_average_is_linear():
    cfg, K, _, pos, t, M, phi, R = _segment(_tiny(), n=40)
    offs = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]
    S = oracle.score_segment(K, pos, t, cfg.theta, M, phi, R, offs)
    singles = [oracle.score_segment(K, pos, t, cfg.theta, M, phi, R, [o]) for o in offs]
    np.testing.assert_allclose(S, np.mean(singles, axis=0), rtol=1e-12, atol=1e-12)


def test_relative_position_shift_invariance():
    """Keys re-rotated at p + s, queried at t + s: same scores (up to fp32 storage)."""
    cfg = _tiny()
    rng = np.random.default_rng(1)
    N, d, G = 32, cfg.head_dim, cfg.group
    F = d // 2
    pre = torch.tensor(rng.normal(size=(N, d)))
    p = torch.arange(N, dtype=torch.int64) * 7
    cal = W.calibration(cfg)
    M, phi, R = (cal[k][0].numpy() for k in ("mag", "phase", "conc"))
    out = []
    for s in (0, 12345):
        re, im = W.rotate(pre[:, :F], pre[:, F:], p + s, cfg)
        K = torch.cat([re, im], -1).to(torch.float32).numpy()
        out.append(oracle.score_segment(K, (p + s).numpy().astype(np.int32), 5000 + s, cfg.theta,
                                        M, phi, R, cfg.offsets))
    np.testing.assert_allclose(out[0], out[1], rtol=0, atol=1e-5 * np.abs(out[0]).max())


def test_norm_term_grows_as_concentration_falls_and_zero_key_scores_zero():
    cfg, K, _, pos, t, M, phi, R = _segment(_tiny(), n=24)
    S_hi = oracle.score_segment(K, pos, t, cfg.theta, M, phi, np.full_like(R, 0.875), cfg.offsets)
    S_lo = oracle.score_segment(K, pos, t, cfg.theta, M, phi, np.full_like(R, 0.125), cfg.offsets)
    S_mid = oracle.score_segment(K, pos, t, cfg.theta, M, phi, np.full_like(R, 0.5), cfg.offsets)
    assert np.all(S_lo > S_hi)
    # the weight is affine in R (midpoint of R gives the midpoint of scores)
    np.testing.assert_allclose(S_mid, 0.5 * (S_hi + S_lo), rtol=1e-12, atol=1e-12)
    Kz = np.zeros_like(K)
    Sz = oracle.score_segment(Kz, pos, t, cfg.theta, M, phi, R, cfg.offsets)
    assert np.all(Sz == 0.0)


# ---------------------------------------------------------------- z-score and max
def test_zscore_max_against_numpy():
    rng = np.random.default_rng(2)
    S = rng.normal(size=(4, 501)) * np.array([[3.0], [0.5], [10.0], [1.0]]) + np.array([[100.0], [-3], [0], [7]])
    mu, sigma, A = oracle.zscore_max(S)
    np.testing.assert_allclose(mu, S.mean(axis=1), rtol=1e-13)
    np.testing.assert_allclose(sigma, S.std(axis=1, ddof=0), rtol=1e-12)
    z = (S - S.mean(axis=1, keepdims=True)) / S.std(axis=1, keepdims=True)
    np.testing.assert_allclose(A, z.max(axis=0), rtol=0, atol=1e-12)
    # per-head positive affine maps leave the aggregate unchanged
    S2 = S * np.array([[2.0], [0.1], [7.0], [1.0]]) + np.array([[5.0], [1.0], [-9.0], [0.0]])
    np.testing.assert_allclose(oracle.zscore_max(S2)[2], A, rtol=0, atol=1e-10)
    # one head: A is that head's z-score
    np.testing.assert_allclose(oracle.zscore_max(S[:1])[2], z[0], rtol=0, atol=1e-12)


def test_zscore_constant_head_gives_zero():
    S = np.vstack([np.full(10, 3.25), np.arange(10.0)])
    mu, sigma, A = oracle.zscore_max(S)
    assert sigma[0] == 0.0 and mu[0] == 3.25
    # a value whose naive sum is inexact (0.1 * 3 != 0.3 in binary) still has zero spread
    for v, n in ((0.1, 3), (1.0 / 3.0, 3000), (123.456, 2047)):
        mu_c, sigma_c, A_c = oracle.zscore_max(np.full((2, n), v))
        assert np.all(sigma_c == 0.0) and np.all(mu_c == v) and np.all(A_c == 0.0)
    z1 = (np.arange(10.0) - 4.5) / np.arange(10.0).std()
    np.testing.assert_allclose(A, np.maximum(z1, 0.0), atol=1e-12)


# ---------------------------------------------------------------- selection
def _brute_kept(A, B, pos=None):
    """Key i is kept iff fewer than B keys rank above it: a higher score, or
    the same score at an earlier position (the same position: a lower slot)."""
    N = len(A)
    p = list(range(N)) if pos is None else [int(x) for x in pos]
    return [i for i in range(N)
            if sum(1 for j in range(N)
                   if A[j] > A[i] or (A[j] == A[i] and (p[j], j) < (p[i], i))) < B]


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_brute_force_rank(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 65))
    B = int(rng.integers(1, N + 4))
    A = rng.integers(-3, 4, size=N).astype(np.float64) * 0.5     # many ties
    if seed % 3 == 0:
        A = rng.normal(size=N)
    idx = oracle.select_topb(A, B)
    assert list(idx) == _brute_kept(A, B)
    assert len(idx) == min(N, B)


@pytest.mark.parametrize("seed", range(12))
def test_select_ties_go_to_the_earlier_position(seed):
    """Positions scrambled across slots (a cache whose slots are not in
    position order): among tied scores the earliest positions are kept, not
    the lowest slots; repeated positions fall back to the lower slot."""
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(2, 65))
    B = int(rng.integers(1, N))
    A = rng.integers(-2, 3, size=N).astype(np.float64)            # heavy ties
    pos = rng.permutation(N * 3)[:N].astype(np.int32)
    if seed % 4 == 3:
        pos = rng.integers(0, 6, size=N).astype(np.int32)          # repeated positions
    idx = oracle.select_topb(A, B, pos)
    assert list(idx) == _brute_kept(A, B, pos)
    assert list(oracle.select_topb(A.astype(np.float32), B, pos)) == list(idx)


def test_select_tie_rule_hand_case():
    """Four keys tie at the cut with slots in reverse position order: the two
    earliest positions (slots 3 and 2) survive, where slot order would keep 0
    and 1."""
    A = np.array([1.0, 1.0, 1.0, 1.0, 5.0])
    pos = np.array([40, 30, 20, 10, 0], dtype=np.int32)
    assert list(oracle.select_topb(A, 3, pos)) == [2, 3, 4]
    assert list(oracle.select_topb(A, 3)) == [0, 1, 4]


def test_select_f32_signed_zero_and_budget_at_least_n():
    A = np.array([0.0, -0.0, 1.0, -0.0, 0.0], dtype=np.float32)
    assert list(oracle.select_topb(A, 3)) == [0, 1, 2]
    assert list(oracle.select_topb(A, 3, np.array([9, 8, 7, 1, 2], dtype=np.int32))) == [2, 3, 4]
    assert list(oracle.select_topb(np.array([3.0, 1.0, 2.0]), 3)) == [0, 1, 2]
    assert list(oracle.select_topb(np.array([3.0, 1.0, 2.0]), 10)) == [0, 1, 2]
    assert len(oracle.select_topb(np.zeros(0), 4)) == 0


# ---------------------------------------------------------------- data movement
def test_gather_and_paged_rows_are_byte_copies():
    rng = np.random.default_rng(4)
    src = rng.integers(0, 2 ** 16, size=(50, 8), dtype=np.uint16)
    idx = np.array([0, 3, 4, 17, 49], dtype=np.int32)
    assert np.array_equal(oracle.gather_rows(src, idx), src[idx])
    pool = rng.integers(0, 2 ** 16, size=(7, 4, 8), dtype=np.uint16)
    pt = np.array([5, 0, 3], dtype=np.int32)
    rows = oracle.paged_rows(pool, pt, 4, 10)
    assert np.array_equal(rows, pool[pt].reshape(12, 8)[:10])


# ---------------------------------------------------------------- decode attention
def test_decode_attention_against_torch_sdpa():
    rng = np.random.default_rng(5)
    G, d, N = 8, 64, 77
    q = torch.tensor(rng.normal(size=(G, d)), dtype=torch.float32).to(torch.bfloat16)
    K = torch.tensor(rng.normal(size=(N, d)), dtype=torch.float32).to(torch.bfloat16)
    V = torch.tensor(rng.normal(size=(N, d)), dtype=torch.float32).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    out = oracle.decode_attn(W.to_stored_numpy(q), W.to_stored_numpy(K), W.to_stored_numpy(V), scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double()[None, :, None, :], K.double()[None, None].expand(1, G, N, d),
        V.double()[None, None].expand(1, G, N, d), scale=scale)[0, :, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    # equal logits: the output is the mean of V
    out0 = oracle.decode_attn(np.zeros((G, d), np.float32), K.float().numpy(), V.float().numpy(), 1.0)
    np.testing.assert_allclose(out0, np.broadcast_to(V.double().mean(0).numpy(), (G, d)), atol=1e-12)


# ---------------------------------------------------------------- whole chain
def test_prune_chain_tiny_shapes_and_budget_cases():
    cfg, K, V, pos, t, M, phi, R = _segment(_tiny(), n=300)
    r = oracle.prune_segment(K, V, pos, t, cfg.theta, M, phi, R, cfg.offsets, 100)
    assert r["idx"].shape == (100,) and np.all(np.diff(r["idx"]) > 0)
    assert np.array_equal(r["K"], K[r["idx"]]) and np.array_equal(r["pos"], pos[r["idx"]])
    # the kept keys are exactly the 100 largest aggregated scores
    thr = np.sort(r["A"])[-100]
    assert np.all(r["A"][r["idx"]] >= thr)
    r2 = oracle.prune_segment(K, V, pos, t, cfg.theta, M, phi, R, cfg.offsets, 300)
    assert np.array_equal(r2["idx"], np.arange(300)) and np.array_equal(r2["V"], V)


# ---------------------------------------------------------------- offline calibration
# Centre magnitude M = mean |q_f|, phase phi = arg sum q_f, concentration R = mean
# resultant length | mean q_f / |q_f| | of sampled pre-RoPE queries (band f = q[f] + i q[f+F]).

def _band_rows(z):
    """Rows [n][2F] (fp32) from complex bands z [n][F] in the half-split layout."""
    return np.concatenate([z.real, z.imag], axis=1).astype(np.float32)


def test_calibrate_identical_samples_are_fully_concentrated():
    z = np.array([1.5 * np.exp(0.7j), 0.25 * np.exp(-2.0j), 3.0 * np.exp(3.0j)])
    q = _band_rows(np.tile(z, (9, 1)))
    M, phi, R = oracle.calibrate(q)
    zs = q[0, :3].astype(np.float64) + 1j * q[0, 3:].astype(np.float64)
    assert np.allclose(M, np.abs(zs), rtol=1e-15, atol=0)
    assert np.allclose(phi, np.angle(zs), rtol=0, atol=1e-15)
    assert np.allclose(R, 1.0, rtol=0, atol=1e-15)


def test_calibrate_antipodal_pairs_have_zero_concentration():
    z = np.array([[2.0 * np.exp(0.3j), 1.0 * np.exp(1.1j)],
                  [-0.5 * np.exp(0.3j), -4.0 * np.exp(1.1j)]])
    M, phi, R = oracle.calibrate(_band_rows(z))
    assert np.allclose(R, 0.0, atol=1e-7)
    assert np.allclose(M, [1.25, 2.5], rtol=1e-6)
    # the sum points along the larger sample: band 0 along +e^{0.3i}, band 1 along -e^{1.1i}
    assert abs(phi[0] - 0.3) < 1e-6 and abs(abs(phi[1] - 1.1) - np.pi) < 1e-6


@pytest.mark.parametrize("a,phi0", [(0.4, 1.0), (1.2, -2.5), (np.pi / 2, 0.1)])
def test_calibrate_symmetric_spread_gives_cosine_concentration(a, phi0):
    """Equal-magnitude samples at phi0 +- a: R = cos a exactly, phase phi0."""
    r = 1.75
    z = np.array([[r * np.exp(1j * (phi0 + a))], [r * np.exp(1j * (phi0 - a))]] * 3)
    M, phi, R = oracle.calibrate(_band_rows(z))
    assert abs(R[0] - np.cos(a)) < 1e-6
    assert abs(M[0] - r) < 1e-6
    if np.cos(a) > 1e-3:
        assert abs(phi[0] - phi0) < 1e-6


def test_calibrate_zero_sample_counts_but_adds_no_direction():
    z = np.array([[0.0 + 0.0j], [2.0 * np.exp(0.5j)]])
    M, phi, R = oracle.calibrate(_band_rows(z))
    assert abs(R[0] - 0.5) < 1e-7 and abs(M[0] - 1.0) < 1e-7 and abs(phi[0] - 0.5) < 1e-7
    Mz, phz, Rz = oracle.calibrate(_band_rows(np.zeros((3, 2))))
    assert np.all(Mz == 0.0) and np.all(phz == 0.0) and np.all(Rz == 0.0)


def test_calibrate_scale_and_rotation():
    rng = np.random.default_rng(4)
    z = (1.0 + 0.2 * rng.standard_normal((64, 5))) * np.exp(1j * (0.3 + 0.5 * rng.standard_normal((64, 5))))
    q = _band_rows(z)
    M, phi, R = oracle.calibrate(q)
    M2, phi2, R2 = oracle.calibrate(q * np.float32(2.0))        # exact scaling
    assert np.array_equal(M2, 2.0 * M) and np.allclose(phi2, phi, atol=1e-15) and np.allclose(R2, R, atol=1e-15)
    beta = 0.9
    M3, phi3, R3 = oracle.calibrate(_band_rows(z * np.exp(1j * beta)))
    assert np.allclose(M3, M, rtol=1e-6) and np.allclose(R3, R, atol=1e-6)
    assert np.allclose(np.angle(np.exp(1j * (phi3 - phi - beta))), 0.0, atol=1e-6)


def test_calibrate_half_split_pairing():
    """Band f pairs element f with element f + F (not f with f + 1)."""
    q = np.array([[3.0, 0.0, 0.0, 4.0]], dtype=np.float32)    # band 0 = 3 + 0i, band 1 = 0 + 4i
    M, phi, R = oracle.calibrate(q)
    assert np.allclose(M, [3.0, 4.0]) and np.allclose(phi, [0.0, np.pi / 2])


def test_calibrate_bf16_matches_fp32_on_representable_values():
    rng = np.random.default_rng(5)
    q = (rng.integers(-64, 64, size=(40, 16)) / 16.0).astype(np.float32)   # exact in bf16
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    for x, y in zip(oracle.calibrate(q), oracle.calibrate(qb)):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- score variants
# The ablated components ([YY] 主实验结果: trigonometric score, adaptive weighting,
# geometric offsets) and the R-weighted centre reading, each pinned to the
# method as read by an exact relation.

def _variant_case(seed=9, d=64, G=3, N=40):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((N, d)).astype(np.float32)
    pos = np.sort(rng.choice(5000, N, replace=False)).astype(np.int32)
    M = rng.uniform(0.5, 2.0, (G, d // 2)).astype(np.float32)
    phi = rng.uniform(0, 2 * np.pi, (G, d // 2)).astype(np.float32)
    R = np.array(rng.choice([0.125, 0.5, 0.875], (G, d // 2)), dtype=np.float32)
    return K, pos, M, phi, R


def test_variant_trig_only_plus_norm_only_is_the_method():
    K, pos, M, phi, R = _variant_case()
    args = (K, pos, 5100, 1e4, M, phi, R, [1, 2, 4, 8, 16])
    S, trig, norm = oracle.score_segment(*args, parts=True)
    St = oracle.score_segment(*args, variant=oracle.VAR_TRIG_ONLY)
    Sn = oracle.score_segment(*args, variant=oracle.VAR_NORM_ONLY)
    assert np.array_equal(St, trig) and np.array_equal(Sn, norm)
    assert np.allclose(St + Sn, S, rtol=1e-14, atol=1e-12)


def test_variant_fixed_weight_reduces_to_the_method_at_zero_concentration():
    K, pos, M, phi, _ = _variant_case(seed=10)
    R0 = np.zeros_like(M)
    args = (K, pos, 5100, 1e4, M, phi)
    assert np.array_equal(oracle.score_segment(*args, R0, [1, 4, 16], variant=oracle.VAR_FIXED_WEIGHT),
                          oracle.score_segment(*args, R0, [1, 4, 16]))
    # and its norm term is the plain magnitude-weighted band norm
    R = _variant_case(seed=10)[4]
    Sf = oracle.score_segment(*args, R, [1], variant=oracle.VAR_FIXED_WEIGHT | oracle.VAR_NORM_ONLY)
    F = K.shape[1] // 2
    bandnorm = np.hypot(K[:, :F].astype(np.float64), K[:, F:].astype(np.float64))
    assert np.allclose(Sf, M.astype(np.float64) @ bandnorm.T, rtol=1e-13)


def test_variant_r_weighted_trig_is_the_method_at_full_concentration_and_scales_with_r():
    K, pos, M, phi, _ = _variant_case(seed=11)
    args = (K, pos, 5100, 1e4, M, phi)
    R1 = np.ones_like(M)
    assert np.array_equal(oracle.score_segment(*args, R1, [1, 2, 4], variant=oracle.VAR_R_WEIGHTED_TRIG),
                          oracle.score_segment(*args, R1, [1, 2, 4]))
    Rh = np.full_like(M, 0.5)
    Stw = oracle.score_segment(*args, Rh, [1, 2, 4], variant=oracle.VAR_R_WEIGHTED_TRIG | oracle.VAR_TRIG_ONLY)
    St = oracle.score_segment(*args, Rh, [1, 2, 4], variant=oracle.VAR_TRIG_ONLY)
    assert np.allclose(Stw, 0.5 * St, rtol=1e-13, atol=1e-12)


def test_variant_flags_are_checked():
    K, pos, M, phi, R = _variant_case()
    with pytest.raises(ValueError):
        oracle.score_segment(K, pos, 5100, 1e4, M, phi, R, [1], variant=oracle.VAR_TRIG_ONLY | oracle.VAR_NORM_ONLY)
    with pytest.raises(ValueError):
        oracle.score_segment(K, pos, 5100, 1e4, M, phi, R, [1], variant=16)


# ---------------------------------------------------------------- fill-freed-slots layout
def test_fill_freed_layout_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "fill_freed_layout.json")))["cases"]
    for c in cases:
        got = oracle.fill_freed_layout(c["kept"], c["N"])
        assert got.tolist() == c["src_of"], c["why"]


def _brute_fill_freed(kept, N):
    """Every arrangement of the kept keys over slots [0, n), filtered by the two
    rules: a kept key below n keeps its slot, and the keys that move land in
    freed slots in the same order as their old slots.  Exactly one survives."""
    import itertools
    n = len(kept)
    found = []
    for perm in itertools.permutations(kept):
        if any(k < n and perm[k] != k for k in kept):
            continue
        moved = [(j, perm[j]) for j in range(n) if perm[j] != j]
        if all(a[1] < b[1] for a, b in zip(moved, moved[1:])):
            found.append(list(perm))
    assert len(found) == 1, f"{kept}, N={N}: {len(found)} arrangements satisfy the rules"
    return found[0]


def test_fill_freed_layout_brute_force_tiny():
    import itertools
    for N in range(1, 8):
        for n in range(0, N + 1):
            for kept in itertools.combinations(range(N), n):
                got = oracle.fill_freed_layout(list(kept), N).tolist()
                assert got == _brute_fill_freed(list(kept), N), (kept, N)


def test_fill_freed_layout_invariants():
    rng = np.random.default_rng(11)
    for N, n in [(1152, 1024), (32768, 2048), (5000, 4096), (300, 1)]:
        kept = np.sort(rng.choice(N, size=n, replace=False)).astype(np.int32)
        src_of = oracle.fill_freed_layout(kept, N)
        assert np.array_equal(np.sort(src_of), kept)             # the same keys, each once
        stay = kept[kept < n]
        assert np.array_equal(src_of[stay], stay)                 # kept keys below n do not move
        moved = np.nonzero(src_of != np.arange(n))[0]
        assert len(moved) == np.count_nonzero(kept >= n)          # only keys from above move
        assert np.all(src_of[moved] >= n) and np.all(np.diff(src_of[moved]) > 0)


def test_fill_freed_layout_rejects_bad_lists():
    with pytest.raises(ValueError):
        oracle.fill_freed_layout([3, 1], 5)                          # not ascending
    with pytest.raises(ValueError):
        oracle.fill_freed_layout([0, 5], 5)                          # slot out of range
