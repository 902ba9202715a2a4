"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU needed).

Each test names the passage it checks.  Citations: "RG" = the reading-guide page of
"Prism: Dynamic Sparse Attention for Native 2K Joint Video-Audio Generation Model
Training"; RG M1/M2/M3 are its Method parts 1-3, RG KI its "Key ideas" list.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ----------------------------------------------------------------- RG M1: audio coupling input

def test_audio_norms_closed_forms():
    """The coupling field is the L2 norm of each token's cross-attention output (RG M1).
    Integer Pythagorean tuples, placed at scattered channels, give exact integer norms; the
    squared form is the exact integer sum of squares."""
    C = 40
    tuples = [((3, 4), 5), ((1, 2, 2), 3), ((2, 3, 6), 7), ((1, 4, 8), 9), ((2, 10, 11), 15),
              ((1, 2, 4, 10), 11), ((12, 16, 21), 29)]
    rng = np.random.default_rng(11)
    x = np.zeros((len(tuples) + 2, C), np.float32)
    want = np.zeros(len(tuples) + 2)
    for i, (t, n) in enumerate(tuples):
        ch = rng.choice(C, len(t), replace=False)
        x[i, ch] = np.array(t) * rng.choice([-1, 1], len(t))
        want[i] = n
    x[-2, 17] = -6.5  # one entry: its magnitude
    want[-2] = 6.5
    # last row stays zero: norm 0
    assert np.array_equal(oracle.audio_norms(x), want)
    assert np.array_equal(oracle.audio_norms(x, squared=True), want ** 2)


def test_audio_norms_constant_rows_and_scaling():
    """|c| sqrt(C) for a constant row (exact when C is a perfect square); a(2^k x) = 2^k a(x)
    exactly."""
    for C, root in ((64, 8), (256, 16), (9, 3)):
        c = np.array([0.75, -1.5, 3.0, -0.125], np.float32)
        x = np.repeat(c[:, None], C, axis=1)
        assert np.array_equal(oracle.audio_norms(x), np.abs(c).astype(np.float64) * root)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 512)).astype(np.float32)
    a = oracle.audio_norms(x)
    for k in (-3, 1, 5):
        assert np.array_equal(oracle.audio_norms(x * np.float32(2.0 ** k)), a * 2.0 ** k)
    assert (a > 0).all()


# ----------------------------------------------------------------------------- constants


def test_candidate_set_matches_pages():
    """RG KI: 16 shapes; RG M2: volumes {64,128,256}; reading: power-of-two edges in {2,4,8}."""
    gc = _golden("pages_constants.json")
    edges, vol = oracle.candidates()
    assert len(edges) == gc["n_candidates"] == 16
    assert sorted(set(vol.tolist())) == gc["volumes"]
    assert (np.prod(edges, axis=1) == vol).all()
    assert set(np.unique(edges).tolist()) <= {2, 4, 8}
    # independently enumerated: every {2,4,8}^3 box with a page volume, in canonical order
    mine = sorted((b[0] * b[1] * b[2], b) for b in itertools.product((2, 4, 8), repeat=3)
                  if b[0] * b[1] * b[2] in gc["volumes"])
    assert [tuple(e) for e in edges.tolist()] == [b for _, b in mine]
    assert [int((vol == B).sum()) for B in gc["volumes"]] == [7, 6, 3]
    # {1,2,4,8} would give 19, which is why the reading drops edge 1
    n19 = sum(1 for b in itertools.product((1, 2, 4, 8), repeat=3) if b[0] * b[1] * b[2] in (64, 128, 256))
    assert n19 == 19


def test_generator_uses_page_thresholds():
    gc = _golden("pages_constants.json")
    for cfg in synth.CONFIGS.values():
        assert cfg.tau128 == gc["tau128"] and cfg.tau256 == gc["tau256"]


# ----------------------------------------------------------------------------- RG M1


def _additive_field(Zgrid, heads, d, amps, freqs, seed):
    """V = sum_axis A_axis cos(2 pi f_axis x_axis / 8 + phi) per channel, no noise."""
    ZT, ZH, ZW = Zgrid
    T, H, W = 8 * ZT, 8 * ZH, 8 * ZW
    rng = np.random.default_rng(seed)
    phi = rng.uniform(0, 2 * np.pi, size=(heads, d, 3))
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    loc = [t % 8, h % 8, w % 8]
    v = np.zeros((T * H * W, heads, d))
    for ax in range(3):
        arg = 2 * np.pi * freqs[ax] * loc[ax].reshape(-1)[:, None, None] / 8 + phi[None, :, :, ax]
        v += amps[ax] * np.cos(arg)
    return v.astype(np.float32), (T, H, W)


@pytest.mark.parametrize("amps,freqs", [((1.0, 0.5, 2.0), (1, 2, 3)), ((0.0, 1.5, 0.0), (2, 1, 1)),
                                        ((1.0, 1.0, 1.0), (0, 3, 1)), ((0.25, 0.0, 3.0), (3, 0, 2))])
def test_closed_form_directional_variance(amps, freqs):
    """RG M1 variance equation on an additive cosine field with whole cycles per zone:
    sigma^2_d = A_d^2/2 for f_d in {1,2,3} and 0 for f_d = 0, r_d = sigma^2_d / sum, and the
    zone's token variance equals the sum (so the density reading gives rho = 1)."""
    v, (T, H, W) = _additive_field((1, 2, 1), 2, 16, amps, freqs, seed=3)
    st = oracle.zone_stats(v, None, T, H, W, 2, 16, 1, 1e-6)
    # float32 storage of the field limits agreement to ~1e-7
    expect = np.array([0.5 * a * a if f else 0.0 for a, f in zip(amps, freqs)])
    for m in range(2):
        np.testing.assert_allclose(st["sig2"][0, m, :3], expect, rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(st["sig2"][0, m, 3], expect.sum(), rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(st["r"][0, m], expect / expect.sum(), rtol=1e-6, atol=1e-7)
        assert st["rho"][0, m] == pytest.approx(1.0, rel=1e-6)
    # a field varying along one axis only gives r = e_axis
    if sum(1 for a, f in zip(amps, freqs) if a and f) == 1:
        ax = [i for i, (a, f) in enumerate(zip(amps, freqs)) if a and f][0]
        np.testing.assert_allclose(st["r"][0, 0], np.eye(3)[ax], atol=1e-7)


def test_rho_of_iid_noise_has_exact_mean():
    """Density reading rho = sum_d sigma^2_d / sigma^2_tok.  For iid Gaussian tokens the
    main-effect sum of squares (21 degrees of freedom per channel) is independent of the
    residual (490), so rho ~ Beta(21D/2, 490D/2) with mean exactly 21/511."""
    heads, d = 1, 64
    T, H, W = 8, 256, 256  # 1024 zones
    rng = np.random.default_rng(11)
    v = rng.standard_normal((T * H * W, heads, d), dtype=np.float32)
    st = oracle.zone_stats(v, None, T, H, W, heads, d, 1, 1e-6)
    rho = st["rho"][0]
    assert rho.shape == (1024,)
    # per-zone std of the Beta law is ~1.6e-3, so the mean of 1024 zones is within ~5e-5
    assert abs(rho.mean() - 21 / 511) < 3e-4
    assert (rho >= 0).all() and (rho <= 1 + 1e-12).all()


def test_ratios_sum_to_one_and_rho_bounded():
    """RG M1: r_{v,d} is a share of sum_d sigma^2 (sums to 1, non-negative); the audio shares
    vhat likewise; the density reading is a variance fraction in [0, 1]."""
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    st = oracle.zone_stats(inp["v"], inp["a"], 8, 16, 16, 2, 64, 1, 1e-6)
    np.testing.assert_allclose(st["r"].sum(-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(st["vhat"].sum(-1), 1.0, atol=1e-12)
    assert (st["r"] >= 0).all() and (st["vhat"] >= 0).all()
    assert ((st["rho"] >= 0) & (st["rho"] <= 1 + 1e-12)).all()
    assert ((st["abar"] >= 0) & (st["abar"] <= 1)).all() and st["abar"].max() == 1.0
    np.testing.assert_allclose(st["g"], st["r"] + st["abar"][None, :, None] * st["vhat"][None] + 1e-6,
                               rtol=0, atol=1e-15)


def test_audio_statistics_closed_form():
    """RG M1 audio terms (reading: abar = zone mean / largest zone mean; vhat = the RG M1
    directional variance of the scalar field a, normalised).  With a = c_m + sum_axis
    A_axis cos(2 pi f x / 8 + phi) per zone, vhat_d = A_d^2 / sum A^2 and abar = c_m / max c."""
    T, H, W = 8, 8, 24  # 3 zones along W
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    amps, freqs, phis = (0.3, 0.1, 0.2), (1, 3, 2), (0.4, 1.1, 2.0)
    loc = [t % 8, h % 8, w % 8]
    base = np.array([2.0, 5.0, 3.0])[w // 8]
    a = base.astype(np.float64)
    for ax in range(3):
        a = a + amps[ax] * np.cos(2 * np.pi * freqs[ax] * loc[ax] / 8 + phis[ax])
    a = a.reshape(-1).astype(np.float32)
    v = np.random.default_rng(0).standard_normal((T * H * W, 1, 8)).astype(np.float32)
    st = oracle.zone_stats(v, a, T, H, W, 1, 8, 1, 1e-6)
    A2 = np.array(amps) ** 2
    for m in range(3):
        np.testing.assert_allclose(st["vhat"][m], A2 / A2.sum(), rtol=1e-5)
    np.testing.assert_allclose(st["abar"], [2 / 5, 1.0, 3 / 5], rtol=1e-6)
    # no audio cache (first layer): abar = 0 so g = r + eps
    st0 = oracle.zone_stats(v, None, T, H, W, 1, 8, 1, 1e-6)
    np.testing.assert_allclose(st0["g"], st0["r"] + 1e-6, atol=1e-15)
    assert (st0["abar"] == 0).all()


def test_constant_zone_degenerate_cases():
    """Flat zones: sum sigma^2 = 0 gives r = 1/3 each, sigma^2_tok = 0 gives rho = 0 (so the
    largest volume); a flat audio field gives vhat = 1/3 each."""
    T, H, W = 8, 8, 8
    v = np.full((512, 2, 4), 3.5, np.float32)
    a = np.full(512, 0.7, np.float32)
    st = oracle.zone_stats(v, a, T, H, W, 2, 4, 1, 1e-6)
    np.testing.assert_allclose(st["r"][0, 0], [1 / 3] * 3)
    assert st["rho"][0, 0] == 0.0
    np.testing.assert_allclose(st["vhat"][0], [1 / 3] * 3)
    sh = oracle.assign_shapes(st["g"], st["rho"], 0.5, 0.25)
    assert sh["volume"][0, 0] == 256


def test_head_groups_use_their_own_channels():
    """Reading: D = channels of the head group; each group has its own statistics."""
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    v = inp["v"]
    st2 = oracle.zone_stats(v, inp["a"], 8, 16, 16, 2, 64, 2, 1e-6)
    for grp in range(2):
        st1 = oracle.zone_stats(np.ascontiguousarray(v[:, grp:grp + 1]), inp["a"], 8, 16, 16, 1, 64, 1, 1e-6)
        np.testing.assert_allclose(st2["sig2"][grp], st1["sig2"][0], rtol=1e-13)
        np.testing.assert_allclose(st2["g"][grp], st1["g"][0], rtol=1e-13)


# ----------------------------------------------------------------------------- RG M2


def test_volume_thresholds():
    """RG M2 thresholds tau128 = 0.5, tau256 = 0.25 (reading: rho >= 0.5 -> 64,
    0.25 <= rho < 0.5 -> 128, rho < 0.25 -> 256)."""
    rho = np.array([[0.0, 0.2499999, 0.25, 0.4999999, 0.5, 0.77, 1.0]])
    g = np.ones((1, rho.shape[1], 3))
    sh = oracle.assign_shapes(g, rho, 0.5, 0.25)
    assert sh["volume"][0].tolist() == [256, 256, 128, 128, 64, 64, 64]
    nb = 512 // sh["volume"][0]
    assert sh["zone_block_off"][0].tolist() == [0] + np.cumsum(nb).tolist()


def test_eq3_worked_examples():
    """Hand-worked values of the RG M2 log2-space optimum and nearest-candidate rule."""
    cases = _golden("eq3_worked.json")["cases"]
    rho_of = {64: 0.9, 128: 0.3, 256: 0.1}
    g = np.array([[c["g"] for c in cases]], float)
    rho = np.array([[rho_of[c["B"]] for c in cases]])
    sh = oracle.assign_shapes(g, rho, 0.5, 0.25)
    edges, _ = oracle.candidates()
    for z, c in enumerate(cases):
        assert sh["volume"][0, z] == c["B"]
        np.testing.assert_allclose(sh["lstar"][0, z], c["lstar"], atol=1e-12)
        assert edges[sh["shape_idx"][0, z]].tolist() == c["shape"]


def _random_g(n, rng):
    kinds = rng.integers(0, 4, size=n)
    g = rng.dirichlet([1, 1, 1], size=n)
    g[kinds == 1] = rng.uniform(0, 2, size=(int((kinds == 1).sum()), 3))       # arbitrary
    g[kinds == 2] = np.exp(rng.normal(0, 3, size=(int((kinds == 2).sum()), 3)))  # wide range
    sym = kinds == 3                                                            # exact symmetries
    g[sym] = rng.integers(1, 4, size=(int(sym.sum()), 3)) / 3.0
    return g + 1e-6


def test_lstar_sums_to_S_and_satisfies_kkt():
    """RG M2: prod b*_d = B (so sum l*_d = S) and b*_d ~ g_d^(-1/2): the stationarity of
    sum g_d (b_d^2 - 1) on the constraint makes g_d (b*_d)^2 equal for every axis."""
    rng = np.random.default_rng(5)
    g = _random_g(20000, rng)[None]
    rho = rng.uniform(0, 1, size=(1, g.shape[1]))
    sh = oracle.assign_shapes(g, rho, 0.5, 0.25)
    S = np.log2(sh["volume"][0])
    np.testing.assert_allclose(sh["lstar"][0].sum(-1), S, atol=1e-10)
    kkt = g[0] * 4.0 ** sh["lstar"][0]
    np.testing.assert_allclose(kkt / kkt[:, :1], 1.0, rtol=1e-9)


def test_lstar_is_the_continuous_minimiser():
    """RG M2 continuous problem solved numerically (fine grid over the constraint surface)
    lands on the closed-form l*."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        g = rng.uniform(0.05, 2.0, size=3)
        S = float(rng.choice([6, 7, 8]))
        sh = oracle.assign_shapes(g[None, None], np.array([[{6: 0.9, 7: 0.3, 8: 0.1}[S]]]), 0.5, 0.25)
        ls = sh["lstar"][0, 0]
        x = np.linspace(ls[0] - 1.5, ls[0] + 1.5, 601)
        y = np.linspace(ls[1] - 1.5, ls[1] + 1.5, 601)
        X, Y = np.meshgrid(x, y, indexing="ij")
        Zc = S - X - Y
        J = g[0] * (4.0 ** X - 1) + g[1] * (4.0 ** Y - 1) + g[2] * (4.0 ** Zc - 1)
        i, j = np.unravel_index(np.argmin(J), J.shape)
        assert abs(X[i, j] - ls[0]) <= 0.0051 and abs(Y[i, j] - ls[1]) <= 0.0051


def _brute_force_sets(g, B):
    """Minimiser sets of the page's loss sum_d g_d (b_d^2 - 1) over the candidates of volume B
    (own enumeration; canonical order = volume, then lexicographic edges)."""
    cands = sorted((b[0] * b[1] * b[2], b) for b in itertools.product((2, 4, 8), repeat=3)
                   if b[0] * b[1] * b[2] in (64, 128, 256))
    idx = [i for i, (vol, _) in enumerate(cands) if vol == B]
    J = np.array([sum(gd * (bd * bd - 1) for gd, bd in zip(g, cands[i][1])) for i in idx])
    jmin = J.min()
    return {idx[n] for n in range(len(idx)) if J[n] <= jmin * (1 + 1e-9) + 1e-15}


def test_quantisation_matches_brute_force_minimisation():
    """RG M2 nearest-candidate rule vs brute-force minimisation of sum_d g_d (b_d^2 - 1) over
    the candidates of the zone's volume: the pick must be a minimiser, and the unique one
    whenever the minimiser is unique.  (Both objectives are separable convex on the same
    integer plane and share their improving exchanges, so their minimiser sets coincide.)"""
    rng = np.random.default_rng(123)
    n = 100000
    g = _random_g(n, rng)
    rho = rng.uniform(0, 1, size=n)
    sh = oracle.assign_shapes(g[None], rho[None], 0.5, 0.25)
    vol, pick = sh["volume"][0], sh["shape_idx"][0]
    ties = 0
    for z in range(n):
        mins = _brute_force_sets(g[z], int(vol[z]))
        assert int(pick[z]) in mins, (g[z], vol[z], pick[z], mins)
        if len(mins) > 1:
            ties += 1
            assert int(pick[z]) == min(mins) or _near_tie(sh["dist"][0, z])
    assert ties < n  # symmetric g produce genuine ties; they are allowed but not everything


def _near_tie(dist):
    d = np.sort(dist[np.isfinite(dist)])
    return (d[1] - d[0]) / max(d[1], 1e-12) < 1e-5


def test_quantisation_on_tiny_config_zones():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    st = oracle.zone_stats(inp["v"], inp["a"], 8, 16, 16, 2, 64, 1, 1e-6)
    sh = oracle.assign_shapes(st["g"], st["rho"], 0.5, 0.25)
    edges, vol = oracle.candidates()
    for m in range(st["g"].shape[1]):
        mins = _brute_force_sets(st["g"][0, m], int(sh["volume"][0, m]))
        assert int(sh["shape_idx"][0, m]) in mins
        assert int(np.prod(edges[sh["shape_idx"][0, m]])) == sh["volume"][0, m]


# ----------------------------------------------------------------------------- block order


def test_permutation_is_a_bijection_with_boxes():
    """Block order reading: each block's tokens are exactly the tokens of one b_T x b_H x b_W
    box of its zone; positions form a bijection; inverse after forward is the identity."""
    T, H, W = 16, 16, 24
    Z = 2 * 2 * 3
    rng = np.random.default_rng(2)
    shape_idx = rng.integers(0, 16, size=(2, Z)).astype(np.uint8)
    pos, bs, nb = oracle.block_layout(T, H, W, shape_idx)
    edges, vol = oracle.candidates()
    N = T * H * W
    for grp in range(2):
        assert np.array_equal(np.sort(pos[grp]), np.arange(N))
        assert nb[grp] == int((512 // vol[shape_idx[grp]]).sum())
        assert bs[grp, 0] == 0 and bs[grp, nb[grp]] == N and (bs[grp, nb[grp]:] == N).all()
        inv = np.empty(N, np.int64)
        inv[pos[grp]] = np.arange(N)
        t, h, w = inv // (H * W), (inv // W) % H, inv % W
        for j in range(nb[grp]):
            rows = np.arange(bs[grp, j], bs[grp, j + 1])
            zone = rows[0] // 512
            assert (rows // 512 == zone).all()
            bT, bH, bW = edges[shape_idx[grp, zone]]
            assert len(rows) == bT * bH * bW
            tt, hh, ww = t[rows], h[rows], w[rows]
            # a box: the right extent on each axis, aligned to the edge inside the zone
            assert len(np.unique(tt)) == bT and len(np.unique(hh)) == bH and len(np.unique(ww)) == bW
            assert tt.min() % bT == 0 and hh.min() % bH == 0 and ww.min() % bW == 0
            # raster order inside the block
            assert (np.diff(inv[rows]) > 0).all()
    x = rng.standard_normal((N, 4, 8)).astype(np.float32)
    y = oracle.permute(x, pos, 4)
    assert np.array_equal(oracle.unpermute(y, pos, 4), x)


# ----------------------------------------------------------------------------- pooling


def test_pooling_constant_and_mass():
    """RG M3 mean-pooled representatives: a constant block pools to the constant; the sizes
    times the means add up to the sum of all rows."""
    T, H, W = 8, 16, 16
    rng = np.random.default_rng(4)
    shape_idx = rng.integers(0, 16, size=(1, 4)).astype(np.uint8)
    pos, bs, nb = oracle.block_layout(T, H, W, shape_idx)
    N = T * H * W
    x = rng.standard_normal((2, N, 16)).astype(np.float32)
    xbar = oracle.pool(x, bs, nb, 1)
    sizes = np.diff(bs[0])[: nb[0]]
    np.testing.assert_allclose((sizes[None, :, None] * xbar[:, : nb[0]]).sum(1), x.astype(np.float64).sum(1),
                               rtol=1e-12, atol=1e-9)
    assert (xbar[:, nb[0]:] == 0).all()
    c = np.full((2, N, 16), 0.375, np.float32)
    np.testing.assert_allclose(oracle.pool(c, bs, nb, 1)[:, : nb[0]], 0.375, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- selection


def _layout_for(cfg):
    inp = synth.make_inputs(cfg)
    return inp, oracle.forward_path(inp)


def test_select_p0_is_plain_topk():
    """RG M3 attended-set equation with p = 0: the Top-p part is empty, so S_i is the
    Top-k of the block scores (independent numpy ranking, stable on ties)."""
    cfg = synth.CONFIGS["tiny"].replace(p=0.0, k_abs=5)
    inp, r = _layout_for(cfg)
    nb = int(r["nblocks"][0])
    s = np.einsum("hid,hjd->hij", r["qbar"][:, :nb], r["kbar"][:, :nb]) * cfg.sm_scale
    for h in range(cfg.heads):
        for i in range(nb):
            order = np.argsort(-s[h, i], kind="stable")
            assert r["sel_count"][h, i] == 5
            assert set(r["sel_idx"][h, i, :5].tolist()) == set(order[:5].tolist())


def test_select_k_all_and_sizes_and_monotone():
    """k = N_b selects every block; |S_i| = max(k, n_p); S_i grows with k and with p."""
    base = synth.CONFIGS["tiny"].replace(gamma=2.0)
    inp = synth.make_inputs(base)
    r = oracle.forward_path(inp)
    nb = int(r["nblocks"][0])
    cnt, idx, info = oracle.select(r["qbar"], r["kbar"], r["nblocks"], 1, base.sm_scale, nb, 0, 0.5)
    assert (cnt[:, :nb] == nb).all()
    prev = None
    for k, p in [(1, 0.3), (2, 0.3), (2, 0.6), (4, 0.6), (4, 0.95)]:
        cnt, idx, info = oracle.select(r["qbar"], r["kbar"], r["nblocks"], 1, base.sm_scale, k, 0, p)
        assert (cnt[:, :nb] == np.maximum(info[:, :nb, 0], info[:, :nb, 1])).all()
        sets = [[set(idx[h, i, : cnt[h, i]].tolist()) for i in range(nb)] for h in range(2)]
        for h in range(2):
            for i in range(nb):
                row = idx[h, i, : cnt[h, i]]
                assert (np.diff(row) > 0).all()  # stored ascending
                if prev is not None:
                    assert prev[h][i] <= sets[h][i]
        prev = sets


def test_select_uniform_probabilities():
    """Q-bar = 0 makes every block probability 1/N_b, so n_p = ceil(p N_b); ties resolve to the
    lowest block indices."""
    nbv = 32
    qbar = np.zeros((1, nbv, 8))
    kbar = np.random.default_rng(1).standard_normal((1, nbv, 8))
    for p in (0.1, 0.33, 0.9):
        cnt, idx, info = oracle.select(qbar, kbar, np.array([nbv], np.int32), 1, 1.0, 1, 0, p)
        n_p = math.ceil(p * nbv)
        assert (cnt[0] == n_p).all()
        assert (idx[0, :, :n_p] == np.arange(n_p)).all()


def test_select_k_from_fraction():
    """README's bsa_sparsity s keeps a fraction 1 - s of key blocks: k = ceil(k_frac N_b)."""
    nbv = 40
    rng = np.random.default_rng(8)
    qbar, kbar = rng.standard_normal((1, nbv, 8)), rng.standard_normal((1, nbv, 8))
    for frac, expect in [(0.05, 2), (0.25, 10), (0.26, 11), (0.0001, 1)]:
        cnt, idx, info = oracle.select(qbar, kbar, np.array([nbv], np.int32), 1, 1.0, 0, frac, 0.0)
        assert (cnt[0] == expect).all() and (info[0, :, 0] == expect).all()


# ----------------------------------------------------------------------------- attention


def _torch_masked_attention(q, k, v, mask, scale):
    import torch

    qt, kt, vt = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    s = torch.einsum("hnd,hmd->hnm", qt, kt) * scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return torch.softmax(s, dim=-1) @ vt, lse


def _token_mask(r, heads, N):
    bs, nb = r["block_start"][0], int(r["nblocks"][0])
    blk = np.searchsorted(bs[: nb + 1], np.arange(N), side="right") - 1
    mask = np.zeros((heads, N, N), bool)
    for h in range(heads):
        for i in range(nb):
            keys = np.zeros(N, bool)
            for j in r["sel_idx"][h, i, : r["sel_count"][h, i]]:
                keys[bs[j]:bs[j + 1]] = True
            mask[h, bs[i]:bs[i + 1]] = keys[None]
    return mask, blk


def test_attention_all_blocks_is_dense_sdpa():
    """All key blocks selected: the sparse attention must equal dense attention
    (torch scaled_dot_product_attention, fp64, CPU)."""
    import torch

    cfg = synth.CONFIGS["tiny"]
    inp, r = _layout_for(cfg)
    nb = int(r["nblocks"][0])
    cnt = np.zeros_like(r["sel_count"])
    cnt[:, :nb] = nb
    idx = np.zeros_like(r["sel_idx"])
    idx[:, :nb, :nb] = np.arange(nb)
    vp = oracle.permute(inp["v"], r["pos"], cfg.heads)
    o, lse = oracle.attn_fwd(r["qp"], r["kp"], vp, r["block_start"], r["nblocks"], 1, cnt, idx, cfg.sm_scale)
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)) for x in (r["qp"], r["kp"], vp))
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], scale=cfg.sm_scale)[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-10)
    s = torch.einsum("hnd,hmd->hnm", q, k) * cfg.sm_scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-12, atol=1e-10)


def test_attention_sparse_equals_masked_dense():
    """RG M3 online-softmax attention solely across S_i equals dense attention under the
    token-level mask built from the block lists; O stays in the hull of the attended V."""
    cfg = synth.CONFIGS["tiny"].replace(gamma=4.0)
    inp, r = _layout_for(cfg)
    vp = oracle.permute(inp["v"], r["pos"], cfg.heads)
    o, lse = oracle.attn_fwd(r["qp"], r["kp"], vp, r["block_start"], r["nblocks"], 1, r["sel_count"],
                             r["sel_idx"], cfg.sm_scale)
    mask, _ = _token_mask(r, cfg.heads, cfg.N)
    ref, rlse = _torch_masked_attention(r["qp"], r["kp"], vp, mask, cfg.sm_scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(lse, rlse.numpy(), rtol=1e-12, atol=1e-10)
    vmax = np.where(mask[..., None], vp[:, None, :, :], -np.inf).max(2)
    vmin = np.where(mask[..., None], vp[:, None, :, :], np.inf).min(2)
    assert (o <= vmax + 1e-9).all() and (o >= vmin - 1e-9).all()


def test_attention_backward_matches_autograd_and_finite_differences():
    """Gradient with the selection held constant: torch autograd (fp64) of the masked dense
    attention, and central finite differences of the oracle's own forward."""
    import torch

    cfg = synth.CONFIGS["tiny"].replace(gamma=4.0)
    inp = synth.make_inputs(cfg, with_dout=True)
    r = oracle.forward_path(inp)
    vp = oracle.permute(inp["v"], r["pos"], cfg.heads)
    dop = oracle.permute(inp["dout"], r["pos"], cfg.heads)
    g = oracle.attn_bwd(r["qp"], r["kp"], vp, dop, r["block_start"], r["nblocks"], 1, r["sel_count"],
                        r["sel_idx"], cfg.sm_scale)
    mask, _ = _token_mask(r, cfg.heads, cfg.N)
    q, k, v = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (r["qp"], r["kp"], vp))
    s = torch.einsum("hnd,hmd->hnm", q, k) * cfg.sm_scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(s, -1) @ v
    o.backward(torch.from_numpy(np.asarray(dop, np.float64)))
    np.testing.assert_allclose(g["dq"], q.grad.numpy(), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(g["dk"], k.grad.numpy(), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(g["dv"], v.grad.numpy(), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(g["delta"], (o.detach().numpy() * dop).sum(-1), rtol=1e-10, atol=1e-10)

    # finite differences of L = sum(dO * O) at a few coordinates (float64 copies)
    def loss(qq, kk, vv):
        oo, _ = oracle.attn_fwd(qq, kk, vv, r["block_start"], r["nblocks"], 1, r["sel_count"], r["sel_idx"],
                                cfg.sm_scale)
        return float((oo * dop).sum())

    rng = np.random.default_rng(0)
    h_ = 1e-2  # inputs go through float32; use a step whose rounding is exact
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        for _ in range(3):
            hh, n, e = rng.integers(cfg.heads), rng.integers(cfg.N), rng.integers(cfg.d)
            base = {"q": r["qp"].copy(), "k": r["kp"].copy(), "v": vp.copy()}
            plus = {kk: vv.copy() for kk, vv in base.items()}
            minus = {kk: vv.copy() for kk, vv in base.items()}
            plus[name][hh, n, e] += h_
            minus[name][hh, n, e] -= h_
            step = (plus[name][hh, n, e] - minus[name][hh, n, e])
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / step
            assert fd == pytest.approx(grad[hh, n, e], rel=2e-3, abs=2e-5)


# ------------------------------------------------ attention by whole-block products (attn_rows)


def test_attn_rows_matches_autograd_of_masked_dense():
    """oracle/attn_rows.py (the matrix-product form used for large key blocks) against torch
    autograd of dense attention under the token mask of the block lists (fp64): O, LSE, dQ of
    every query block and dK, dV of every key block."""
    import torch

    from oracle import attn_rows

    cfg = synth.CONFIGS["tiny"].replace(gamma=4.0)
    inp = synth.make_inputs(cfg, with_dout=True)
    r = oracle.forward_path(inp)
    vp = oracle.permute(inp["v"], r["pos"], cfg.heads)
    dop = oracle.permute(inp["dout"], r["pos"], cfg.heads)
    mask, _ = _token_mask(r, cfg.heads, cfg.N)
    q, k, v = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (r["qp"], r["kp"], vp))
    s = torch.einsum("hnd,hmd->hnm", q, k) * cfg.sm_scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    lse = torch.logsumexp(s, -1)
    o = torch.softmax(s, -1) @ v
    o.backward(torch.from_numpy(np.asarray(dop, np.float64)))
    bs, nb = r["block_start"][0], int(r["nblocks"][0])
    for h in range(cfg.heads):
        H = attn_rows.Head(r["qp"], r["kp"], vp, dop, bs, nb, r["sel_count"], r["sel_idx"], h, cfg.sm_scale)
        for i in range(nb):
            rows, oi, li = H.fwd(i)
            np.testing.assert_allclose(oi, o.detach().numpy()[h, rows], rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(li, lse.detach().numpy()[h, rows], rtol=1e-12, atol=1e-10)
            rows, dq = H.dq(i)
            np.testing.assert_allclose(dq, q.grad.numpy()[h, rows], rtol=1e-9, atol=1e-9)
        for j in range(nb):
            rows, dk, dv = H.dkdv(j)
            np.testing.assert_allclose(dk, k.grad.numpy()[h, rows], rtol=1e-9, atol=1e-9)
            np.testing.assert_allclose(dv, v.grad.numpy()[h, rows], rtol=1e-9, atol=1e-9)


def test_attn_rows_matches_c_oracle_on_mixed_volumes():
    """The matrix-product form against the C oracle's per-row loops on a bf16-exact layout with
    64-, 128- and 256-row blocks and Top-p-extended lists, on sampled query and key blocks."""
    from oracle import attn_rows

    cfg = synth.Config("mixed", 8, 16, 32, 2, 64, "bf16", blobs=1, k_abs=0, k_frac=0.1, p=0.9, backward=True,
                       seed=3101, gamma=8.0)
    inp = synth.make_inputs(cfg, with_dout=True)
    r = oracle.forward_path(inp)
    vols = np.array([64] * 7 + [128] * 6 + [256] * 3)[r["shapes"]["shape_idx"]]
    assert len(np.unique(vols)) >= 2
    vp = oracle.permute(inp["v"], r["pos"], cfg.heads)
    dop = oracle.permute(inp["dout"], r["pos"], cfg.heads)
    g = oracle.attn_bwd(r["qp"], r["kp"], vp, dop, r["block_start"], r["nblocks"], 1, r["sel_count"],
                        r["sel_idx"], cfg.sm_scale)
    of, lf = oracle.attn_fwd(r["qp"], r["kp"], vp, r["block_start"], r["nblocks"], 1, r["sel_count"], r["sel_idx"],
                             cfg.sm_scale)
    bs, nb = r["block_start"][0], int(r["nblocks"][0])
    for h in range(cfg.heads):
        H = attn_rows.Head(r["qp"], r["kp"], vp, dop, bs, nb, r["sel_count"], r["sel_idx"], h, cfg.sm_scale)
        col = attn_rows.selector_counts(r["sel_count"], r["sel_idx"], nb, h)
        for i in range(0, nb, 3):
            rows, oi, li = H.fwd(i)
            np.testing.assert_allclose(oi, of[h, rows], rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(li, lf[h, rows], rtol=1e-12, atol=1e-10)
            rows, dq = H.dq(i)
            np.testing.assert_allclose(dq, g["dq"][h, rows], rtol=1e-9, atol=1e-9)
        for j in range(0, nb, 3):
            assert len(H.selectors(j)) == col[j]
            rows, dk, dv = H.dkdv(j)
            np.testing.assert_allclose(dk, g["dk"][h, rows], rtol=1e-9, atol=1e-9)
            np.testing.assert_allclose(dv, g["dv"][h, rows], rtol=1e-9, atol=1e-9)
