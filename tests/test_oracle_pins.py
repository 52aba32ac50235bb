"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is a closed
form, a hand-worked fixture under tests/golden/, a brute-force search, a
library routine solving the same problem another way, or an invariant.
CPU only.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------- audio norm map

def test_norm_map_pythagorean_rows():
    # integer rows with integer norms: (3,4)->5, (5,12)->13, (8,15)->17, (1,2,2)->3
    H = np.zeros((5, 6))
    H[0, :2] = (3, 4)
    H[1, 2:4] = (5, 12)
    H[2, [0, 5]] = (8, -15)
    H[3, 1:4] = (1, -2, 2)
    norms, a = orc.audio_norm_map(H)
    assert norms.tolist() == [5.0, 13.0, 17.0, 3.0, 0.0]
    want = [float(np.float32(k / 17)) for k in (5, 13, 17, 3, 0)]      # closed forms k/17
    assert a.dtype == np.float32 and a.tolist() == want
    assert a[2] == 1.0                                  # the largest token maps to 1


def test_norm_map_constant_and_one_hot_rows():
    C = 64
    H = np.zeros((3, C))
    H[0] = 1.0                                          # sqrt(64) = 8
    H[1, 17] = -2.5                                     # one-hot: |value|
    H[2] = 0.5                                          # 0.5 sqrt(64) = 4
    norms, a = orc.audio_norm_map(H)
    assert norms.tolist() == [8.0, 2.5, 4.0]
    assert a.tolist() == [1.0, 0.3125, 0.5]


def test_norm_map_matches_hypot_and_is_sign_and_scale_invariant():
    rng = np.random.default_rng(5)
    H = rng.standard_normal((40, 24)) * rng.uniform(0.01, 3.0, size=(40, 1))
    norms, a = orc.audio_norm_map(H)
    ref = np.array([math.hypot(*row) for row in H])       # a different library routine
    np.testing.assert_allclose(norms, ref, rtol=1e-14)
    assert int(np.argmax(a)) == int(np.argmax(ref)) and a.max() == 1.0
    assert (orc.audio_norm_map(-H)[1] == a).all()
    assert (orc.audio_norm_map(H * 2.0 ** 7)[1] == a).all()   # powers of two scale exactly
    _, a_chunked = orc.audio_norm_map(H, chunk=7)
    assert (a_chunked == a).all()


def test_norm_map_degenerate_inputs():
    _, a = orc.audio_norm_map(np.zeros((10, 8)))
    assert a.dtype == np.float32 and (a == 0).all()      # an all-zero clip stays zero
    norms, a = orc.audio_norm_map(np.zeros((0, 8)))
    assert norms.shape == (0,) and a.shape == (0,)


# ---------------------------------------------------------------- candidates

def test_candidate_set_matches_hand_typed_table():
    rows = [list(map(int, r.split())) for r in _read_rows("candidate_shapes.txt")]
    want = [tuple(r[2:]) for r in rows]
    got = orc.candidate_shapes()
    assert len(got) == 16                                     # the pages' count
    assert got == want
    for (idx, B, bt, bh, bw), s in zip(rows, got):
        assert bt * bh * bw == B and 8 % bt == 0 and 8 % bh == 0 and 8 % bw == 0


def test_candidate_set_is_every_power_of_two_box_without_unit_edges():
    boxes = {(2 ** a, 2 ** b, 2 ** c) for a, b, c in itertools.product(range(4), repeat=3)
             if 2 ** (a + b + c) in (64, 128, 256)}
    with_unit = {s for s in boxes if 1 in s}
    assert len(boxes) == 19 and len(with_unit) == 3
    assert set(orc.candidate_shapes()) == boxes - with_unit


# ---------------------------------------------------------------- E3 optimum

@pytest.mark.parametrize("seed", range(6))
def test_optimum_solves_the_constrained_minimisation(seed):
    """E3 is the minimiser of sum_d g_d (b_d^2 - 1) subject to prod_d b_d = B.
    Solve that problem numerically (SLSQP) and compare."""
    from scipy.optimize import minimize
    rng = np.random.default_rng(seed)
    g = np.exp(rng.uniform(-6, 3, size=3))
    for B in (64, 128, 256):
        S = math.log2(B)
        obj = lambda x: float(np.sum(g * (np.exp2(2 * np.clip(x, -60, 60)) - 1)))
        con = {"type": "eq", "fun": lambda x: float(np.sum(x) - S)}
        res = minimize(obj, x0=np.full(3, S / 3), constraints=[con], method="SLSQP",
                       options={"ftol": 1e-14, "maxiter": 500})
        assert res.success
        ls = orc.optimum_log2(g[None, :], np.array([B]))[0]
        np.testing.assert_allclose(ls, res.x, atol=2e-5)
        assert abs(ls.sum() - S) < 1e-12                      # the product constraint
        # b*_d proportional to g_d^(-1/2)
        ratio = np.exp2(ls) * np.sqrt(g)
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)


def test_optimum_is_scale_invariant():
    rng = np.random.default_rng(7)
    g = np.exp(rng.uniform(-5, 2, size=(50, 3)))
    B = rng.choice([64, 128, 256], size=50)
    a = orc.optimum_log2(g, B)
    b = orc.optimum_log2(g * 37.5, B)
    np.testing.assert_allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------- shape choice

def _frac(s):
    return Fraction(s)


def test_hand_worked_shapes():
    for row in _read_rows("hand_worked_shapes.txt"):
        gpart, lpart, spart, dpart = [p.split() for p in row.split("|")]
        g = np.array([float(x) for x in gpart[:3]])
        B = int(gpart[3])
        lstar_hand = [float(_frac(x)) for x in lpart]
        shape_hand = tuple(int(x) for x in spart)
        ls = orc.optimum_log2(g[None, :], np.array([B]))[0]
        np.testing.assert_allclose(ls, lstar_hand, atol=1e-12)
        idx, _ = orc.nearest_shape(ls, B)
        assert orc.candidate_shapes()[idx] == shape_hand, row
        D = sum((math.log2(shape_hand[d]) - lstar_hand[d]) ** 2 for d in range(3))
        assert abs(D - float(_frac(dpart[0]))) < 1e-12


def test_rounding_ties_fall_in_the_window():
    """g = (1+1e-6, 1e-6, 1e-6), B = 64: (2,4,8) and (2,8,4) are equidistant in exact
    arithmetic (l*_H = l*_W) but their float64 distances differ in the last bits;
    the tie window must still pick the lower index."""
    ls = orc.optimum_log2(np.array([[1 + 1e-6, 1e-6, 1e-6]]), np.array([64]))[0]
    assert ls[1] == ls[2]
    idx, _ = orc.nearest_shape(ls, 64)
    assert orc.candidate_shapes()[idx] == (2, 4, 8)
    ls = orc.optimum_log2(np.array([[1e-6, 1e-6, 1 + 1e-6]]), np.array([128]))[0]
    idx, _ = orc.nearest_shape(ls, 128)
    assert orc.candidate_shapes()[idx] == (8, 8, 2)


def test_nearest_shape_brute_force():
    """Over random optima: the pick is at the minimum distance over every box of
    the volume (enumerated here as exponent triples), and no lower-index
    candidate lies within the window."""
    rng = np.random.default_rng(3)
    cands = orc.candidate_shapes()
    for _ in range(400):
        B = int(rng.choice([64, 128, 256]))
        S = int(math.log2(B))
        ls = rng.normal(S / 3, 1.5, size=3)
        trip = [(a, b, c) for a in (1, 2, 3) for b in (1, 2, 3) for c in (1, 2, 3) if a + b + c == S]
        dist = {t: sum((t[d] - ls[d]) ** 2 for d in range(3)) for t in trip}
        Dmin = min(dist.values())
        idx, _ = orc.nearest_shape(ls, B)
        pick = tuple(int(math.log2(x)) for x in cands[idx])
        assert abs(dist[pick] - Dmin) <= 1e-9
        for j in range(idx):
            s = cands[j]
            if s[0] * s[1] * s[2] == B:
                t = tuple(int(math.log2(x)) for x in s)
                assert dist[t] > Dmin + 1e-9


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_fast_axis_gets_the_finest_edge(axis):
    """A zone that varies only along one axis, with no audio coupling, gets the
    smallest edge that its volume offers on that axis: 2 at volumes 64 and 128,
    4 at 256 ([P3] core ideas: finer partition along fast-changing axes)."""
    r = np.zeros((1, 3))
    r[0, axis] = 1.0
    g = orc.indicator(r, np.zeros(1), np.full((1, 3), 1 / 3))
    for B, edge in ((64, 2), (128, 2), (256, 4)):
        idx, _ = orc.nearest_shape(orc.optimum_log2(g, np.array([B]))[0], B)
        assert orc.candidate_shapes()[idx][axis] == edge


# ---------------------------------------------------------------- statistics (E1)

def _grid_values(T, H, W, C, fn):
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    vals = fn(t.reshape(-1), h.reshape(-1), w.reshape(-1))
    return np.repeat(vals[:, None], C, axis=1) if vals.ndim == 1 else vals


def test_variance_of_a_field_varying_only_along_T():
    T, H, W, C = 16, 8, 16, 5
    rng = np.random.default_rng(0)
    f = rng.normal(size=T)
    u = rng.normal(size=C)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    V = f[t.reshape(-1)][:, None] * u[None, :]
    s2, r = orc.video_variance(orc.axis_profiles(V, T, H, W))
    # the H and W slices hold identical values: only rounding of their mean remains
    assert np.all(s2[:, 1] < 1e-28) and np.all(s2[:, 2] < 1e-28)
    np.testing.assert_allclose(r, np.tile([1.0, 0.0, 0.0], (len(r), 1)), atol=1e-25)
    # closed form of sigma2_T per zone: mean_c u_c^2 * population variance of f over the zone's 8 slices
    for zt in range(T // 8):
        fz = f[8 * zt:8 * zt + 8]
        want = np.mean(u ** 2) * np.mean((fz - fz.mean()) ** 2)
        for m in range(len(r)):
            if m // ((H // 8) * (W // 8)) == zt:
                assert abs(s2[m, 0] - want) < 1e-12 * max(1.0, want)


def test_alternating_slices_have_unit_variance():
    V = _grid_values(8, 8, 8, 3, lambda t, h, w: np.where(t % 2 == 0, 1.0, -1.0))
    s2, r = orc.video_variance(orc.axis_profiles(V, 8, 8, 8))
    assert s2[0, 0] == 1.0 and s2[0, 1] == 0.0 and s2[0, 2] == 0.0
    assert tuple(r[0]) == (1.0, 0.0, 0.0)


def test_ramp_along_H_has_the_variance_of_0_to_7():
    V = _grid_values(8, 16, 8, 4, lambda t, h, w: (h % 8).astype(float))
    s2, _ = orc.video_variance(orc.axis_profiles(V, 8, 16, 8))
    np.testing.assert_allclose(s2[:, 1], 5.25, atol=1e-12)       # (8^2 - 1) / 12
    assert np.all(s2[:, 0] < 1e-28) and np.all(s2[:, 2] < 1e-28)


def test_variance_averages_over_channels():
    """Half the channels alternate along T, half along W: each axis carries the
    channel-average, 1/2 (the 1/D factor of E1)."""
    t, h, w = np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij")
    a = np.where(t.reshape(-1) % 2 == 0, 1.0, -1.0)
    b = np.where(w.reshape(-1) % 2 == 0, 1.0, -1.0)
    V = np.stack([a, a, b, b], axis=1)
    s2, r = orc.video_variance(orc.axis_profiles(V, 8, 8, 8))
    assert tuple(s2[0]) == (0.5, 0.0, 0.5)
    assert tuple(r[0]) == (0.5, 0.0, 0.5)


def test_constant_zone_falls_back_to_thirds():
    V = np.full((512, 3), 2.5)
    s2, r = orc.video_variance(orc.axis_profiles(V, 8, 8, 8))
    assert np.all(s2 == 0) and np.all(r == 1.0 / 3.0)


def test_iid_noise_is_isotropic():
    rng = np.random.default_rng(5)
    V = rng.normal(size=(8 * 8 * 8, 4096))
    s2, r = orc.video_variance(orc.axis_profiles(V, 8, 8, 8))
    np.testing.assert_allclose(r[0], 1 / 3, atol=0.02)
    np.testing.assert_allclose(s2[0], 7 / 8 / 64, rtol=0.05)     # E[(1/8)sum(mean64 - mean)^2] = (7/8)/64


def test_zone_mean_is_the_same_along_every_axis():
    rng = np.random.default_rng(9)
    V = rng.normal(size=(16 * 8 * 8, 7))
    P = orc.axis_profiles(V, 16, 8, 8)
    mu = P.mean(axis=2)                                           # [nZ, 3, C]
    np.testing.assert_allclose(mu[:, 0], mu[:, 1], atol=1e-14)
    np.testing.assert_allclose(mu[:, 0], mu[:, 2], atol=1e-14)
    np.testing.assert_allclose(mu[0, 0], V[orc.permutation(16, 8, 8, [3, 3])[:512]].mean(axis=0), atol=1e-14)


def test_zone_order_is_raster():
    """Zone m = (zt*nH + zh)*nW + zw: mark each zone by a constant value."""
    T, H, W = 16, 24, 8
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    mark = ((t // 8) * 3 + (h // 8)) * 1 + (w // 8)
    V = mark.reshape(-1, 1).astype(float)
    P = orc.axis_profiles(V, T, H, W)
    np.testing.assert_array_equal(P[:, 0, 0, 0], np.arange(6))


# ---------------------------------------------------------------- audio terms (readings)

def test_audio_constant_map():
    a = np.full(512, 0.3)
    abar, s2, vhat = orc.audio_terms(a, 8, 8, 8)
    assert abs(abar[0] - 0.3) < 1e-15 and np.all(s2 == 0) and np.all(vhat == 1 / 3)


def test_audio_ramp_along_W():
    t, h, w = np.meshgrid(np.arange(8), np.arange(8), np.arange(8), indexing="ij")
    a = (w.reshape(-1) / 7.0)
    abar, s2, vhat = orc.audio_terms(a, 8, 8, 8)
    assert abs(abar[0] - 0.5) < 1e-15
    assert tuple(vhat[0]) == (0.0, 0.0, 1.0)
    assert abs(s2[0, 2] - 5.25 / 49) < 1e-15


def test_indicator_is_E2():
    r = np.array([[0.2, 0.3, 0.5]])
    vhat = np.array([[0.1, 0.6, 0.3]])
    g = orc.indicator(r, np.array([0.5]), vhat, eps=1e-6)
    np.testing.assert_allclose(g[0], [0.2 + 0.05 + 1e-6, 0.3 + 0.3 + 1e-6, 0.5 + 0.15 + 1e-6], atol=1e-15)


# ---------------------------------------------------------------- volume and density

def test_volume_thresholds():
    rho = np.array([0.0, 0.2499999, 0.25, 0.3, 0.4999999, 0.5, 0.9, 1.0])
    np.testing.assert_array_equal(orc.volume(rho), [256, 256, 128, 128, 128, 64, 64, 64])


def test_density_properties():
    """Static zone with weak coupling -> 256; strong coupling -> 64; the most
    varying zone -> 64 ([P2] step 2, [P3] §2)."""
    s2 = np.array([[1e-6, 1e-6, 1e-6], [1.0, 2.0, 0.5], [1e-6, 0.0, 0.0], [0.1, 0.1, 0.1]])
    abar = np.array([0.1, 0.0, 0.7, 0.3])
    rho, S = orc.density(s2, abar)
    np.testing.assert_array_equal(orc.volume(rho), [256, 64, 64, 128])
    assert rho[1] == 1.0


# ---------------------------------------------------------------- layout and permutation

def test_block_layout_counts():
    offs, NB = orc.block_layout([3, 7, 13])          # volumes 64, 128, 256
    assert NB == 8 + 4 + 2
    np.testing.assert_array_equal(np.diff(offs), [64] * 8 + [128] * 4 + [256] * 2)
    assert offs[8] == 512 and offs[12] == 1024 and offs[-1] == 1536


def test_permutation_hand_worked_first_block():
    """Zone 0 of an 8x8x8 grid with shape (2,4,8): the first block holds
    t in {0,1}, h in 0..3, w in 0..7 in raster order; the second block starts at
    h = 4."""
    pi = orc.permutation(8, 8, 8, [0])
    want = [(t * 8 + h) * 8 + w for t in range(2) for h in range(4) for w in range(8)]
    np.testing.assert_array_equal(pi[:64], want)
    np.testing.assert_array_equal(pi[64:72], [(0 * 8 + 4) * 8 + w for w in range(8)])


@pytest.mark.parametrize("seed", range(3))
def test_permutation_properties(seed):
    rng = np.random.default_rng(seed)
    T, H, W = 16, 24, 16
    nZ = (T // 8) * (H // 8) * (W // 8)
    shapes = rng.integers(0, 16, size=nZ)
    pi = orc.permutation(T, H, W, shapes)
    N = T * H * W
    assert np.array_equal(np.sort(pi), np.arange(N))             # bijection
    X = rng.normal(size=(N, 3))
    np.testing.assert_array_equal(orc.to_raster(orc.to_block_major(X, pi), pi), X)
    offs, NB = orc.block_layout(shapes)
    cands = orc.candidate_shapes()
    zone_of_block = np.repeat(np.arange(nZ), [512 // np.prod(cands[s]) for s in shapes])
    for i in range(NB):
        toks = pi[offs[i]:offs[i + 1]]
        t, rem = np.divmod(toks, H * W)
        h, w = np.divmod(rem, W)
        bt, bh, bw = cands[shapes[zone_of_block[i]]]
        # contiguous axis-aligned box of the zone's shape, tokens in raster order
        assert (t.max() - t.min() + 1, h.max() - h.min() + 1, w.max() - w.min() + 1) == (bt, bh, bw)
        assert t.min() % bt == 0 and h.min() % bh == 0 and w.min() % bw == 0
        assert np.all(np.diff(toks) > 0)
        assert offs[i] // 512 == zone_of_block[i]


# ---------------------------------------------------------------- pooling and scores

def test_pool_blocks_is_the_block_mean():
    N, d = 1024, 3
    offs = np.array([0, 64, 128, 256, 512, 1024])
    X = np.arange(N * d, dtype=float).reshape(N, 1, d)
    Pb = orc.pool_blocks(X, offs, 0)
    for i in range(len(offs) - 1):
        a, b = offs[i], offs[i + 1]
        first = (a + b - 1) / 2 * d                               # mean row index * d
        np.testing.assert_allclose(Pb[i], first + np.arange(d), atol=1e-12)


def test_block_logits_round_once_to_float32():
    Qb = np.array([[1.0, 2.0, 0.0], [0.5, -1.0, 3.0]])
    Kb = np.array([[2.0, 1.0, 1.0], [0.0, 0.0, 4.0]])
    s = 0.125
    L = orc.block_logits(Qb, Kb, s)
    assert L.dtype == np.float32
    np.testing.assert_array_equal(L, np.array([[0.5, 0.0], [0.375, 1.5]], dtype=np.float32))
    # a value that is not a float32: 1/3 must be the nearest float32
    L = orc.block_logits(np.array([[1.0]]), np.array([[1.0 / 3.0]]), 1.0)
    assert L[0, 0] == np.float32(1.0 / 3.0)


# ---------------------------------------------------------------- selection (E4)

def _brute_select(L, k, p):
    """E4 by enumeration: Top-k = the k highest-probability blocks (lower index
    first on ties); Top-p = among the smallest subsets whose probability reaches
    p, the one of largest mass (lexicographically lowest indices on ties)."""
    L = np.asarray(L, dtype=np.float64)
    NB = len(L)
    P = np.exp(L - L.max())
    P /= P.sum()
    rank = sorted(range(NB), key=lambda j: (-L[j], j))
    topk = set(rank[:min(k, NB)])
    topp = None
    for n in range(1, NB + 1):
        best = None
        for sub in itertools.combinations(range(NB), n):
            m = sum(P[j] for j in sub)
            if m >= p - 1e-12:
                key = (-m, sorted(rank.index(j) for j in sub))
                if best is None or key < best[0]:
                    best = (key, set(sub))
        if best is not None:
            topp = best[1]
            break
    if topp is None:
        topp = set(range(NB))
    return sorted(topk | topp)


@pytest.mark.parametrize("seed", range(40))
def test_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    NB = int(rng.integers(1, 10))
    L = rng.normal(scale=rng.choice([0.1, 1.0, 3.0]), size=NB).astype(np.float32)
    if seed % 5 == 0 and NB > 2:
        L[1] = L[0]                                           # an exact tie
    k = int(rng.integers(0, NB + 2))
    p = float(rng.choice([0.0, 0.3, 0.5, 0.9, 0.95, 1.0]))
    sel, flag = orc.select_row(L, k, p)
    if flag and p < 1.0:
        pytest.skip("row lies on a decision boundary")
    assert list(sel) == _brute_select(L, k, p)


def test_selection_invariants():
    rng = np.random.default_rng(11)
    for _ in range(200):
        NB = int(rng.integers(1, 300))
        L = rng.normal(scale=2.0, size=NB).astype(np.float32)
        k = int(rng.integers(0, 20))
        p = float(rng.uniform(0, 1))
        sel, flag = orc.select_row(L, k, p)
        P = np.exp(L.astype(float) - L.max())
        P /= P.sum()
        assert len(sel) >= min(k, NB)
        assert P[sel].sum() >= p - 1e-12
        if len(sel) > max(k, 1):
            rank = sorted(sel, key=lambda j: (-L[j], j))
            assert P[rank[:-1]].sum() < p + 1e-12
        others = np.setdiff1d(np.arange(NB), sel)
        if others.size:
            assert L[sel].min() >= L[others].max()


def test_selection_closed_forms():
    L = np.zeros(16, dtype=np.float32)                         # uniform scores
    sel, _ = orc.select_row(L, 0, 0.9)
    np.testing.assert_array_equal(sel, np.arange(15))          # ceil(0.9 * 16) = 15, lowest indices
    sel, _ = orc.select_row(L, 3, 0.0)
    np.testing.assert_array_equal(sel, [0, 1, 2])
    L = np.array([0.0, 5.0, 1.0, 5.0], dtype=np.float32)
    sel, _ = orc.select_row(L, 0, 0.0)
    np.testing.assert_array_equal(sel, [1])                    # argmax, lower index on the tie
    sel, _ = orc.select_row(L, 10, 0.5)
    np.testing.assert_array_equal(sel, [0, 1, 2, 3])           # k >= NB selects all


# ---------------------------------------------------------------- attention

def _tiny_case(seed=0, T=8, H=16, W=16, d=16, k=3, p=0.8):
    rng = np.random.default_rng(seed)
    N = T * H * W
    nZ = (T // 8) * (H // 8) * (W // 8)
    shapes = rng.integers(0, 16, size=nZ)
    pi = orc.permutation(T, H, W, shapes)
    offs, NB = orc.block_layout(shapes)
    Q, K, V, dO = (rng.normal(size=(N, 1, d)) for _ in range(4))
    Qp, Kp, Vp, dOp = (orc.to_block_major(X, pi) for X in (Q, K, V, dO))
    sc = 1.0 / math.sqrt(d)
    Lg = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
    co, ci, _ = orc.select(Lg, k, p)
    return dict(Q=Q, K=K, V=V, dO=dO, Qp=Qp, Kp=Kp, Vp=Vp, dOp=dOp, pi=pi, offs=offs,
                NB=NB, co=co, ci=ci, scale=sc, N=N, d=d)


def _mask(c):
    """Dense boolean token mask in raster order from the block CSR."""
    N, offs, pi = c["N"], c["offs"], c["pi"]
    Mp = np.zeros((N, N), dtype=bool)
    for i in range(c["NB"]):
        for j in c["ci"][c["co"][i]:c["co"][i + 1]]:
            Mp[offs[i]:offs[i + 1], offs[j]:offs[j + 1]] = True
    M = np.zeros_like(Mp)
    M[np.ix_(pi, pi)] = Mp
    return M


def test_forward_with_everything_selected_is_dense_sdpa():
    c = _tiny_case(k=10 ** 6)
    assert c["co"][-1] == c["NB"] ** 2
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"])
    O = orc.to_raster(out["O"], c["pi"])
    q, k, v = (torch.from_numpy(c[x][:, 0, :]).unsqueeze(0) for x in ("Q", "K", "V"))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(np.float32(c["scale"])))[0]
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    s = float(np.float32(c["scale"])) * (q[0] @ k[0].T)
    np.testing.assert_allclose(orc.to_raster(out["lse"], c["pi"]), torch.logsumexp(s, 1).numpy(), atol=1e-12)


def test_forward_equals_masked_dense_sdpa():
    c = _tiny_case(seed=1)
    M = _mask(c)
    assert 0 < M.mean() < 1
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"])
    q, k, v = (torch.from_numpy(c[x][:, 0, :]).unsqueeze(0) for x in ("Q", "K", "V"))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(M).unsqueeze(0), scale=float(np.float32(c["scale"])))[0]
    np.testing.assert_allclose(orc.to_raster(out["O"], c["pi"]), ref.numpy(), atol=1e-12)


def test_backward_equals_autograd_of_masked_dense_attention():
    c = _tiny_case(seed=2)
    M = torch.from_numpy(_mask(c))
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"], dOp=c["dOp"])
    q, k, v = (torch.from_numpy(c[x][:, 0, :]).clone().requires_grad_(True) for x in ("Q", "K", "V"))
    s = float(np.float32(c["scale"])) * (q @ k.T)
    s = s.masked_fill(~M, float("-inf"))
    o = torch.softmax(s, dim=1) @ v
    o.backward(torch.from_numpy(c["dO"][:, 0, :]))
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        np.testing.assert_allclose(orc.to_raster(out[name], c["pi"]), t.grad.numpy(), atol=1e-11)


def test_backward_by_finite_differences():
    """Central differences of <O, dO> against the oracle's own forward."""
    c = _tiny_case(seed=3, d=8)
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"], dOp=c["dOp"])

    def loss(Qp, Kp, Vp):
        o = orc.attention(Qp, Kp, Vp, c["offs"], c["co"], c["ci"], 0, c["scale"])["O"]
        return float(np.sum(o * c["dOp"][:, 0, :]))

    rng = np.random.default_rng(0)
    h = 1e-6
    for name, grad in (("Qp", "dQ"), ("Kp", "dK"), ("Vp", "dV")):
        for _ in range(4):
            r, col = int(rng.integers(0, c["N"])), int(rng.integers(0, c["d"]))
            args = {x: c[x] for x in ("Qp", "Kp", "Vp")}
            plus = args[name].copy()
            plus[r, 0, col] += h
            minus = args[name].copy()
            minus[r, 0, col] -= h
            fd = (loss(**{**args, name: plus}) - loss(**{**args, name: minus})) / (2 * h)
            assert abs(fd - out[grad][r, col]) < 1e-6 * max(1.0, abs(fd))


def test_key_block_grads_and_unselected_keys():
    c = _tiny_case(seed=4, H=32, W=32, k=1, p=0.05)
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"], dOp=c["dOp"])
    chosen = set(int(x) for x in c["ci"])
    offs = c["offs"]
    for j in range(c["NB"]):
        dk, dv = orc.key_block_grads(c["Qp"], c["Kp"], c["Vp"], c["dOp"], offs, c["co"], c["ci"], j, 0, c["scale"])
        np.testing.assert_allclose(dk, out["dK"][offs[j]:offs[j + 1]], atol=1e-12)
        np.testing.assert_allclose(dv, out["dV"][offs[j]:offs[j + 1]], atol=1e-12)
        if j not in chosen:
            assert not np.any(out["dK"][offs[j]:offs[j + 1]]) and not np.any(out["dV"][offs[j]:offs[j + 1]])
    assert len(chosen) < c["NB"]


def test_squared_product_terms_by_brute_force():
    """The summed squared products that the parity bars use, against explicit
    loops over every product of every gradient element: dQ[q,c] sums
    scale dS[q,t] K[t,c] over keys t, dK[t,c] sums scale dS[q,t] Q[q,c] over
    queries q, dV[t,c] sums P[q,t] dO[q,c] over queries q (torch autograd
    supplies P and dS independently of the oracle)."""
    c = _tiny_case(seed=6, H=8, W=8, d=4, k=2, p=0.5)
    M = torch.from_numpy(_mask(c))
    out = orc.attention(c["Qp"], c["Kp"], c["Vp"], c["offs"], c["co"], c["ci"], 0, c["scale"], dOp=c["dOp"])
    sc = float(np.float32(c["scale"]))
    q, k, v = (torch.from_numpy(c[x][:, 0, :]) for x in ("Q", "K", "V"))
    do = torch.from_numpy(c["dO"][:, 0, :])
    s = (sc * (q @ k.T)).masked_fill(~M, float("-inf")).requires_grad_(True)
    Pm = torch.softmax(s, dim=1)
    (Pm @ v).backward(do)
    P, dS = Pm.detach().numpy(), (s.grad / 1.0).numpy()     # dS = dL/ds (the score gradient before the scale)
    Q, K, dO = q.numpy(), k.numpy(), do.numpy()
    N, d = Q.shape
    tQ, tK, tV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for a in range(N):          # every (query a, key b) product, channels side by side
        for b in range(N):
            tQ[a] += (sc * dS[a, b] * K[b]) ** 2
            tK[b] += (sc * dS[a, b] * Q[a]) ** 2
            tV[b] += (P[a, b] * dO[a]) ** 2
    assert 0 < (P > 0).mean() < 1
    for name, want in (("tQ", tQ), ("tK", tK), ("tV", tV)):
        np.testing.assert_allclose(orc.to_raster(out[name], c["pi"]), want, rtol=1e-10, atol=1e-300)
    j = int(c["ci"][0])
    offs = c["offs"]
    _, _, tk, tv = orc.key_block_grads(c["Qp"], c["Kp"], c["Vp"], c["dOp"], offs, c["co"], c["ci"], j, 0,
                                       c["scale"], with_terms=True)
    np.testing.assert_allclose(tk, out["tK"][offs[j]:offs[j + 1]], rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(tv, out["tV"][offs[j]:offs[j + 1]], rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- end to end

def test_zone_shapes_on_a_designed_grid():
    """Four zones built so that the decision is known: zone 0 alternates along W
    only (finest W edge, full variance -> 64), zone 1 is constant with no audio
    (-> 256), zone 2 is constant but sits under strong audio coupling (-> 64),
    zone 3 alternates along T with a quarter of zone 0's variance and weak audio
    (rho = 0.25 -> 128)."""
    T, H, W = 8, 16, 16
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.reshape(-1), h.reshape(-1), w.reshape(-1)
    zone = (h // 8) * 2 + (w // 8)
    V = np.zeros(T * H * W)
    V[zone == 0] = np.where(w[zone == 0] % 2 == 0, 1.0, -1.0)
    V[zone == 1] = 0.7
    V[zone == 2] = -0.2
    V[zone == 3] = np.where(t[zone == 3] % 2 == 0, 0.5, -0.5)
    a = np.zeros(T * H * W)
    a[zone == 2] = 0.8
    a[zone == 3] = 0.1
    res = orc.zone_shapes(V[:, None].repeat(2, axis=1), a, T, H, W)
    np.testing.assert_array_equal(res["B"], [64, 256, 64, 128])
    np.testing.assert_allclose(res["rho"], [1.0, 0.0, 0.8, 0.25], atol=1e-15)
    cands = orc.candidate_shapes()
    assert cands[res["shape"][0]][2] == 2
    assert cands[res["shape"][3]][0] == 2
    assert res["NB"] == 8 + 2 + 8 + 4
    assert res["near_tie"][3]                              # rho sits exactly on tau256


# ---------------------------------------------------------------- next row f3: routing and the flat path

def test_sharpness_closed_forms():
    NB = 12
    L = np.zeros((4, NB))
    L[1, 5] = 1000.0                                      # one block takes all the mass
    L[2, :3] = math.log(2.0)                              # three blocks weigh twice the rest
    L[3] = np.arange(NB) * 0.0 + 7.0                      # constant row, shifted
    M = orc.block_sharpness(L)
    assert M[0] == 0.0 and M[3] == 0.0                    # uniform rows
    assert math.isclose(M[1], (NB - 1) / NB ** 2, rel_tol=1e-15)
    # two-level row: p_hot = 2/(NB+3), p_cold = 1/(NB+3), variance by exact rationals
    ph, pc, mu = Fraction(2, NB + 3), Fraction(1, NB + 3), Fraction(1, NB)
    want = (3 * (ph - mu) ** 2 + (NB - 3) * (pc - mu) ** 2) / NB
    assert math.isclose(M[2], float(want), rel_tol=1e-12)
    assert (orc.block_sharpness(L + 5.0) == M).all()     # a constant per row does not matter


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flat_route_is_a_stable_ranking(seed):
    rng = np.random.default_rng(seed)
    M = rng.integers(0, 6, size=40).astype(np.float64)   # many ties
    for ratio in (0.0, 0.1, 0.5, 0.99, 1.0):
        flat = orc.flat_route(M, ratio)
        n = int(math.floor(ratio * 40))
        want = np.zeros(40, dtype=bool)
        want[np.argsort(M, kind="stable")[:n]] = True     # stable: ties to the lower index
        assert (flat == want).all() and flat.sum() == n


def _constant_key_problem(seed):
    rng = np.random.default_rng(seed)
    offs = np.array([0, 64, 192, 256, 512, 576])
    N, d = offs[-1], 16
    Kp = np.empty((N, 1, d))
    for j in range(len(offs) - 1):
        Kp[offs[j]:offs[j + 1], 0] = rng.standard_normal(d)   # every key of block j equal
    Qp = rng.standard_normal((N, 1, d))
    Vp = rng.standard_normal((N, 1, d))
    return offs, Qp, Kp, Vp


def test_taylor_path_is_exact_when_keys_are_constant_per_block():
    offs, Qp, Kp, Vp = _constant_key_problem(3)
    sel, i, scale = [0, 2, 3], 1, 0.3
    o, lse = orc.taylor_attn_fwd_block(Qp, Kp, Vp, offs, sel, i, 0, scale)
    keys = np.concatenate([np.arange(offs[j], offs[j + 1]) for j in sel])
    q = torch.tensor(Qp[offs[i]:offs[i + 1], 0])[None, None]
    k = torch.tensor(Kp[keys, 0])[None, None]
    v = torch.tensor(Vp[keys, 0])[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(np.float32(scale)))[0, 0].numpy()
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)
    s = float(np.float32(scale)) * (q[0, 0].numpy() @ k[0, 0].numpy().T)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-12)


def test_taylor_path_with_a_zero_query_is_the_mean_value():
    offs, Qp, Kp, Vp = _constant_key_problem(4)
    rng = np.random.default_rng(9)
    Kp = rng.standard_normal(Kp.shape)                   # keys no longer constant: q = 0 ignores them
    Qp[offs[2]:offs[3]] = 0.0
    sel = [1, 4]
    o, lse = orc.taylor_attn_fwd_block(Qp, Kp, Vp, offs, sel, 2, 0, 0.25)
    keys = np.concatenate([np.arange(offs[j], offs[j + 1]) for j in sel])
    np.testing.assert_allclose(o, np.broadcast_to(Vp[keys, 0].mean(axis=0), o.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(len(keys)), rtol=1e-14)


def _torch_block_mean_attention(Q, K, V, offs, sel, i, scale):
    """Block-mean attention of query block i written directly on token tensors
    (the means are taken inside, so autograd reaches every token)."""
    q = Q[offs[i]:offs[i + 1]]
    kb = torch.stack([K[offs[j]:offs[j + 1]].mean(dim=0) for j in sel])
    vb = torch.stack([V[offs[j]:offs[j + 1]].mean(dim=0) for j in sel])
    cnt = torch.tensor([float(offs[j + 1] - offs[j]) for j in sel], dtype=torch.float64)
    w = torch.softmax(scale * (q @ kb.T) + torch.log(cnt)[None, :], dim=1)
    return w @ vb


def test_taylor_backward_matches_autograd():
    rng = np.random.default_rng(21)
    offs = np.array([0, 64, 192, 256, 512, 576])
    N, d = offs[-1], 8
    Qp, Kp, Vp, dOp = (rng.standard_normal((N, 1, d)) for _ in range(4))
    sel, i, scale = [0, 1, 3, 4], 2, 0.4
    dq, g = orc.taylor_attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, 0, scale)
    Q, K, V = (torch.tensor(x[:, 0], requires_grad=True) for x in (Qp, Kp, Vp))
    o = _torch_block_mean_attention(Q, K, V, offs, sel, i, float(np.float32(scale)))
    (o * torch.tensor(dOp[offs[i]:offs[i + 1], 0])).sum().backward()
    np.testing.assert_allclose(dq, Q.grad[offs[i]:offs[i + 1]].numpy(), rtol=1e-10, atol=1e-12)
    for j in sel:
        B = offs[j + 1] - offs[j]
        np.testing.assert_allclose(np.broadcast_to(g[j][0] / B, (B, d)), K.grad[offs[j]:offs[j + 1]].numpy(),
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(np.broadcast_to(g[j][1] / B, (B, d)), V.grad[offs[j]:offs[j + 1]].numpy(),
                                   rtol=1e-10, atol=1e-12)
    assert not K.grad[offs[2]:offs[3]].any()                      # an unselected block gets nothing


def test_routed_attention_gradients_by_finite_differences():
    rng = np.random.default_rng(22)
    offs = np.array([0, 64, 128, 256, 320])
    N, d = offs[-1], 4
    Qp, Kp, Vp, dOp = (rng.standard_normal((N, 1, d)) * 0.5 for _ in range(4))
    co = np.array([0, 2, 4, 7, 9])
    ci = np.array([0, 2, 1, 3, 0, 1, 2, 2, 3])
    flat = np.array([True, False, True, False])
    scale = 0.7
    r = orc.routed_attention(Qp, Kp, Vp, offs, co, ci, flat, 0, scale, dOp=dOp)
    loss = lambda Q, K, V: float((orc.routed_attention(Q, K, V, offs, co, ci, flat, 0, scale)["O"] * dOp[:, 0]).sum())
    h = 1e-6
    for name, X, G in (("Q", Qp, r["dQ"]), ("K", Kp, r["dK"]), ("V", Vp, r["dV"])):
        for t, c in ((5, 1), (70, 3), (130, 0), (300, 2)):
            Xp, Xm = X.copy(), X.copy()
            Xp[t, 0, c] += h
            Xm[t, 0, c] -= h
            args = {"Q": (Qp, Kp, Vp), "K": (Qp, Kp, Vp), "V": (Qp, Kp, Vp)}[name]
            sub = {"Q": 0, "K": 1, "V": 2}[name]
            ap, am = list(args), list(args)
            ap[sub], am[sub] = Xp, Xm
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert math.isclose(G[t, c], fd, rel_tol=1e-5, abs_tol=1e-8), (name, t, c, G[t, c], fd)


# ---------------------------------------------------------------- next row f4: Hilbert zone order

@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_hilbert_order_walks_face_adjacent_zones_on_cubes(n):
    T = H = W = 8 * n
    order = orc.hilbert_zone_order(T, H, W)
    assert sorted(order.tolist()) == list(range(n ** 3))
    coords = [np.array(np.unravel_index(m, (n, n, n))) for m in order]
    assert (coords[0] == 0).all()                                 # starts at the origin
    for a, b in zip(coords, coords[1:]):
        assert int(np.abs(a - b).sum()) == 1                      # one step along one axis


def _subcube_runs_contiguous(order, dims, j):
    """True when, along `order` (raster zone indices over a grid of `dims`
    zones), the zones of every aligned 2^j sub-cube form one contiguous run."""
    coords = np.array(np.unravel_index(np.asarray(order), dims)).T
    cube_id = [tuple(c >> j) for c in coords]
    seen, prev = set(), None
    for c in cube_id:
        if c != prev:
            if c in seen:
                return False
            seen.add(c)
            prev = c
    return True


@pytest.mark.parametrize("n", [2, 4, 8])
def test_hilbert_order_visits_every_aligned_subcube_in_one_run(n):
    """The defining property of a Hilbert curve: it fills each aligned 2^j
    sub-cube completely before it leaves it, at every level j.  A snake
    (boustrophedon) walk is also face-adjacent, but it leaves a 2-cube after
    two zones and comes back later, so it fails here."""
    order = orc.hilbert_zone_order(8 * n, 8 * n, 8 * n)
    for j in range(1, int(math.log2(n)) + 1):
        assert _subcube_runs_contiguous(order, (n, n, n), j), j
    snake = []
    for t in range(n):
        for hh in range(n):
            hs = hh if t % 2 == 0 else n - 1 - hh
            ws = range(n) if (t * n + hh) % 2 == 0 else range(n - 1, -1, -1)
            snake += [(t * n + hs) * n + w for w in ws]
    assert sorted(snake) == list(range(n ** 3))
    if n >= 4:   # on a 2-cube the only aligned 2-cube is the whole grid
        assert not _subcube_runs_contiguous(snake, (n, n, n), 1)


def test_hilbert_order_keeps_subcube_runs_on_other_grids():
    """On a grid that is not a power-of-two cube the zones outside it are
    skipped, so every aligned sub-cube's part inside the grid is still one run."""
    dims = (3, 5, 2)
    order = orc.hilbert_zone_order(8 * dims[0], 8 * dims[1], 8 * dims[2])
    for j in (1, 2):
        assert _subcube_runs_contiguous(order, dims, j), j


def test_hilbert_order_on_other_grids_is_the_cube_order_restricted():
    T, H, W = 8 * 3, 8 * 5, 8 * 2
    order = orc.hilbert_zone_order(T, H, W)
    assert sorted(order.tolist()) == list(range(3 * 5 * 2))
    cube = orc.hilbert_zone_order(64, 64, 64)                     # 8 x 8 x 8 zones
    inside = [np.unravel_index(m, (8, 8, 8)) for m in cube]
    want = [(t * 5 + h) * 2 + w for t, h, w in inside if t < 3 and h < 5 and w < 2]
    assert order.tolist() == want


def test_layout_and_permutation_follow_the_zone_order():
    T, H, W = 16, 24, 16
    rng = np.random.default_rng(3)
    shape = rng.integers(0, 16, size=2 * 3 * 2)
    order = orc.hilbert_zone_order(T, H, W)
    offs, nb = orc.block_layout(shape, order)
    offs_r, nb_r = orc.block_layout(shape)
    assert nb == nb_r and offs[-1] == T * H * W
    assert (orc.block_layout(shape, np.arange(len(shape)))[0] == offs_r).all()
    pi = orc.permutation(T, H, W, shape, order)
    pi_r = orc.permutation(T, H, W, shape)
    assert sorted(pi.tolist()) == list(range(T * H * W))
    for pos, m in enumerate(order):                               # each zone's 512 tokens move as a unit
        assert (pi[512 * pos:512 * (pos + 1)] == pi_r[512 * m:512 * (m + 1)]).all()


# ---------------------------------------------------------------- next row f4: sub-block scoring

def _runs_tensor(run_means, d):
    """[64 * len(run_means), 1, d] rows: every row of run r equals run_means[r]."""
    return np.repeat(np.asarray(run_means, dtype=np.float64), orc.SUB, axis=0)[:, None, :d]


def test_subblock_logits_are_the_plain_scores_for_64_token_blocks():
    rng = np.random.default_rng(40)
    nb, d = 9, 16
    offs = np.arange(nb + 1) * 64
    Q = rng.standard_normal((64 * nb, 1, d))
    K = rng.standard_normal((64 * nb, 1, d))
    want = orc.block_logits(orc.pool_blocks(Q, offs, 0), orc.pool_blocks(K, offs, 0), 0.25)
    got = orc.subblock_logits(Q, K, offs, 0, 0.25)
    assert got.dtype == np.float32 and (got == want).all()


def test_subblock_logits_equal_the_plain_scores_when_runs_share_one_mean():
    # small integers times 2^-3: every mean and dot product below is exact
    rng = np.random.default_rng(41)
    d = 8
    offs = np.array([0, 256, 384, 448, 704])                      # blocks of 256, 128, 64, 256
    sizes = np.diff(offs) // 64
    qb = rng.integers(-4, 5, size=(len(sizes), d)) / 8.0
    kb = rng.integers(-4, 5, size=(len(sizes), d)) / 8.0
    Q = _runs_tensor(np.repeat(qb, sizes, axis=0), d)
    K = _runs_tensor(np.repeat(kb, sizes, axis=0), d)
    want = orc.block_logits(orc.pool_blocks(Q, offs, 0), orc.pool_blocks(K, offs, 0), 0.5)
    got = orc.subblock_logits(Q, K, offs, 0, 0.5)
    assert (got == want).all()


def test_subblock_logits_closed_forms():
    d = 4
    e0 = [1.0, 0.0, 0.0, 0.0]
    # query block of two runs with means 2 e0 and 0, key block of two runs both e0:
    # run-pair scores 2, 2, 0, 0, so the score is log((e^2 + 1) / 2)
    Q = _runs_tensor([[2.0, 0, 0, 0], [0.0, 0, 0, 0]], d)
    K = _runs_tensor([e0, e0], d)
    got = orc.subblock_logits(Q, K, np.array([0, 128]), 0, 1.0)
    assert math.isclose(float(got[0, 0]), math.log((math.e ** 2 + 1.0) / 2.0), rel_tol=2 ** -23)
    # one query run against a key block of four runs scored 0, 1, 2, 3: log((1 + e + e^2 + e^3) / 4)
    Q = _runs_tensor([e0] * 4, d)
    K = _runs_tensor([[0.0, 0, 0, 0], e0, [2.0, 0, 0, 0], [3.0, 0, 0, 0]], d)
    offs = np.array([0, 256])
    got = orc.subblock_logits(Q, K, offs, 0, 1.0)
    want = math.log(sum(math.exp(s) for s in range(4)) / 4.0)
    assert math.isclose(float(got[0, 0]), want, rel_tol=2 ** -23)
    # a large score range: the factored maximum keeps it finite (log(mean) of e^900 and e^0)
    K = _runs_tensor([[900.0, 0, 0, 0], [0.0, 0, 0, 0], [0.0, 0, 0, 0], [0.0, 0, 0, 0]], d)
    got = orc.subblock_logits(Q, K, offs, 0, 1.0)
    assert math.isclose(float(got[0, 0]), 900.0 + math.log(0.25), rel_tol=2 ** -23)


def test_subblock_logits_lie_between_the_plain_score_and_the_best_run_pair():
    rng = np.random.default_rng(42)
    d = 8
    offs = np.array([0, 64, 320, 448, 512, 768])
    N = int(offs[-1])
    Q = rng.standard_normal((N, 1, d))
    K = rng.standard_normal((N, 1, d))
    scale = 0.5
    got = orc.subblock_logits(Q, K, offs, 0, scale).astype(np.float64)
    plain = orc.block_logits(orc.pool_blocks(Q, offs, 0), orc.pool_blocks(K, offs, 0), scale).astype(np.float64)
    nb = len(offs) - 1
    for i in range(nb):
        for j in range(nb):
            # brute force: every run pair's score from explicit token loops
            best = -math.inf
            for a in range(offs[i], offs[i + 1], 64):
                qa = [sum(Q[t, 0, c] for t in range(a, a + 64)) / 64.0 for c in range(d)]
                for b in range(offs[j], offs[j + 1], 64):
                    kb = [sum(K[t, 0, c] for t in range(b, b + 64)) / 64.0 for c in range(d)]
                    best = max(best, scale * sum(x * y for x, y in zip(qa, kb)))
            tol = 2 ** -22 * max(1.0, abs(best))
            assert plain[i, j] - tol <= got[i, j] <= best + tol, (i, j)
            if offs[i + 1] - offs[i] > 64 or offs[j + 1] - offs[j] > 64:
                assert got[i, j] > plain[i, j] + 1e-6, (i, j)          # Jensen, strict for unequal runs


def test_subblock_logits_do_not_depend_on_the_order_of_runs_in_a_block():
    rng = np.random.default_rng(43)
    d = 8
    offs = np.array([0, 256, 320])
    runs_q = rng.integers(-4, 5, size=(5, d)) / 8.0
    runs_k = rng.integers(-4, 5, size=(5, d)) / 8.0
    base = orc.subblock_logits(_runs_tensor(runs_q, d), _runs_tensor(runs_k, d), offs, 0, 0.5)
    p = [2, 0, 3, 1, 4]
    moved = orc.subblock_logits(_runs_tensor(runs_q[p], d), _runs_tensor(runs_k[p], d), offs, 0, 0.5)
    assert (base == moved).all()


def test_subblock_logits_rows_argument_scores_a_subset():
    rng = np.random.default_rng(44)
    offs = np.array([0, 128, 192, 448])
    Q = rng.standard_normal((448, 1, 16))
    K = rng.standard_normal((448, 1, 16))
    full = orc.subblock_logits(Q, K, offs, 0, 0.25)
    part = orc.subblock_logits(Q, K, offs, 0, 0.25, rows=[2, 0])
    assert (part == full[[2, 0]]).all()
