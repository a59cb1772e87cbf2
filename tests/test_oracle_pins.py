"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Sources: reproduction notes of arXiv 2610.13674 (daiwk.github.io), section "核心公式"
(group scores, kernel kappa = eps + s-bar^T L L^T s-bar > 0, prefix states H0/H1/H2,
readout); its section "本地结果与边界" (dense kernel and HD recursion checked equal);
and the arXiv abstract page (the method starts from a second-order Taylor approximation
of softmax). Each test names the plausible oracle mistake it would catch.
"""
import os
import shutil
import subprocess
import ctypes

import numpy as np
import pytest

import oracle
from oal_synth import HeadParams, random_params, small, draw_L


def _case(seed, B=1, Hq=2, Hkv=1, T=12, d=8, dv=5, g_hi=3, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d)) * scale
    k = rng.standard_normal((B, Hkv, T, d)) * scale
    v = rng.standard_normal((B, Hkv, T, dv))
    p = random_params(rng, Hq, d, g_hi=g_hi)
    return q, k, v, p


# --------------------------------------------------------------------------------------
# 1. A worked example done by hand (d=4 so 1/sqrt(d) = 1/2; dv=2; G=2; T=3), stored with
# its derivation in tests/golden/worked_example_d4.json.
# Catches: L used untransposed (L s-bar gives 12.5 at (0,0)), a missing 1/sqrt(d), a wrong
# group offset into s-bar, exclusive causality, a dropped eps.

import json as _json

_GOLD = _json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                     "worked_example_d4.json")))
WQ = np.array(_GOLD["q"], float)[None, None]
WK = np.array(_GOLD["k"], float)[None, None]
WV = np.array(_GOLD["v"], float)[None, None]
WP = HeadParams(np.array([_GOLD["n_groups"]], np.int32), np.array([_GOLD["group_of_dim"]], np.uint8),
                np.array([_GOLD["L"]], np.float32), np.array([_GOLD["eps"]], np.float32))


def test_worked_example_by_hand():
    kap = oracle.kappa_matrix(WQ, WK, WP, 0, 0)
    np.testing.assert_allclose(kap, _GOLD["kappa"], rtol=0, atol=1e-13)
    y, den = oracle.dense(WQ, WK, WV, WP, return_den=True)
    np.testing.assert_allclose(y[0, 0], [[1, 0], [42 / 47, 5 / 47], [0, 1]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[0, 0], _GOLD["y"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(den[0, 0], _GOLD["den"], rtol=0, atol=1e-13)


def test_worked_example_state_by_hand():
    # H0 = sum [v;1] = [0,3,3]; H1_0 = 1*[1,0,1] + 2*[0,1,1] + 1*[-1,2,1] = [0,4,4];
    # H2_(3,3) = 1*[1,0,1] + 4*[0,1,1] + 9*[-1,2,1] = [-8,22,14];
    # H2_(0,3) = 1*[1,0,1] - 4*[0,1,1] + 3*[-1,2,1] = [-2,2,0].
    H = oracle.state(WK, WV)[0, 0]
    d = 4
    idx = lambda r, t: 1 + d + r * d - r * (r - 1) // 2 + (t - r)
    rows = _GOLD["state_rows"]
    np.testing.assert_allclose(H[0], rows["H0"])
    np.testing.assert_allclose(H[1], rows["H1_0"])
    np.testing.assert_allclose(H[idx(3, 3)], rows["H2_3_3"])
    np.testing.assert_allclose(H[idx(0, 3)], rows["H2_0_3"])
    assert H.shape[0] == 1 + d + d * (d + 1) // 2


# --------------------------------------------------------------------------------------
# 2. Dense kernel sum == the pages' H0/H1/H2 recurrence (their own equivalence check).
# Catches a wrong (eps, L) -> (a, b, C) expansion, a wrong 1/d vs 1/sqrt(d), wrong GQA map.

@pytest.mark.parametrize("d,g_hi,seed", [(4, 1, 1), (4, 4, 2), (8, 2, 3), (8, 4, 4),
                                         (64, 4, 5), (64, 6, 6)])
def test_dense_equals_recurrence(d, g_hi, seed):
    T = 16 if d == 64 else 24
    q, k, v, p = _case(seed, B=2, Hq=4, Hkv=2, T=T, d=d, dv=3, g_hi=g_hi)
    y = oracle.dense(q, k, v, p)
    yr, H = oracle.recurrence(q, k, v, p, return_state=True)
    assert np.abs(y - yr).max() <= 1e-12 * max(1.0, np.abs(y).max())
    # the upper-triangle state equals the recurrence's full H2 folded onto r <= t
    Hu = oracle.state(k, v)
    nf = 1 + d
    np.testing.assert_allclose(Hu[:, :, :nf], H[:, :, :nf], rtol=1e-12, atol=1e-12)
    f = nf
    for r in range(d):
        for t in range(r, d):
            np.testing.assert_allclose(Hu[:, :, f], H[:, :, nf + r * d + t], rtol=1e-12, atol=1e-10)
            f += 1


# --------------------------------------------------------------------------------------
# 3. kappa > 0: kappa >= eps for every pair (PSD parameterisation). Includes an L with zero
# and negative diagonal entries and huge scores. Catches a sign error in the square.

def test_kappa_at_least_eps():
    for seed in range(4):
        q, k, v, p = _case(10 + seed, Hq=3, T=20, d=16, g_hi=5, scale=4.0)
        p.L[0, 1, 1] = 0.0
        p.L[1] *= -1.0
        for h in range(3):
            kap = oracle.kappa_matrix(q, k, p, 0, h)
            low = np.tril(np.ones_like(kap, dtype=bool))
            assert (kap[low] >= p.eps[h]).all()


# --------------------------------------------------------------------------------------
# 4. Readout is a positive-weighted average: each y_i lies in the coordinate-wise hull of
# v_{<=i}. Catches a sign slip that makes a weight negative, or a non-causal key.

def test_convex_hull():
    q, k, v, p = _case(20, B=2, Hq=4, Hkv=2, T=40, d=16, dv=6, g_hi=4, scale=2.0)
    y = oracle.dense(q, k, v, p)
    n_rep = 2
    for b in range(2):
        for h in range(4):
            vv = v[b, h // n_rep]
            lo = np.minimum.accumulate(vv, axis=0)
            hi = np.maximum.accumulate(vv, axis=0)
            assert (y[b, h] >= lo - 1e-12).all() and (y[b, h] <= hi + 1e-12).all()


# --------------------------------------------------------------------------------------
# 5. G=1: all dims in one group, with L chosen so that kappa = 1 + s + s^2/2 (s = q.k/sqrt d),
# the second-order Taylor expansion of exp(s) named on the abstract page. Compared with a
# separately written textbook Taylor-kernel attention. Catches a wrong constant slot in L.

@pytest.mark.parametrize("eps", [1e-3, 0.1, 0.0])
def test_g1_is_second_order_taylor(eps):
    rng = np.random.default_rng(30)
    B, H, T, d, dv = 1, 2, 33, 16, 4
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, dv))
    c = np.sqrt(1 - eps)
    L1 = np.array([[c, 0.0], [1 / (2 * c), np.sqrt((1 - 2 * eps) / (4 * (1 - eps)))]], np.float64)
    p = HeadParams(np.ones(H, np.int32), np.zeros((H, d), np.uint8),
                   np.stack([L1, L1]).astype(np.float64), np.full(H, eps))
    y = oracle.dense(q, k, v, p)
    for h in range(H):
        s = (q[0, h] @ k[0, h].T) / np.sqrt(d)
        w = np.tril(1.0 + s + 0.5 * s * s)
        ref = (w @ v[0, h]) / w.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(y[0, h], ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------------------
# 6. L = 0 and eps > 0: kappa is constant, so y_i is the prefix mean of v (H0 path alone).

def test_l_zero_gives_prefix_mean():
    q, k, v, p = _case(40, Hq=2, T=25, d=8, dv=3)
    p.L[:] = 0.0
    y = oracle.dense(q, k, v, p)
    mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, 26)[:, None]
    np.testing.assert_allclose(y[0, 0], mean, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y[0, 1], mean, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------------------
# 7. Trivial cases: T = 1 returns v_0; constant v returns v everywhere.

def test_t1_and_constant_v():
    q, k, v, p = _case(50, Hq=2, T=1, d=8, dv=4)
    y = oracle.dense(q, k, v, p)
    np.testing.assert_allclose(y[0, 0, 0], v[0, 0, 0], rtol=1e-15)
    q, k, v, p = _case(51, Hq=2, T=17, d=8, dv=4)
    v[:] = np.array([0.5, -2.0, 3.0, 7.0])
    y = oracle.dense(q, k, v, p)
    np.testing.assert_allclose(y, np.broadcast_to(np.array([0.5, -2.0, 3.0, 7.0]), y.shape),
                               rtol=1e-13)


# --------------------------------------------------------------------------------------
# 8. Normalisation: (L, eps) -> (alpha L, alpha^2 eps) leaves y unchanged.

def test_scale_invariance():
    q, k, v, p = _case(60, Hq=2, T=20, d=8, g_hi=3)
    y = oracle.dense(q, k, v, p)
    p2 = HeadParams(p.n_groups, p.group_of_dim, p.L.astype(np.float64) * 3.0,
                    p.eps.astype(np.float64) * 9.0)
    np.testing.assert_allclose(oracle.dense(q, k, v, p2), y, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------------------
# 9. Group split: splitting the last group in two and giving the new group a copy of the
# old L row (zero column appended, zero diagonal) leaves kappa and y unchanged, because
# s_old = s_a + s_b enters L^T s-bar linearly. Catches any per-group scale or a wrong
# group index. Permuting dims consistently in q, k and the group map leaves y unchanged.

def test_group_split_invariance():
    rng = np.random.default_rng(70)
    d, Hq, T = 16, 1, 20
    q = rng.standard_normal((1, Hq, T, d)) * 2
    k = rng.standard_normal((1, Hq, T, d)) * 2
    v = rng.standard_normal((1, Hq, T, 3))
    G = 3
    gam = np.array([[0] * 8 + [1] * 4 + [2] * 4], np.uint8)
    L = draw_L(rng, G, G).astype(np.float64)
    p = HeadParams(np.array([G], np.int32), gam, L[None], np.array([1e-3]))
    y = oracle.dense(q, k, v, p)
    gam2 = gam.copy()
    gam2[0, 14:16] = 3                     # last group {12..15} -> {12,13} and {14,15}
    L2 = np.zeros((G + 2, G + 2))
    L2[:G + 1, :G + 1] = L
    L2[G + 1, :G + 1] = L[G]               # copy of the split group's row
    p2 = HeadParams(np.array([G + 1], np.int32), gam2, L2[None], np.array([1e-3]))
    np.testing.assert_allclose(oracle.dense(q, k, v, p2), y, rtol=1e-12, atol=1e-13)


def test_dim_permutation_invariance():
    q, k, v, p = _case(80, B=1, Hq=2, Hkv=1, T=18, d=16, g_hi=4)
    y = oracle.dense(q, k, v, p)
    perm = np.random.default_rng(81).permutation(16)
    p2 = HeadParams(p.n_groups, p.group_of_dim[:, perm], p.L, p.eps)
    np.testing.assert_allclose(oracle.dense(q[..., perm], k[..., perm], v, p2), y,
                               rtol=1e-12, atol=1e-13)


def test_dense_rows_match_dense():
    inp = small(90, B=2, Hq=4, Hkv=2, T=30)
    y = oracle.dense(inp.q, inp.k, inp.v, inp.params)
    rows = [(0, 0, 0), (1, 3, 29), (0, 2, 17), (1, 1, 5)]
    yr = oracle.dense_rows(inp.q, inp.k, inp.v, inp.params, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(yr[n], y[b, h, i])


def test_causality():
    q, k, v, p = _case(95, Hq=2, T=20, d=8)
    y = oracle.dense(q, k, v, p)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 12] += 1.0
    v2[0, 0, 12] -= 3.0
    y2 = oracle.dense(q, k2, v2, p)
    np.testing.assert_array_equal(y2[:, :, :12], y[:, :, :12])
    assert np.abs(y2[:, :, 12:] - y[:, :, 12:]).max() > 1e-6


# --------------------------------------------------------------------------------------
# 10. Mutation check: plausible mistakes planted in a private copy of the oracle (compiled
# on the CPU into a temporary directory) must each fail one of the pins above.

MUTATIONS = {
    "L_untransposed": ("z += L[g * (g_max + 1) + m] * sbar[g];",
                       "z += L[m * (g_max + 1) + g] * sbar[g];"),
    "no_inv_sqrt_d": ("sbar[g] *= inv_sqrt_d;", "sbar[g] *= 1.0;"),
    "group_offset": ("sbar[1 + group_of_dim[r]] += q[r] * k[r];",
                     "sbar[group_of_dim[r]] += q[r] * k[r];"),
    "exclusive_causal": ("for (int j = 0; j <= i; ++j) {               /* causal, inclusive: j <= i */",
                         "for (int j = 0; j < i || j == 0; ++j) {"),
    "dropped_eps": ("double kap = eps;", "double kap = 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    mfile = tmp_path / "mut.c"
    mfile.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-o", str(so), str(mfile), "-lm"])
    lib = ctypes.CDLL(str(so))
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._load()
        for fn in ("oal_oracle_dense", "oal_oracle_kappa_matrix"):
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        oracle._lib = lib
        lib.oal_oracle_kappa.restype = ctypes.c_double
        kap = oracle.kappa_matrix(WQ, WK, WP, 0, 0)
        y = oracle.dense(WQ, WK, WV, WP)
        ok = (np.allclose(kap, [[10.5, 0, 0], [10.5, 1.25, 0], [6.25, 6.5, 6.25]]) and
              np.allclose(y[0, 0], [[1, 0], [42 / 47, 5 / 47], [0, 1]]))
        assert not ok, f"planted mistake {name} passed the worked-example pin"
    finally:
        oracle._lib = saved


# --------------------------------------------------------------------------------------
# 11. Causal contribution score chi (section "核心公式", first display): the mean over the
# T(T+1)/2 causal pairs of |q_ir k_jr| / sqrt(d), per prompt, query head and dim, and its
# mean over prompts. The oracle is the double loop over pairs; the pins below fix it by a
# hand-worked example, closed forms and an independent factorisation.

_CGOLD = _json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                      "contribution_example_d4.json")))
CQ = np.array(_CGOLD["q"], float)[:, None]
CK = np.array(_CGOLD["k"], float)[:, None]


def test_contribution_worked_example_by_hand():
    # Catches: a dropped absolute value, anti-causal or all-pairs sums, a T^2 normaliser,
    # a missing 1/sqrt(d), a wrong prompt average.
    chi, chi_mean = oracle.contribution(CQ, CK)
    np.testing.assert_allclose(chi[:, 0], _CGOLD["chi"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(chi_mean[0], _CGOLD["chi_mean"], rtol=0, atol=1e-15)


def test_contribution_constant_inputs_closed_form():
    # q_ir = a_r and k_jr = c_r for every token: every pair contributes |a_r c_r| / sqrt(d),
    # so the mean over pairs is that value whatever T is (catches any normaliser other
    # than the pair count, and a missing or doubled 1/sqrt(d)).
    rng = np.random.default_rng(3)
    d = 16
    a, c = rng.standard_normal(d), rng.standard_normal(d)
    for T in (1, 2, 7, 40):
        q = np.broadcast_to(a, (1, 1, T, d)).copy()
        k = np.broadcast_to(c, (1, 1, T, d)).copy()
        chi, _ = oracle.contribution(q, k)
        np.testing.assert_allclose(chi[0, 0], np.abs(a * c) / 4.0, rtol=1e-13, atol=0)


def test_contribution_matches_prefix_factorisation():
    # Independent evaluation: sum_{j<=i} |q_ir k_jr| = |q_ir| * (inclusive prefix sum of
    # |k_jr|), summed over i (a cumulative sum instead of the pair loop).
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T, d = 2, 6, 2, 33, 8
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    chi, chi_mean = oracle.contribution(q, k)
    kpre = np.cumsum(np.abs(k), axis=2)
    kv_of = np.arange(Hq) // (Hq // Hkv)
    ref = (np.abs(q) * kpre[:, kv_of]).sum(axis=2) / np.sqrt(d) / (T * (T + 1) / 2)
    np.testing.assert_allclose(chi, ref, rtol=1e-13, atol=0)
    np.testing.assert_allclose(chi_mean, ref.mean(axis=0), rtol=1e-13, atol=0)


def test_contribution_single_token_and_causality():
    # T = 1: the only pair is (0, 0). Changing k at the last position changes only the pair
    # (T-1, T-1): the difference is |q_{T-1}| * (|k'| - |k|) / sqrt(d) / |Omega|.
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 1, 8))
    k = rng.standard_normal((1, 1, 1, 8))
    chi, _ = oracle.contribution(q, k)
    np.testing.assert_allclose(chi[0, 0], np.abs(q[0, 0, 0] * k[0, 0, 0]) / np.sqrt(8), rtol=1e-15)
    T = 10
    q = rng.standard_normal((1, 1, T, 8))
    k = rng.standard_normal((1, 1, T, 8))
    k2 = k.copy()
    k2[0, 0, T - 1] *= 3.0
    c1, _ = oracle.contribution(q, k)
    c2, _ = oracle.contribution(q, k2)
    expect = np.abs(q[0, 0, T - 1]) * 2.0 * np.abs(k[0, 0, T - 1]) / np.sqrt(8) / (T * (T + 1) / 2)
    np.testing.assert_allclose(c2[0, 0] - c1[0, 0], expect, rtol=1e-10, atol=1e-15)


def test_contribution_invariances():
    # Sign flips of q or k entries leave chi unchanged, scaling q by s scales it by |s|,
    # and permuting the dims permutes it.
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 2, 9, 8))
    k = rng.standard_normal((2, 1, 9, 8))
    chi, _ = oracle.contribution(q, k)
    sq = rng.choice([-1.0, 1.0], size=q.shape)
    sk = rng.choice([-1.0, 1.0], size=k.shape)
    np.testing.assert_allclose(oracle.contribution(q * sq, k * sk)[0], chi, rtol=1e-14)
    np.testing.assert_allclose(oracle.contribution(-2.5 * q, k)[0], 2.5 * chi, rtol=1e-14)
    perm = rng.permutation(8)
    np.testing.assert_allclose(oracle.contribution(q[..., perm], k[..., perm])[0], chi[..., perm],
                               rtol=1e-14)


def test_contribution_gqa_map_closed_form():
    # Query head h reads KV head h // (Hq/Hkv): with q = 1 and KV head m's keys all equal
    # to m+1, chi of head h is (h // rep + 1) / sqrt(d) in every dim.
    Hq, Hkv, T, d = 6, 3, 5, 4
    q = np.ones((1, Hq, T, d))
    k = np.stack([np.full((T, d), m + 1.0) for m in range(Hkv)])[None]
    chi, _ = oracle.contribution(q, k)
    expect = (np.arange(Hq) // (Hq // Hkv) + 1.0) / 2.0
    np.testing.assert_allclose(chi[0], np.repeat(expect[:, None], d, axis=1), rtol=1e-15)


CHI_MUTATIONS = {
    "chi_no_abs": ("acc[r] += fabs(qb[(size_t)i * d + r] * kb[(size_t)j * d + r] / sqrt_d);",
                   "acc[r] += (qb[(size_t)i * d + r] * kb[(size_t)j * d + r] / sqrt_d);"),
    "chi_anticausal": ("for (int j = 0; j <= i; ++j)\n                for (int r = 0; r < d; ++r)\n"
                       "                    acc[r] +=",
                       "for (int j = i; j < T; ++j)\n                for (int r = 0; r < d; ++r)\n"
                       "                    acc[r] +="),
    "chi_square_norm": ("double n_pairs = (double)T * (double)(T + 1) / 2.0;",
                        "double n_pairs = (double)T * (double)T;"),
    "chi_no_sqrt_d": ("double sqrt_d = sqrt((double)d);", "double sqrt_d = 1.0;"),
    "chi_gqa_modulo": ("int b = bh / Hq, h = bh % Hq, kv = h / rep;",
                       "int b = bh / Hq, h = bh % Hq, kv = h % Hkv;"),
    "chi_mean_sum": ("chi_mean[(size_t)h * d + r] = s / B;", "chi_mean[(size_t)h * d + r] = s;"),
}


@pytest.mark.parametrize("name", sorted(CHI_MUTATIONS))
def test_contribution_pins_catch_planted_mistakes(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    old, new = CHI_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    mfile = tmp_path / "mut.c"
    mfile.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-o", str(so), str(mfile), "-lm"])
    lib = ctypes.CDLL(str(so))
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._load()
        lib.oal_oracle_contribution.argtypes = real.oal_oracle_contribution.argtypes
        oracle._lib = lib
        failed = []
        for test in (test_contribution_worked_example_by_hand, test_contribution_gqa_map_closed_form):
            try:
                test()
            except AssertionError:
                failed.append(test.__name__)
        assert failed, f"planted mistake {name} passed the contribution pins"
    finally:
        oracle._lib = saved


# --------------------------------------------------------------------------------------
# 12. Backward of the dense definition (oracle.backward): gradients of sum(dy * y) with
# respect to q, k, v, L and eps, pinned by central finite differences of oracle.dense (fp64;
# L and eps as fp64 arrays so that the perturbations are exact), a closed form for L = 0,
# and the scale invariance of y under (L, eps) -> (a L, a^2 eps).

def _bwd_case(seed, B=1, Hq=2, Hkv=1, T=5, d=4, dv=3, g_hi=3):
    q, k, v, p = _case(seed, B, Hq, Hkv, T, d, dv, g_hi=g_hi)
    p64 = HeadParams(p.n_groups, p.group_of_dim, p.L.astype(np.float64), p.eps.astype(np.float64) + 0.05)
    dy = np.random.default_rng(seed + 1).standard_normal((B, Hq, T, dv))
    return q, k, v, p64, dy


def _loss(q, k, v, p, dy):
    return float((oracle.dense(q, k, v, p) * dy).sum())


def _fd(f, x, idx, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("seed", [31, 32])
def test_backward_matches_finite_differences(seed):
    # Catches: a wrong sign or missing term in the denominator gradient, a dropped factor 2
    # of dz, a missing 1/sqrt(d), a transposed L index, dk/dv sums over the wrong pairs.
    q, k, v, p, dy = _bwd_case(seed)
    dq, dk, dv, dL, deps = oracle.backward(q, k, v, p, dy)
    rng = np.random.default_rng(seed + 2)
    checks = []
    for arr, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "q":
                f = lambda x: _loss(x, k, v, p, dy)
            elif name == "k":
                f = lambda x: _loss(q, x, v, p, dy)
            else:
                f = lambda x: _loss(q, k, x, p, dy)
            checks.append((name, idx, _fd(f, arr, idx), grad[idx]))
    for h in range(p.L.shape[0]):
        G = int(p.n_groups[h])
        for a in range(G + 1):
            for c in range(a + 1):
                def f(x, h=h, a=a, c=c):
                    return _loss(q, k, v, HeadParams(p.n_groups, p.group_of_dim, x, p.eps), dy)
                checks.append(("L", (h, a, c), _fd(f, p.L, (h, a, c)), dL[h, a, c]))
        def fe(x):
            return _loss(q, k, v, HeadParams(p.n_groups, p.group_of_dim, p.L, x), dy)
        checks.append(("eps", (h,), _fd(fe, p.eps, (h,)), deps[h]))
    for name, idx, num, ana in checks:
        assert abs(num - ana) <= 1e-6 * (1.0 + abs(num)), (name, idx, num, ana)
    # entries outside each head's lower triangle carry no gradient
    for h in range(p.L.shape[0]):
        G = int(p.n_groups[h])
        mask = np.tril(np.ones_like(dL[h]))
        mask[G + 1:, :] = 0
        assert np.all(dL[h][mask == 0] == 0.0)


def test_backward_l_zero_closed_form():
    # L = 0: kappa = eps for every pair, y_i is the prefix mean of v, so dv_j = sum_{i>=j}
    # dy_i / (i+1), dq = dk = 0, and deps = 0 (y does not depend on a constant kernel's size).
    q, k, v, p, dy = _bwd_case(41, Hq=2, T=6)
    pz = HeadParams(p.n_groups, p.group_of_dim, np.zeros_like(p.L), p.eps)
    dq, dk, dv, dL, deps = oracle.backward(q, k, v, pz, dy)
    T = q.shape[2]
    want = np.zeros_like(v)
    for h in range(2):
        for j in range(T):
            want[0, 0, j] += sum(dy[0, h, i] / (i + 1) for i in range(j, T))
    np.testing.assert_allclose(dv, want, rtol=1e-12, atol=1e-14)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    np.testing.assert_allclose(deps, 0.0, atol=1e-12)
    assert np.abs(dL).max() == 0.0


def test_backward_scale_invariance():
    # y(a L, a^2 eps) = y(L, eps), so d/da at a = 1: sum(L * dL) + 2 eps deps = 0 per head.
    q, k, v, p, dy = _bwd_case(43, Hq=3, Hkv=1, T=7, d=8, dv=4)
    _, _, _, dL, deps = oracle.backward(q, k, v, p, dy)
    for h in range(3):
        s = float((p.L[h] * dL[h]).sum() + 2 * p.eps[h] * deps[h])
        scale = float(np.abs(p.L[h] * dL[h]).sum() + abs(2 * p.eps[h] * deps[h]))
        assert abs(s) <= 1e-10 * max(scale, 1.0), (h, s, scale)


BWD_MUTATIONS = {
    "bwd_dden_sign": ("dden -= dyi[c] * yrow[c];", "dden += dyi[c] * yrow[c];"),
    "bwd_no_factor_2": ("const double dz = 2.0 * z[m] * dkap;", "const double dz = z[m] * dkap;"),
    "bwd_no_inv_sqrt_d": ("const double ds = dsbar[1 + gam[r]] * inv_sqrt_d;",
                          "const double ds = dsbar[1 + gam[r]];"),
    "bwd_L_transposed": ("dsbar[g] += Lh[g * gm1 + m] * dz;", "dsbar[g] += Lh[m * gm1 + g] * dz;"),
    "bwd_dv_no_kappa": ("dvb[(size_t)j * dv + c] += kap * dnum[c];", "dvb[(size_t)j * dv + c] += dnum[c];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_pins_catch_planted_mistakes(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    old, new = BWD_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    mfile = tmp_path / "mut.c"
    mfile.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-o", str(so), str(mfile), "-lm"])
    lib = ctypes.CDLL(str(so))
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._load()
        for fn in ("oal_oracle_backward", "oal_oracle_dense", "oal_oracle_kappa"):
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        lib.oal_oracle_kappa.restype = ctypes.c_double
        # the mutant library's forward is the real one (only the backward was changed): the
        # finite-difference pin must fail against the mutant's backward
        oracle._lib = lib
        failed = []
        for test, args in ((test_backward_matches_finite_differences, (31,)),
                           (test_backward_l_zero_closed_form, ()), (test_backward_scale_invariance, ())):
            try:
                test(*args)
            except AssertionError:
                failed.append(test.__name__)
        assert failed, f"planted mistake {name} passed the backward pins"
    finally:
        oracle._lib = saved


# --------------------------------------------------------------------------------------
# 6. The parity metric itself. Every GPU parity test and smoke() decide pass or fail with
# oracle.row_error = max over rows of ||y_i - y*_i||_inf / ||y*_i||_inf (row-normwise
# relative error over the last axis). Hand-computed values pin it; each case names the
# plausible mistake it catches.

def test_row_error_hand_computed():
    re_ = oracle.row_error
    # one row: |2.5 - 2| / max(|1|, |2|, |-4|) = 0.5 / 4
    assert re_([[1.0, 2.5, -4.0]], [[1.0, 2.0, -4.0]]) == 0.125
    # a zero reference entry: its absolute error counts against the row norm, 0.3 / 3
    # (an elementwise ratio would divide by zero)
    assert abs(re_([[0.3, 3.0]], [[0.0, 3.0]]) - 0.1) < 1e-15
    # the error sits in a small-magnitude column: normwise 1e-6 / 10 = 1e-7, whereas an
    # elementwise relative error would report 1.0
    assert abs(re_([[2e-6, 10.0]], [[1e-6, 10.0]]) - 1e-7) < 1e-20
    # per-row normalisation: row 0 has 0.5 / 100, row 1 has 0.001 / 0.01 = 0.1; a global
    # normaliser would give 0.5 / 100 = 0.005
    assert abs(re_([[100.5, 0.0], [0.011, 0.0]], [[100.0, 0.0], [0.01, 0.0]]) - 0.1) < 1e-12
    # max over rows, not mean: rows at 0.25 and 0 give 0.25 (the mean would be 0.125)
    assert re_([[1.25, 0.0], [3.0, -3.0]], [[1.0, 0.0], [3.0, -3.0]]) == 0.25
    # the last axis is the row: [B, H, T, d] arrays, worst row (b=1, h=0, t=2) = 0.5 / 2
    y_ref = np.ones((2, 3, 4, 5))
    y_ref[1, 0, 2] = [2.0, -2.0, 1.0, 0.5, 0.0]
    y_ref[1, 0, 0, 1] = 10.0    # the error's column has norm 10, its row norm 2
    y = y_ref.copy()
    y[1, 0, 2, 1] += 0.5
    y[0, 2, 3, 4] += 0.1        # a second, smaller row error (0.1 / 1)
    assert re_(y, y_ref) == 0.25
    # read along the wrong axis the same data give max(0.5 / 10, 0.1 / 1) = 0.1
    assert abs(re_(np.swapaxes(y, -1, -2), np.swapaxes(y_ref, -1, -2)) - 0.1) < 1e-12
    # an exact match is 0, an empty array is 0
    assert re_(y_ref, y_ref) == 0.0 and re_(np.zeros((0, 64)), np.zeros((0, 64))) == 0.0


def test_row_error_nan_and_inf_fail():
    """A NaN or Inf output anywhere makes the metric NaN or Inf, so `err <= tol` is False."""
    y_ref = np.ones((3, 4))
    for bad in (np.nan, np.inf, -np.inf):
        y = y_ref.copy()
        y[1, 2] = bad
        e = oracle.row_error(y, y_ref)
        assert not (e <= 3e-2), (bad, e)
