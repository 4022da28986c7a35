"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: a closed form, a
library routine (scipy / numpy), a published table, an invariant, or brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.special
import scipy.stats

import oracle as O
import tq_workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLD, "page_figures.json")))
BOOK = json.load(open(os.path.join(GOLD, "textbook.json")))


# ------------------------------------------------------------------------- codebook

@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kb", [1, 2, 3, 4])
def test_codebook_fixed_point_against_scipy(d, kb):
    """Lloyd-Max optimality: boundaries are midpoints and each centroid is its cell's
    conditional mean, recomputed with scipy's betainc and numerical quadrature."""
    c, b, _ = O.codebook(d, kb)
    L = 1 << kb
    p = (d - 1) / 2
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(c, -c[::-1], rtol=0, atol=0)
    np.testing.assert_allclose(b, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-18)
    lognorm = (2 * p - 1) * math.log(2) + scipy.special.betaln(p, p)
    dens = lambda t: t * math.exp((p - 1) * math.log1p(-t * t) - lognorm)
    edges = [-1.0] + list(b) + [1.0]
    for i in range(L):
        lo, hi = edges[i], edges[i + 1]
        mass = scipy.special.betainc(p, p, (1 + hi) / 2) - scipy.special.betainc(p, p, (1 + lo) / 2)
        mom, _ = scipy.integrate.quad(dens, lo, hi, epsabs=1e-16, epsrel=1e-13, limit=200)
        assert abs(mom / mass - c[i]) <= 1e-11 * max(1.0, abs(c[i]) * math.sqrt(d))


@pytest.mark.parametrize("d", [64, 128, 256, 1024])
def test_codebook_one_bit_closed_form(d):
    """kb = 1: the centroids are +-E|t| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    c, _, _ = O.codebook(d, 1)
    e_abs = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - e_abs) < 1e-11 * e_abs and abs(c[0] + e_abs) < 1e-11 * e_abs


@pytest.mark.parametrize("kb,key", [(2, "levels4"), (3, "levels8"), (4, "levels16")])
def test_codebook_gaussian_limit(kb, key):
    """As d grows, sqrt(d) * c approaches Max's N(0,1) quantiser (published table)."""
    c, _, _ = O.codebook(65536, kb)
    got = math.sqrt(65536) * c[len(c) // 2:]
    np.testing.assert_allclose(got, BOOK["gaussian_lloyd_max"][key], atol=1.2e-3)


def test_codebook_gaussian_limit_mse():
    """Distortion per coordinate of the 3-bit table times d -> Max's 0.03454."""
    d = 65536
    c, b, _ = O.codebook(d, 3)
    edges = [-1.0] + list(b) + [1.0]
    p = (d - 1) / 2
    lognorm = (2 * p - 1) * math.log(2) + scipy.special.betaln(p, p)
    mse = 0.0
    for i in range(8):
        f = lambda t, ci=c[i]: (t - ci) ** 2 * math.exp((p - 1) * math.log1p(-t * t) - lognorm)
        v, _ = scipy.integrate.quad(f, edges[i], edges[i + 1], epsabs=1e-18, limit=200,
                                    points=None)
        mse += v
    assert abs(d * mse - BOOK["gaussian_lloyd_max"]["mse8"]) < 2e-4


def test_coordinate_law_cdf_against_monte_carlo_sphere():
    """The law used for the codebook is that of one coordinate of a uniform unit vector."""
    d = 128
    r = np.random.default_rng(7)
    x = r.standard_normal((200000, d))
    t = x[:, 0] / np.linalg.norm(x, axis=1)
    for q in (-0.15, -0.05, 0.0, 0.02, 0.1):
        emp = np.mean(t <= q)
        assert abs(emp - O.coord_cdf(d, q)) < 4 * math.sqrt(0.25 / len(t))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_stored_codebook_is_fp16_rounding_with_midpoints(d):
    c, _, _ = O.codebook(d, 3)
    cs, bs = O.stored_codebook(d, 3)
    np.testing.assert_array_equal(cs, c.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(bs, 0.5 * (cs[:-1] + cs[1:]))
    assert bs[3] == 0.0 and np.array_equal(bs, -bs[::-1])
    np.testing.assert_array_equal(bs, bs.astype(np.float32).astype(np.float64))   # exact in fp32


def _cell_distortion(d, c, b):
    """d * sum_i int_{cell i} (t - c_i)^2 f(t) dt for the coordinate law of a uniform unit
    vector in R^d, cells bounded by b, by scipy quadrature (independent of the oracle)."""
    p = (d - 1) / 2
    lognorm = (2 * p - 1) * math.log(2) + scipy.special.betaln(p, p)
    edges = [-1.0] + list(b) + [1.0]
    tot = 0.0
    for i in range(len(c)):
        f = lambda t, ci=c[i]: (t - ci) ** 2 * math.exp((p - 1) * math.log1p(-t * t) - lognorm)
        v, _ = scipy.integrate.quad(f, edges[i], edges[i + 1], epsabs=1e-20, epsrel=1e-13, limit=400)
        tot += v
    return d * tot


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kb", [1, 2, 3, 4])
def test_stored_table_distortion_cost(d, kb):
    """The stored table (binary16 centroids, boundaries at their midpoints) is the library's
    storage format, not a reading of the pages.  Its cost: d * MSE of the stored table is at
    least the fp64 Lloyd-Max optimum's (which minimises it) and within 1e-5 of it (relative;
    measured at most 3.3e-6)."""
    c, b, _ = O.codebook(d, kb)
    cs, bs = O.stored_codebook(d, kb)
    opt, st = _cell_distortion(d, c, b), _cell_distortion(d, cs, bs)
    assert st >= opt * (1 - 1e-9)
    assert st <= opt * (1 + 1e-5), (d, kb, opt, st)


# ------------------------------------------------------------------------- fp16 / tables

def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = O.f16_bits_fast(bits)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f16_encode_matches_numpy_rounding():
    r = np.random.default_rng(1)
    xs = np.concatenate([
        r.standard_normal(20000) * 10.0 ** r.integers(-9, 5, 20000),
        (np.arange(2048) + 0.5) * 2.0 ** -24,            # subnormal ties
        (1024 + np.arange(1024) + 0.5) * 2.0 ** -10,     # normal ties in [1, 2)
        [65504.0, 65519.99, 65520.0, 1e6, -0.0, 0.0, 6.0e-8, 2.9802322387695312e-08],
    ])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([O.double_to_f16(x) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_splitmix64_published_outputs():
    exp = [int(h, 16) for h in BOOK["splitmix64_seed0"]["outputs"]]
    assert [O.splitmix64_at(0, i) for i in range(len(exp))] == exp


def test_tables_law():
    """sigma is balanced +-1 and S is N(0,1) rounded to fp16 (KS test, moments)."""
    d = 256
    sigma, S = O.tables(d, W.TABLE_SEED)
    assert set(np.unique(sigma)) <= {-1, 1}
    assert abs(sigma.mean()) < 4 / math.sqrt(d)
    s = O.f16_bits_fast(S).ravel()
    assert abs(s.mean()) < 4 / math.sqrt(s.size)
    assert abs(s.var() - 1) < 0.02
    assert scipy.stats.kstest(s, "norm").pvalue > 1e-3
    assert np.array_equal(O.tables(d, W.TABLE_SEED)[1], S)
    assert not np.array_equal(O.tables(d, W.TABLE_SEED + 1)[1], S)


# ------------------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_hadamard_matches_scipy(d):
    np.testing.assert_array_equal(O.hadamard(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_is_orthogonal_and_preserves_norm(d):
    sigma, _ = O.tables(d, W.TABLE_SEED)
    P = O.rotate(sigma, np.eye(d))   # row r = Pi e_r, i.e. columns of Pi
    np.testing.assert_allclose(P @ P.T, np.eye(d), atol=1e-13)
    x = np.random.default_rng(3).standard_normal((16, d))
    y = O.rotate(sigma, x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    e0 = np.zeros(d); e0[0] = 1
    np.testing.assert_allclose(O.rotate(np.ones(d, np.int8), e0)[0], np.ones(d) / math.sqrt(d))


# ------------------------------------------------------------------------- key encode

def _keys(d, n, seed=11):
    return np.random.default_rng(seed).standard_normal((n, d))


@pytest.mark.parametrize("d", [128, 256])
def test_key_encode_invariants(d):
    c32, b32 = O.stored_codebook(d, 3)
    sigma, S = O.tables(d, W.TABLE_SEED)
    k = _keys(d, 64)
    k[3] = 0.0                                  # zero key: u = 0
    r = O.quantize_keys(k, c32, b32, sigma, S)
    u = O.rotate(sigma, k) / np.where(r["norm"] > 0, r["norm"], 1)[:, None]
    np.testing.assert_allclose(r["norm"], np.linalg.norm(k, axis=1), rtol=1e-14)
    lo = np.concatenate([[-np.inf], b32])[r["idx"]]
    hi = np.concatenate([b32, [np.inf]])[r["idx"]]
    assert np.all((lo < u) & (u <= hi))         # idx = #{b_i < u}
    chat = c32[r["idx"]]
    np.testing.assert_allclose(r["rnorm"] ** 2, (u * u).sum(1) - 2 * (u * chat).sum(1) + (chat * chat).sum(1),
                               rtol=1e-10, atol=1e-14)
    assert np.all(r["idx"][3] == np.searchsorted(b32, 0.0, side="left"))
    Sd = O.f16_bits_fast(S)
    p = (u - chat) @ Sd.T
    np.testing.assert_array_equal(r["z"], (p >= 0).astype(np.uint8))


def _rotate_numpy(sigma, k):
    """Pi k with Pi = H diag(sigma) / sqrt(d), H from scipy (not the oracle's rotation)."""
    d = sigma.shape[0]
    H = scipy.linalg.hadamard(d).astype(np.float64)
    return (np.asarray(k, np.float64) * sigma.astype(np.float64)) @ H.T / math.sqrt(d)


@pytest.mark.parametrize("d,kb", [(128, 3), (256, 3), (64, 1), (64, 2), (64, 3), (64, 4), (128, 2), (128, 4)])
def test_key_margins_against_numpy(d, kb):
    """u_margin (distance of the unit rotated key to the nearest stored boundary) and p_margin
    (|S r|) decide which GPU/oracle differences the parity window forgives; both recomputed
    with scipy's Hadamard matrix and numpy's fp16 decode of S."""
    c32, b32 = O.stored_codebook(d, kb)
    sigma, S = O.tables(d, W.TABLE_SEED)
    k = _keys(d, 48, seed=21)
    r = O.quantize_keys(k, c32, b32, sigma, S, kb=kb)
    u = _rotate_numpy(sigma, k) / np.linalg.norm(k, axis=1)[:, None]
    um = np.abs(u[:, :, None] - b32[None, None, :]).min(-1)
    np.testing.assert_allclose(r["u_margin"], um, rtol=0, atol=1e-15)
    idx = np.searchsorted(b32, u, side="left")          # #{i : b_i < u}
    np.testing.assert_array_equal(r["idx"], idx)
    Sd = S.view(np.float16).astype(np.float64)
    p = (u - c32[idx]) @ Sd.T
    np.testing.assert_allclose(r["p_margin"], np.abs(p), rtol=1e-11, atol=1e-15)
    np.testing.assert_array_equal(r["z"], (p >= 0).astype(np.uint8))


def test_key_margins_hand_built_rows():
    """Unit keys with coordinates placed at chosen distances from the stored boundaries (the
    key is Pi^T u, so the rotation returns u): the margins are those distances."""
    d = 128
    c32, b32 = O.stored_codebook(d, 3)
    sigma, S = O.tables(d, W.TABLE_SEED)
    rng = np.random.default_rng(7)
    u = c32[rng.integers(0, 8, d)]                      # centroids: far from every boundary
    placed = {0: (b32[4], 3e-7), 1: (b32[5], -2e-6), 2: (b32[1], 5e-5), 3: (b32[6], -1e-6)}
    for j, (bb, delta) in placed.items():
        u[j] = 0.0
    rest = np.ones(d, bool)
    rest[list(placed)] = False
    target = 1.0 - sum((bb + delta) ** 2 for bb, delta in placed.values())
    u[rest] *= math.sqrt(target / (u[rest] ** 2).sum())
    for j, (bb, delta) in placed.items():
        u[j] = bb + delta
    assert abs(np.linalg.norm(u) - 1) < 1e-15
    far = np.abs(u[rest][:, None] - b32[None, :]).min(-1)
    assert far.min() > 1e-4
    H = scipy.linalg.hadamard(d).astype(np.float64)
    k = (sigma * (H @ u) / math.sqrt(d)) * 3.7            # Pi^T u = diag(sigma) H u / sqrt(d)
    r = O.quantize_keys(k[None], c32, b32, sigma, S)
    for j, (bb, delta) in placed.items():
        assert abs(r["u_margin"][0, j] - abs(delta)) < 1e-14, (j, r["u_margin"][0, j], delta)
    np.testing.assert_allclose(r["u_margin"][0, rest], far, rtol=0, atol=1e-14)
    assert r["idx"][0, 0] == 5 and r["idx"][0, 1] == 5 and r["idx"][0, 2] == 2 and r["idx"][0, 3] == 6


@pytest.mark.parametrize("d", [128, 256])
def test_force_idx_rederives_the_row(d):
    """A code chosen inside the rounding window changes the residual and with it every sign
    bit of the row: with force_idx the oracle keeps the given codes and recomputes gamma, the
    signs and |S r| from them (checked against numpy); the unforced rows are unchanged."""
    c32, b32 = O.stored_codebook(d, 3)
    sigma, S = O.tables(d, W.TABLE_SEED)
    k = _keys(d, 6, seed=33)
    base = O.quantize_keys(k, c32, b32, sigma, S)
    forced = base["idx"].copy()
    forced[1, 5] = min(7, forced[1, 5] + 1)
    forced[1, 40] = max(0, forced[1, 40] - 1)
    forced[4, 17] = 7 - forced[4, 17]
    assert (forced != base["idx"]).sum() == 3
    r = O.quantize_keys(k, c32, b32, sigma, S, force_idx=forced)
    np.testing.assert_array_equal(r["idx"], forced)
    u = _rotate_numpy(sigma, k) / np.linalg.norm(k, axis=1)[:, None]
    res = u - c32[forced]
    np.testing.assert_allclose(r["rnorm"], np.linalg.norm(res, axis=1), rtol=1e-12)
    p = res @ S.view(np.float16).astype(np.float64).T
    np.testing.assert_array_equal(r["z"], (p >= 0).astype(np.uint8))
    np.testing.assert_allclose(r["p_margin"], np.abs(p), rtol=1e-11, atol=1e-15)
    np.testing.assert_array_equal(r["u_margin"], base["u_margin"])
    for row in (0, 2, 3, 5):
        for key in ("z", "rnorm", "p_margin"):
            np.testing.assert_array_equal(r[key][row], base[key][row])
    assert (r["z"][1] != base["z"][1]).any() and (r["z"][4] != base["z"][4]).any()


@pytest.mark.parametrize("d", [128, 256])
def test_key_mse_reconstruction_quality_band(d):
    """cos(k, n Pi^T c[idx]) ~ sqrt(1 - D) with D = d * MSE of the codebook (~0.034)."""
    c32, b32 = O.stored_codebook(d, 3)
    sigma, S = O.tables(d, W.TABLE_SEED)
    k = _keys(d, 400, seed=5)
    r = O.quantize_keys(k, c32, b32, sigma, S)
    Pi = O.rotate(sigma, np.eye(d)).T
    khat = (c32[r["idx"]] @ Pi) * r["norm"][:, None]
    cos = (k * khat).sum(1) / np.linalg.norm(k, axis=1) / np.linalg.norm(khat, axis=1)
    assert 0.975 <= cos.mean() <= 0.99


def test_qjl_estimate_is_unbiased_over_projection_draws():
    """E_S[est<q,k>] = <q,k> (the pages' TurboQuantProd property); the MSE-only part of
    the estimate is biased (negative control)."""
    d = 128
    c32, b32 = O.stored_codebook(d, 3)
    r = np.random.default_rng(21)
    k = r.standard_normal(d)
    q = k + 0.3 * r.standard_normal(d)          # correlated pair: large <q,k>
    truth = float(q @ k)
    sigma, _ = O.tables(d, W.TABLE_SEED)
    M = 2500
    est = np.zeros(M)
    mse_only = np.zeros(M)
    for m in range(M):
        _, S = O.tables(d, 1000 + m)
        sig = sigma
        qr = O.quantize_keys(k[None], c32, b32, sig, S)
        kw = O.pack_keys(qr["idx"], qr["z"])
        kn = np.array([[qr["norm"][0], qr["rnorm"][0]]], np.float64)
        qprime = O.rotate(sig, q)[0]
        w = O.f16_bits_fast(S) @ qprime
        idx, z = O.unpack_keys(kw, d)
        n, g = kn[0]
        mse = qprime @ c32[idx[0]]
        est[m] = n * (mse + g * math.sqrt(math.pi / 2) / d * (w @ (2.0 * z[0] - 1)))
        mse_only[m] = n * mse
    sd = est.std()
    assert abs(est.mean() - truth) <= 4 * sd / math.sqrt(M)
    assert abs(mse_only.mean() - truth) > 8 * sd / math.sqrt(M)


@pytest.mark.parametrize("d,kb", [(128, 3), (64, 1), (64, 2), (64, 4), (128, 4)])
def test_decode_scores_equal_estimator(d, kb):
    """orc_decode's raw scores use the same estimator (cross-check through the decoder, which
    reads the packed record of the key width)."""
    c32, b32 = O.stored_codebook(d, kb)
    sigma, S = O.tables(d, W.TABLE_SEED)
    r = np.random.default_rng(4)
    k = r.standard_normal((5, d))
    q = r.standard_normal((1, 1, d))
    qr = O.quantize_keys(k, c32, b32, sigma, S, kb=kb)
    v = O.quantize_values(r.standard_normal((5, d)), 2)
    kw = O.pack_keys(qr["idx"], qr["z"], kb)
    kn = np.stack([qr["norm"], qr["rnorm"]], 1).astype(np.float32)
    _, sc = O.decode(d=d, kb=kb, vb=2, c32=c32, sigma=sigma, S_bits=S, B=1, Hq=1, Hkv=1,
                     kw=kw, kn=kn, vw=O.pack_values(v["code"], 2), vs=v["scale"], cap=5,
                     n_packed=5, rk=None, rv=None, buf=0, n_ring=0, q=q, scale=1.0,
                     want_scores=True)
    qprime = O.rotate(sigma, q[0, 0])[0]
    w = O.f16_bits_fast(S) @ qprime
    for t in range(5):
        n, g = float(kn[t, 0]), float(kn[t, 1])
        e = n * (qprime @ c32[qr["idx"][t]] + g * math.sqrt(math.pi / 2) / d * (w @ (2.0 * qr["z"][t] - 1)))
        assert abs(sc[0, 0, t] - e) < 1e-9 * max(1, abs(e))


# ------------------------------------------------------------------------- values

@pytest.mark.parametrize("vb", [2, 4])
def test_value_quantiser_invariants(vb):
    d = 128
    r = np.random.default_rng(9)
    v = r.standard_normal((200, d))
    v[7, :32] = 0.0                              # all-zero group -> s = 0
    res = O.quantize_values(v, vb)
    half = 1 << (vb - 1)
    s = np.repeat(O.f16_bits_fast(res["scale"]), 32, axis=1)
    vhat = O.dequant_values(res["code"], res["scale"], vb)
    assert res["code"].max() <= 2 * half - 1
    inside = (v < (half - 1) * s + s) & (s > 0) & (v >= -half * s)
    assert np.all(np.abs(v - vhat)[inside] <= s[inside] / 2 * (1 + 1e-12))
    assert np.all(res["scale"][7, 0] == 0) and np.all(res["code"][7, :32] == half)
    # the group maximum lands in the top (or, for negative maxima, bottom) level
    for row in range(10):
        for g in range(4):
            seg = v[row, 32 * g:32 * g + 32]
            j = int(np.argmax(np.abs(seg)))
            if res["scale"][row, g] == 0:
                continue
            assert res["code"][row, 32 * g + j] in (0, 2 * half - 1)
    if vb == 2:
        assert set(np.unique(res["code"])) == {0, 1, 2, 3}
    # exhaustive floor check: code - half = floor(v / s) clamped
    fl = np.clip(np.floor(v / np.where(s > 0, s, 1)), -half, half - 1) + half
    np.testing.assert_array_equal(res["code"][s > 0], fl[s > 0].astype(np.uint8))


@pytest.mark.parametrize("vb,key", [(2, "bits2"), (4, "bits4")])
def test_value_quality_band_matches_page(vb, key):
    """Page: cos_sim of 2-bit / 4-bit values at head_dim 256 (groups of 32)."""
    fig = PAGE["value_cos_sim"]
    d = fig["head_dim"]
    v = np.random.default_rng(13).standard_normal((2000, d))
    res = O.quantize_values(v, vb)
    vh = O.dequant_values(res["code"], res["scale"], vb)
    cos = ((v * vh).sum(1) / np.linalg.norm(v, axis=1) / np.linalg.norm(vh, axis=1)).mean()
    tol = 0.01 if vb == 2 else 0.002
    assert abs(cos - fig[key]) <= tol


# ------------------------------------------------------------------------- packing

def test_pack_single_bit_patterns():
    """Key word w holds coordinates 8w..8w+7 as nibbles: code in bits 0-2, sign in bit 3."""
    d = 128
    for j in (0, 1, 7, 8, 63, 127):
        for code in range(8):
            idx = np.zeros((1, d), np.uint8); idx[0, j] = code
            z = np.zeros((1, d), np.uint8)
            w = O.pack_keys(idx, z)
            expect = np.zeros(d // 8, np.uint32); expect[j // 8] = code << (4 * (j % 8))
            np.testing.assert_array_equal(w[0], expect)
        z = np.zeros((1, d), np.uint8); z[0, j] = 1
        w = O.pack_keys(np.zeros((1, d), np.uint8), z)
        expect = np.zeros(d // 8, np.uint32); expect[j // 8] = 8 << (4 * (j % 8))
        np.testing.assert_array_equal(w[0], expect)
    # values: four 2-bit codes per byte, least significant first
    code = np.zeros((1, d), np.uint8); code[0, 5] = 3
    w = O.pack_values(code, 2)
    assert w[0, 0] == 3 << 10 and w[0, 1:].sum() == 0
    assert w[0].view(np.uint8)[1] == 0b1100   # byte 1 holds codes 4..7
    code = np.zeros((1, d), np.uint8); code[0, 9] = 0xF
    w = O.pack_values(code, 4)
    assert w[0, 1] == 0xF << 4


def test_pack_key_planes_hand_computed_words():
    """Key widths 1, 2 and 4: a code plane of kb-bit fields (least significant first) and a
    sign plane of one bit per coordinate after it; the expected words are worked by hand."""
    d = 64
    j = np.arange(d)
    # kb = 2: codes 0,1,2,3,0,... -> every byte 0b11100100; signs where j % 3 == 0
    w = O.pack_keys((j % 4)[None].astype(np.uint8), (j % 3 == 0)[None].astype(np.uint8), 2)[0]
    assert w.shape == (6,)
    assert list(w[:4]) == [0xE4E4E4E4] * 4
    assert w[4] == 0x49249249 and w[5] == 0x92492492   # bits 0,3,..,30 and 1,4,..,31
    # kb = 4: codes j % 16 -> nibbles 0..7 then 8..15; signs for j < 5
    w = O.pack_keys((j % 16)[None].astype(np.uint8), (j < 5)[None].astype(np.uint8), 4)[0]
    assert w.shape == (10,)
    assert list(w[:8]) == [0x76543210, 0xFEDCBA98] * 4
    assert w[8] == 0x1F and w[9] == 0
    # kb = 1: codes j % 2 -> odd bits; signs for j >= 60
    w = O.pack_keys((j % 2)[None].astype(np.uint8), (j >= 60)[None].astype(np.uint8), 1)[0]
    assert list(w) == [0xAAAAAAAA, 0xAAAAAAAA, 0, 0xF0000000]
    # a record is (kb + 1) d / 32 words at every width
    for kb in (1, 2, 3, 4):
        assert O.key_words(128, kb) == (kb + 1) * 4 and O.key_words(64, kb) == (kb + 1) * 2


@pytest.mark.parametrize("d,kb", [(256, 3), (64, 1), (64, 2), (64, 4), (128, 2), (128, 4)])
@pytest.mark.parametrize("vb", [2, 4])
def test_pack_round_trip(vb, d, kb):
    r = np.random.default_rng(2)
    idx = r.integers(0, 1 << kb, (50, d), dtype=np.uint8)
    z = r.integers(0, 2, (50, d), dtype=np.uint8)
    i2, z2 = O.unpack_keys(O.pack_keys(idx, z, kb), d, kb)
    np.testing.assert_array_equal(i2, idx); np.testing.assert_array_equal(z2, z)
    c = r.integers(0, 1 << vb, (50, d), dtype=np.uint8)
    np.testing.assert_array_equal(O.unpack_values(O.pack_values(c, vb), d, vb), c)


# ------------------------------------------------------------------------- attention

def _softmax_attention(q, K, V, scale):
    s = K @ q * scale
    p = np.exp(s - s.max())
    return p @ V / p.sum()


def test_decode_ring_only_is_textbook_attention():
    d, G, buf = 128, 4, 128
    r = np.random.default_rng(17)
    sigma, S = O.tables(d, W.TABLE_SEED)
    c32, _ = O.stored_codebook(d, 3)
    n_ring = 37
    rk = r.standard_normal((2, buf, d)).astype(np.float16)
    rv = r.standard_normal((2, buf, d)).astype(np.float16)
    q = r.standard_normal((1, 2 * G, d))
    out = O.decode(d=d, kb=3, vb=2, c32=c32, sigma=sigma, S_bits=S, B=1, Hq=2 * G, Hkv=2,
                   kw=None, kn=None, vw=None, vs=None, cap=0, n_packed=0,
                   rk=rk.view(np.uint16), rv=rv.view(np.uint16), buf=buf, n_ring=n_ring,
                   q=q, scale=1 / math.sqrt(d))
    for h in range(2 * G):
        kv = h // G
        ref = _softmax_attention(q[0, h], rk[kv, :n_ring].astype(np.float64),
                                 rv[kv, :n_ring].astype(np.float64), 1 / math.sqrt(d))
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-12, atol=1e-14)


def test_decode_single_and_two_packed_tokens():
    d = 128
    r = np.random.default_rng(19)
    sigma, S = O.tables(d, W.TABLE_SEED)
    c32, b32 = O.stored_codebook(d, 3)
    k = r.standard_normal((2, d)); v = r.standard_normal((2, d)); q = r.standard_normal((1, 1, d))
    kq = O.quantize_keys(k, c32, b32, sigma, S)
    vq = O.quantize_values(v, 2)
    kw = O.pack_keys(kq["idx"], kq["z"]); vw = O.pack_values(vq["code"], 2)
    kn = np.stack([kq["norm"], kq["rnorm"]], 1).astype(np.float32)
    vhat = O.dequant_values(vq["code"], vq["scale"], 2)
    common = dict(d=d, kb=3, vb=2, c32=c32, sigma=sigma, S_bits=S, B=1, Hq=1, Hkv=1,
                  kw=kw, kn=kn, vw=vw, vs=vq["scale"], cap=2, rk=None, rv=None, buf=0, n_ring=0, q=q)
    o1 = O.decode(n_packed=1, scale=0.1, **common)
    np.testing.assert_allclose(o1[0, 0], vhat[0], rtol=0, atol=1e-15)
    o2, sc = O.decode(n_packed=2, scale=0.1, want_scores=True, **common)
    a = 1 / (1 + math.exp(-(sc[0, 0, 0] - sc[0, 0, 1]) * 0.1))
    np.testing.assert_allclose(o2[0, 0], a * vhat[0] + (1 - a) * vhat[1], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------- bytes formula

def test_kv_bytes_formula_matches_pages():
    f = PAGE["kv_cache_llama31_8b_32k"]
    assert W.fp16_kv_bytes(f["layers"], 1, f["kv_heads"], f["seq"], f["head_dim"]) == f["fp16_MB"] * 2**20
    g = PAGE["kv_cache_llama2_7b"]
    b2048 = W.fp16_kv_bytes(g["layers"], 1, g["heads"], 2048, g["head_dim"])
    b8192 = W.fp16_kv_bytes(g["layers"], 1, g["heads"], 8192, g["head_dim"])
    assert round(b2048 / 1e9, 2) == g["seq2048_GB"]
    assert round(b8192 / 1e9, 1) == g["seq8192_GB"]
    assert W.packed_record_bytes(128, 2) == 112 and W.packed_record_bytes(256, 4) == 280


def test_prefill_is_causal_estimator_attention():
    """The prefill oracle against numpy written from the estimator: scores
    n (q'.c[idx] + gamma sqrt(pi/2)/d w.(2z - 1)) with q' = Pi q (scipy's Hadamard matrix) and
    w = S q', a causal mask from position pos0, softmax of scale * s, bin-centre values."""
    d, kb, vb, Hq, Hkv, T, n_packed, pos0 = 64, 2, 2, 4, 2, 5, 9, 3
    c32, b32 = O.stored_codebook(d, kb)
    sigma, S = O.tables(d, W.TABLE_SEED)
    r = np.random.default_rng(23)
    k = r.standard_normal((Hkv * n_packed, d))
    v = r.standard_normal((Hkv * n_packed, d))
    q = r.standard_normal((1, T, Hq, d))
    kq = O.quantize_keys(k, c32, b32, sigma, S, kb=kb)
    vq = O.quantize_values(v, vb)
    kw = O.pack_keys(kq["idx"], kq["z"], kb).reshape(Hkv, n_packed, -1)
    kn = np.stack([kq["norm"], kq["rnorm"]], 1).astype(np.float32).reshape(Hkv, n_packed, 2)
    vw = O.pack_values(vq["code"], vb).reshape(Hkv, n_packed, -1)
    vs = vq["scale"].reshape(Hkv, n_packed, -1)
    scale = 1 / math.sqrt(d)
    common = dict(d=d, kb=kb, vb=vb, c32=c32, sigma=sigma, S_bits=S, B=1, T=T, Hq=Hq, Hkv=Hkv, kw=kw, kn=kn,
                  vw=vw, vs=vs, cap=n_packed, n_packed=n_packed, q=q, scale=scale)
    got = O.prefill(pos0=pos0, causal=True, **common)
    full = O.prefill(pos0=pos0, causal=False, **common)
    Sd = S.view(np.float16).astype(np.float64)
    idx = kq["idx"].reshape(Hkv, n_packed, d)
    z = kq["z"].reshape(Hkv, n_packed, d).astype(np.float64)
    nrm = kn[..., 0].astype(np.float64)
    gam = kn[..., 1].astype(np.float64)
    vhat = O.dequant_values(vq["code"], vq["scale"], vb).reshape(Hkv, n_packed, d)
    G = Hq // Hkv
    for i in range(T):
        for h in range(Hq):
            g = h // G
            qp = _rotate_numpy(sigma, q[0, i, h][None])[0]
            w = Sd @ qp
            s = nrm[g] * ((c32[idx[g]] @ qp) + gam[g] * math.sqrt(math.pi / 2) / d * ((2 * z[g] - 1) @ w))
            for out, n in ((got, min(n_packed, pos0 + i + 1)), (full, n_packed)):
                e = np.exp(scale * (s[:n] - s[:n].max()))
                np.testing.assert_allclose(out[0, i, h], e @ vhat[g, :n] / e.sum(), rtol=1e-10, atol=1e-12)
    # a query token past the history attends to all of it; before it (pos0 < 0 is not allowed
    # by the library) the causal window would be empty: zeros
    assert not O.prefill(pos0=-1, causal=True, **{**common, "T": 1, "q": q[:, :1]}).any()

