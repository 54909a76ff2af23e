"""Pins of the oracle's MXFP4 W4A4 arithmetic (CPU only).

The W4A4 routed experts are the OCP Microscaling (MX) analog of the NVFP4 W4A4
routed experts of the "anvil-serving" dossier (section "Quantization
boundary"): e2m1 weights with an E8M0 scale per 32 along K, and the expert's
inputs x and h quantized to MXFP4 before each product.  What fixes the
expected values here: the E2M1 value table of the OCP MX v1.0 specification,
brute-force nearest-value search, a characterization of the shared exponent,
a hand-worked fixture, numpy's BLAS product with scipy's expit, and random
perturbations for the decision slack.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# OCP MX v1.0, FP4 (E2M1): magnitude by code bits 2..0; bit 3 is the sign
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
CODE_VAL = np.concatenate([E2M1_TABLE, -E2M1_TABLE])


# ------------------------------------------------------- brute-force models

def _nearest_e2m1(y):
    """Nearest of the 16 code values (exhaustive), ties to the even mantissa
    bit (code bit 0); values past +-6 land on +-6 as the nearest."""
    y = np.asarray(y, np.float64)
    dist = np.abs(y[..., None] - CODE_VAL)
    cand = dist == dist.min(axis=-1, keepdims=True)
    even = cand & ((np.arange(16) & 1) == 0)
    pick = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))
    return CODE_VAL[pick]


def _exponent(amax):
    """The E with max|v| / 2^E in [4, 8), clamped to [-127, 127]; -127 for 0."""
    amax = np.asarray(amax, np.float64)
    E = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), 0).astype(np.int64) - 2
    for _ in range(2):  # repair log2 rounding at powers of two
        E = np.where((amax > 0) & (amax / np.ldexp(1.0, E) >= 8), E + 1, E)
        E = np.where((amax > 0) & (amax / np.ldexp(1.0, E) < 4), E - 1, E)
    return np.where(amax > 0, np.clip(E, -127, 127), -127)


def _mx_brute(v):
    v = np.asarray(v, np.float64)
    b = v.reshape(*v.shape[:-1], -1, 32)
    E = _exponent(np.abs(b).max(-1))
    X = np.ldexp(1.0, E)[..., None]
    return (_nearest_e2m1(b / X) * X).reshape(v.shape), (E + 127).astype(np.uint8)


# ------------------------------------------------------------- decoders

def test_e2m1_decoder_matches_the_ocp_table(orc):
    got = np.array([orc.e2m1_to_f64(c) for c in range(16)])
    assert np.array_equal(got, CODE_VAL)
    assert math.copysign(1.0, orc.e2m1_to_f64(8)) == -1.0  # code 8 is -0


def test_e8m0_decoder_all_bytes(orc):
    for b in range(255):
        assert orc.e8m0_to_f64(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(orc.e8m0_to_f64(255))


def test_mxfp4_matrix_decoder_nibble_order_and_scale_index(orc):
    """Byte j holds element 2j in its low nibble; scale byte (r, j // 32)."""
    rng = np.random.default_rng(40)
    rows, K = 5, 96
    codes = rng.integers(0, 16, size=(rows, K))
    sc = rng.integers(100, 150, size=(rows, K // 32)).astype(np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    want = CODE_VAL[codes] * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))
    got = orc.decode_matrix(orc.MXFP4, rows, K, q, sc)
    assert np.array_equal(got, want)


def test_mxfp4_decoder_rejects_a_nan_scale(orc):
    q = np.zeros((1, 16), np.uint8)
    sc = np.array([[255]], np.uint8)
    with pytest.raises(RuntimeError):
        orc.decode_matrix(orc.MXFP4, 1, 32, q, sc)


def test_workload_mxfp4_weights_decode_within_half_a_step(orc):
    """The input generator's codes decode to within half an e2m1 spacing of
    the drawn weights (scale chosen so nothing saturates)."""
    rng = np.random.default_rng(41)
    w = rng.standard_normal((32, 256)).astype(np.float32) * 0.03
    q, sc = W.quantize_mxfp4(w)
    dq = orc.decode_matrix(orc.MXFP4, 32, 256, q, sc)
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(w) / X
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * X
    assert np.all(np.abs(dq - w) <= half * (1 + 1e-12))
    assert np.all(a <= 6)


# ------------------------------------------------------------ quantizer

def test_e2m1_round_against_brute_force(orc):
    rng = np.random.default_rng(42)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    ys = np.concatenate([ties, -ties, CODE_VAL, [7.0, 6.5, 100.0, -1e9, 1e-300, 0.0],
                         rng.uniform(-8, 8, 5000), rng.standard_normal(2000) * 0.3])
    got = np.array([orc.e2m1_round(y) for y in ys])
    assert np.array_equal(got, _nearest_e2m1(ys))


def test_mx_exponent_characterization(orc):
    """E puts the block maximum in [4, 8) times 2^E, inside [-127, 127]."""
    rng = np.random.default_rng(43)
    amax = np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-120, 120, 4000))
    edges = np.ldexp(1.0, np.arange(-120, 120))
    amax = np.concatenate([amax, edges, np.nextafter(edges, 0), np.nextafter(edges, np.inf)])
    got = np.array([orc.mx_exponent(a) for a in amax])
    r = amax / np.ldexp(1.0, got)
    assert np.all((r >= 4) & (r < 8))
    assert orc.mx_exponent(0.0) == -127
    assert orc.mx_exponent(2.0 ** -140) == -127   # clamped below
    assert orc.mx_exponent(2.0 ** -125) == -127   # exactly at the bottom
    assert orc.mx_exponent(1.5 * 2.0 ** -124) == -126


def test_mx_quantize_against_brute_force(orc):
    rng = np.random.default_rng(44)
    v = rng.standard_normal((40, 256)) * np.ldexp(1.0, rng.integers(-20, 20, (40, 1)))
    v[3, 32:64] = 0.0                                      # a zero block
    v[5, :32] = np.ldexp(rng.integers(-6, 7, 32), -3)      # exact grid values
    out, eb = orc.mx_quantize(v)
    want, web = _mx_brute(v)
    assert np.array_equal(out, want)
    assert np.array_equal(eb, web)


def test_mx_quantize_hand_fixture(orc):
    fx = json.load(open(os.path.join(GOLDEN, "mx_quantize_hand.json")))
    for blk in fx["blocks"]:
        out, eb = orc.mx_quantize(np.array(blk["v"], np.float64))
        assert np.array_equal(out, np.array(blk["out"], np.float64)), blk["derivation"]
        assert int(eb[0]) == blk["scale_byte"], blk["derivation"]


def test_mx_quantize_invariants(orc):
    rng = np.random.default_rng(45)
    v = rng.standard_normal((30, 128)) * 3.0
    q, eb = orc.mx_quantize(v)
    q2, eb2 = orc.mx_quantize(q)                     # idempotent
    assert np.array_equal(q2, q) and np.array_equal(eb2, eb)
    for j in (-9, -1, 1, 13):                         # powers of two commute
        qj, ebj = orc.mx_quantize(np.ldexp(v, j))
        assert np.array_equal(qj, np.ldexp(q, j))
        assert np.array_equal(ebj.astype(int), eb.astype(int) + j)
    X = np.repeat(np.ldexp(1.0, eb.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(v) / X
    bound = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, np.where(a <= 6, 1.0, a - 6))) * X
    assert np.all(np.abs(q - v) <= bound * (1 + 1e-12))


# ----------------------------------------------------------- W4A4 layer

def _mx_inputs(seed, T, d, E, F, Fs=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    mats = {}
    for nm, shape in (("wg", (E, F, d)), ("wu", (E, F, d)), ("wd", (E, d, F))):
        w = rng.standard_normal(shape).astype(np.float32) / np.sqrt(shape[-1])
        parts = [W.quantize_mxfp4(w[e]) for e in range(E)]
        mats[nm] = np.stack([p[0] for p in parts])
        mats[nm + "_s"] = np.stack([p[1] for p in parts])
    inp = dict(x=x, **mats)
    if Fs:
        for nm, shape in (("sg", (Fs, d)), ("su", (Fs, d)), ("sd", (d, Fs))):
            inp[nm] = (rng.standard_normal(shape) / np.sqrt(shape[-1])).astype(np.float32)
    return inp


def _np_decode(q, sc):
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(*q.shape[:-1], -1)
    return CODE_VAL[codes] * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=-1))


def _np_w4a4(X, w, wg, wu, wd):
    """numpy/BLAS + scipy: Wd MX(w * silu(Wg MX(x)) * Wu MX(x)), MX by brute force."""
    xq, _ = _mx_brute(X)
    g = xq @ wg.T
    h = w[:, None] * (g * sps.expit(g)) * (xq @ wu.T)
    hq, _ = _mx_brute(h)
    return hq @ wd.T


def _spec(d, E, k, F, n_shared=0, Fs=0, sf=0):
    import oracle
    return dict(d=d, E=E, k=k, F=F, n_shared=n_shared, Fs=Fs, x_fmt=oracle.F32,
                expert_fmt=oracle.MXFP4, shared_fmt=sf)


def test_w4a4_dense_E1_k1_against_numpy(orc):
    T, d, F = 23, 128, 96
    inp = _mx_inputs(46, T, d, 1, F)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    y, oa, _ = orc.moe_experts(_spec(d, 1, 1, F), inp, ids, w)
    want = _np_w4a4(inp["x"].astype(np.float64), np.ones(T), _np_decode(inp["wg"][0], inp["wg_s"][0]),
                    _np_decode(inp["wu"][0], inp["wu_s"][0]), _np_decode(inp["wd"][0], inp["wd_s"][0]))
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oa, want, rtol=1e-11, atol=1e-12)


def test_w4a4_forced_routing_folds_the_weight_before_quantizing_h(orc):
    """y = sum_s E_{id_s}(x; w_s) + S(x): the router weight is folded into h
    before h is quantized, and the shared expert sees the unquantized x."""
    T, d, E, F, Fs = 11, 64, 4, 64, 32
    inp = _mx_inputs(47, T, d, E, F, Fs)
    ids = np.tile(np.array([[2, 0]], np.int32), (T, 1))
    w = np.tile(np.array([[0.6, 0.4]]), (T, 1))
    y, oa, so = orc.moe_experts(_spec(d, E, 2, F, 1, Fs, orc.F32), inp, ids, w)
    X = inp["x"].astype(np.float64)
    dec = lambda nm, e: _np_decode(inp[nm][e], inp[nm + "_s"][e])
    ex = lambda e, wt: _np_w4a4(X, np.full(T, wt), dec("wg", e), dec("wu", e), dec("wd", e))
    S = X @ inp["sg"].T.astype(np.float64)
    S = ((S * sps.expit(S)) * (X @ inp["su"].T.astype(np.float64))) @ inp["sd"].T.astype(np.float64)
    np.testing.assert_allclose(so, S, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oa.reshape(T, 2, d)[:, 0], ex(2, 0.6), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y, ex(2, 0.6) + ex(0, 0.4) + S, rtol=1e-11, atol=1e-12)
    # folding after the quantization would be a different (wrong) layer
    assert np.max(np.abs(ex(2, 0.6) - 0.6 * ex(2, 1.0))) > 1e-3


# ------------------------------------------------------ decision slack

def test_mx_slack_bounds_every_perturbation(orc):
    """delta_j bounds |MX(h')_j - MX(h)_j| for every h' within dh of h (the
    box's corners, random points, and each coordinate alone at its ends), and
    slack = |wd| delta bounds the change of wd MX(h').  Planted: block 0
    (scale 2^-2) holds values on either side of the 1.75 tie; block 1
    a maximum just below 2 (the exponent may rise); block 2 a maximum just
    above 4 (the exponent may fall); block 3 nothing near a decision."""
    rng = np.random.default_rng(48)
    F, d = 128, 40
    h = np.clip(rng.standard_normal(F) * 0.5, -1.5, 1.5)
    h[0] = 1.9
    h[3] = 0.4375 * (1 - 1e-6)
    h[4] = -0.4375 * (1 + 1e-6)
    h[5] = 0.4375 * (1 + 1e-6)
    h[40] = 2.0 * (1 - 1e-7)
    h[70] = 4.0 * (1 + 1e-7)
    dh = np.abs(h) * 1e-5 + 1e-12
    wd = rng.standard_normal((d, F))
    hq, delta, slack, mag = orc.mx_slack(h, dh, wd)
    assert np.array_equal(hq, _mx_brute(h)[0])
    np.testing.assert_allclose(mag, np.abs(wd) @ np.abs(hq), rtol=1e-12)
    np.testing.assert_allclose(slack, np.abs(wd) @ delta, rtol=1e-12)
    assert delta[3] > 0 and delta[4] > 0 and delta[5] > 0 and np.all(delta[96:] == 0)
    assert np.any(delta[32:64] > 0) and np.any(delta[64:96] > 0)
    pts = [h + dh * s for s in rng.choice([-1.0, 1.0], size=(3000, F))]
    pts += [h + dh * rng.uniform(-1, 1, F) for _ in range(1000)]
    for j in range(F):
        for s in (-1.0, 1.0):
            p = h.copy()
            p[j] += s * dh[j]
            pts.append(p)
    P = np.array(pts)
    Q = _mx_brute(P)[0]
    reach = np.abs(Q - hq).max(axis=0)
    assert np.all(reach <= delta)
    assert np.all(np.abs((Q - hq) @ wd.T) <= slack * (1 + 1e-12) + 1e-300)
    # every delta is reached by some point of the box (the bound is tight)
    np.testing.assert_array_equal(reach, delta)


def test_w4a4_bounds_layer_agrees_and_covers_an_fp32_computation(orc):
    """moe_experts_mx returns the same layer as moe_experts; with no error its
    slack is zero; and a float32 computation of the experts (numpy BLAS, the
    quantizations by brute force) lies within gamma*(mag + slack) + slack of
    the oracle for the error constants the GPU parity tests use."""
    T, d, E, F = 300, 256, 3, 128
    inp = _mx_inputs(49, T, d, E, F)
    rng = np.random.default_rng(50)
    ids = np.stack([rng.permutation(E)[:2] for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet([1, 1], T)
    spec = _spec(d, E, 2, F)
    y0, oa0, _ = orc.moe_experts(spec, inp, ids, w)
    y1, oa1, _, sl0, mag0 = orc.moe_experts_mx(spec, inp, ids, w, 0.0, 0.0)
    assert np.array_equal(oa0, oa1) and np.array_equal(y0, y1) and np.all(sl0 == 0)
    g_gu, g_dn, eta = (d / 16 + 8) * 2.0 ** -24, (F / 16 + 8) * 2.0 ** -24, 2.0 ** -16
    _, oa, _, slack, mag = orc.moe_experts_mx(spec, inp, ids, w, g_gu, eta)
    assert np.array_equal(oa, oa0)
    x32 = _mx_brute(inp["x"].astype(np.float64))[0].astype(np.float32)
    f32 = np.float32
    for e in range(E):
        dec = lambda nm: _np_decode(inp[nm][e], inp[nm + "_s"][e]).astype(np.float32)
        rows = np.nonzero(ids == e)
        f = rows[0] * 2 + rows[1]
        g = x32[rows[0]] @ dec("wg").T
        u = x32[rows[0]] @ dec("wu").T
        h = w[rows].astype(f32)[:, None] * (g / (f32(1) + np.exp(-g))) * u
        out32 = _mx_brute(h.astype(np.float64))[0].astype(np.float32) @ dec("wd").T
        err = np.abs(out32.astype(np.float64) - oa[f])
        assert np.all(err <= g_dn * (mag[f] + slack[f]) + slack[f]), e
