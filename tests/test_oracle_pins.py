"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected result: an exhaustive brute force, a
closed form, an invariant of the mathematics, a hand-worked fixture, or an
independent library routine (numpy's BLAS product, numpy's stable argsort,
scipy's softmax / expit, torch's bfloat16 and numpy's float16 decoders).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoders

def test_f16_decoder_exhaustive(orc):
    """All 65,536 binary16 patterns against numpy's float16."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(b) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_decoder_exhaustive(orc):
    """All 65,536 bfloat16 patterns against torch.bfloat16."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_matrix(orc.BF16, 1, 65536, bits)[0]
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_int4_nibble_order_and_sign_all_bytes(orc):
    """Every byte value: low nibble is the even element, two's complement codes."""
    K = 512
    row = np.arange(256, dtype=np.uint8)                       # 256 bytes = 512 nibbles
    scales = np.full(K // 32, 0x3C00, np.uint16)                 # fp16 1.0
    got = orc.decode_matrix(orc.I4G32, 1, K, row, scales)[0]
    lo = np.array([(b & 15) - 16 * ((b & 15) >= 8) for b in range(256)])
    hi = np.array([(b >> 4) - 16 * ((b >> 4) >= 8) for b in range(256)])
    assert np.array_equal(got[0::2], lo) and np.array_equal(got[1::2], hi)


def test_int4_group_scale_indexing(orc):
    """Scale j//32 of row r multiplies element (r, j): a distinct power of two per
    (row, group) makes any transposed or shifted scale index visible."""
    rows, K = 3, 128
    q = np.ones((rows, K), np.int8)
    packed = W.pack_int4(q)
    exps = np.arange(rows * (K // 32)).reshape(rows, K // 32)      # scale = 2^-e
    scales = np.array(2.0 ** -exps, np.float16).view(np.uint16)
    got = orc.decode_matrix(orc.I4G32, rows, K, packed, scales)
    want = np.repeat(2.0 ** -exps, 32, axis=1)
    assert np.array_equal(got, want)


def test_int8_row_decoder_all_codes(orc):
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(2, 128)
    s = np.array([0.5, -3.0], np.float16).view(np.uint16)
    got = orc.decode_matrix(orc.I8ROW, 2, 128, q, s)
    assert np.array_equal(got, q.astype(np.float64) * np.array([[0.5], [-3.0]]))


@pytest.mark.parametrize("b", sorted(W.IG32))
def test_bbit_decoder_every_code_and_group_scale_index(orc, b):
    """b-bit group-32 codes: every code of the symmetric range decodes to
    code * scale(row, j // 32), with a distinct power-of-two scale per
    (row, group) so a shifted or transposed scale index shows."""
    lim = (1 << (b - 1)) - 1
    codes = np.arange(-lim, lim + 1)
    rows, K = 3, 32 * ((len(codes) + 31) // 32 + 1)
    q = np.resize(codes, rows * K).reshape(rows, K).astype(np.int8)
    g = np.arange(K // 32)[None, :]
    exps = (g + 5 * np.arange(rows)[:, None]) % 15     # normal fp16 powers of two
    scales = np.array(2.0 ** -exps, np.float16).view(np.uint16)
    got = orc.decode_matrix(orc.FMT_NAMES[W.IG32[b]], rows, K, q, scales)
    assert np.array_equal(got, q.astype(np.float64) * np.repeat(2.0 ** -exps, 32, axis=1))


@pytest.mark.parametrize("b", sorted(W.IG32))
def test_bbit_decoder_rejects_codes_outside_the_range(orc, b):
    lim = (1 << (b - 1)) - 1
    s = np.full(1, 0x3C00, np.uint16)
    for bad in (lim + 1, -lim - 1):
        if not -128 <= bad <= 127:
            continue
        q = np.zeros(32, np.int8)
        q[9] = bad
        with pytest.raises(RuntimeError):
            orc.decode_matrix(orc.FMT_NAMES[W.IG32[b]], 1, 32, q, s)


def test_8bit_groups_with_one_scale_per_row_equal_int8_rows(orc):
    """8-bit group-32 codes whose groups share one scale per row decode exactly
    like the int8 per-row format (a different decoder of the same values)."""
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, size=(5, 96)).astype(np.int8)
    row_s = np.array(rng.uniform(0.01, 2.0, 5), np.float16)
    g = orc.decode_matrix(orc.I8G32, 5, 96, q, np.repeat(row_s.view(np.uint16)[:, None], 3, axis=1))
    r = orc.decode_matrix(orc.I8ROW, 5, 96, q, row_s.view(np.uint16))
    assert np.array_equal(g, r)


@pytest.mark.parametrize("fmt,bound_div", [(W.I4G32, 2.0), (W.I8ROW, 2.0)]
                         + [(f, 2.0) for f in W.IG32.values()])
def test_quantize_roundtrip_bound(orc, fmt, bound_div):
    """Symmetric round-to-nearest: |decode(quantize(w)) - w| <= s/2 (+ fp16 slack)."""
    rng = np.random.default_rng(7)
    w = rng.standard_normal((64, 256)).astype(np.float32) * 0.02
    q, s = W.store(w, fmt)
    dec = orc.decode_matrix(orc.FMT_NAMES[fmt], 64, 256, q, s)
    sv = s.view(np.float16).astype(np.float64)
    per = sv[:, None] if fmt == W.I8ROW else np.repeat(sv, 32, axis=1)
    # the scale is fp16-rounded, so max|w|/s may exceed the top code by < 1 ulp
    assert np.all(np.abs(dec - w) <= per / bound_div * (1 + 2e-3) + 1e-12)


# ------------------------------------------------------------- stable top-k

def _brute_topk(l, k):
    """rank(e) = #{j : l_j > l_e or (l_j == l_e and j < e)}; slot s = rank s."""
    E = len(l)
    rank = [sum(1 for j in range(E) if l[j] > l[e] or (l[j] == l[e] and j < e)) for e in range(E)]
    return [rank.index(s) for s in range(k)]


@pytest.mark.parametrize("E", [1, 3, 5, 7])
def test_topk_exhaustive_small(orc, E):
    """Every logit vector in {0,1,2}^E and every k: oracle == brute-force ranks."""
    pats = np.array(np.meshgrid(*[[0.0, 1.0, 2.0]] * E, indexing="ij")).reshape(E, -1).T
    for k in range(1, E + 1):
        ids, w = orc.topk_softmax(pats, k)
        want = np.array([_brute_topk(list(p), k) for p in pats])
        assert np.array_equal(ids, want), (E, k)


def test_topk_exhaustive_E8(orc):
    pats = np.array(np.meshgrid(*[[0.0, 1.0, 2.0]] * 8, indexing="ij")).reshape(8, -1).T
    for k in (1, 2, 5, 8):
        ids, _ = orc.topk_softmax(pats, k)
        want = np.array([_brute_topk(list(p), k) for p in pats])
        assert np.array_equal(ids, want)


def test_topk_random_large_E_against_stable_argsort(orc):
    """E=512, k=10 with heavy ties: numpy's stable argsort of -logits is the same order."""
    rng = np.random.default_rng(3)
    L = rng.integers(-4, 5, size=(200, 512)).astype(np.float64)
    ids, _ = orc.topk_softmax(L, 10)
    want = np.argsort(-L, axis=1, kind="stable")[:, :10]
    assert np.array_equal(ids, want)


def test_topk_signed_zero_is_a_tie(orc):
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    ids, w = orc.topk_softmax(L, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]


def test_topk_rejects_nonfinite(orc):
    with pytest.raises(RuntimeError):
        orc.topk_softmax(np.array([[0.0, np.nan, 1.0]]), 1)


def test_topk_golden_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "topk_hand.json")))
    L = np.array([[float(v) for v in row] for row in g["logits"]])
    assert math.copysign(1.0, L[0, 3]) < 0          # the fixture holds a real -0.0
    ids, w = orc.topk_softmax(L, g["k"])
    assert ids.tolist() == g["ids"]
    want = np.array([[eval(e, {"exp": math.exp}) for e in row] for row in g["weights_closed_form"]])
    np.testing.assert_allclose(w, want, rtol=1e-15, atol=1e-16)


# -------------------------------------------------------------- softmax

def test_softmax_properties_and_scipy(orc):
    rng = np.random.default_rng(11)
    L = rng.standard_normal((300, 64)) * 3
    for k in (1, 2, 10, 64):
        ids, w = orc.topk_softmax(L, k)
        assert np.all(np.abs(w.sum(1) - 1) <= 4e-16 * k)
        assert np.all(np.diff(w, axis=1) <= 0)                  # non-increasing by slot
        chosen = np.take_along_axis(L, ids.astype(np.int64), 1)
        np.testing.assert_allclose(w, sps.softmax(chosen, axis=1), rtol=1e-13, atol=1e-300)
        if k == 1:
            assert np.all(w == 1.0)
    ids, w = orc.topk_softmax(np.full((3, 16), 0.25), 4)
    assert np.allclose(w, 0.25, rtol=0, atol=1e-16)


def test_softmax_shift_invariance(orc):
    rng = np.random.default_rng(5)
    L = rng.standard_normal((50, 32))
    ids1, w1 = orc.topk_softmax(L, 6)
    ids2, w2 = orc.topk_softmax(L + 1000.0, 6)
    assert np.array_equal(ids1, ids2)
    np.testing.assert_allclose(w1, w2, rtol=1e-11)


# ----------------------------------------------------------- route plan

def test_route_plan_golden_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "route_plan_hand.json")))
    off, perm, inv = orc.route_plan(np.array(g["ids"]), g["E"])
    assert off.tolist() == g["offsets"]
    assert perm.tolist() == g["perm"]
    assert inv.tolist() == g["inv_perm"]


@pytest.mark.parametrize("n,E", [(0, 8), (1, 1), (1000, 7), (40960, 512), (163, 512)])
def test_route_plan_invariants_and_argsort(orc, n, E):
    rng = np.random.default_rng(n + E)
    ids = rng.integers(0, E, size=n).astype(np.int32)
    off, perm, inv = orc.route_plan(ids, E)
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(ids, minlength=E))
    assert np.array_equal(perm, np.argsort(ids, kind="stable"))          # library sort
    assert np.array_equal(np.sort(perm), np.arange(n))                    # bijection
    assert np.array_equal(inv[perm], np.arange(n))
    for e in range(E):
        grp = perm[off[e]:off[e + 1]]
        assert np.all(ids[grp] == e) and np.all(np.diff(grp) > 0)


# ---------------------------------------------------------------- router

def test_router_integer_exact(orc):
    """Small integers: fp64 logits equal the int64 product exactly."""
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, size=(20, 96))
    wr = rng.integers(-3, 4, size=(40, 96))
    got = orc.router_logits(x.astype(np.float32), orc.F32, wr.astype(np.float32), orc.F32, 96, 40)
    assert np.array_equal(got, (x @ wr.T).astype(np.float64))


def test_router_against_blas_with_bias_and_bf16(orc):
    rng = np.random.default_rng(4)
    x = W.to_bf16_bits(rng.standard_normal((33, 256)).astype(np.float32))
    wr = W.to_bf16_bits(rng.standard_normal((24, 256)).astype(np.float32) / 16)
    bias = rng.standard_normal(24).astype(np.float32)
    got = orc.router_logits(x, orc.BF16, wr, orc.BF16, 256, 24, bias=bias,
                            tokens=np.array([32, 0, 5]))
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    wf = W.bf16_bits_to_f32(wr).astype(np.float64)
    want = xf[[32, 0, 5]] @ wf.T + bias.astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- experts

def _spec(d, E, k, F, n_shared=0, Fs=0, x_fmt=0, ef=0, sf=0):
    return dict(d=d, E=E, k=k, F=F, n_shared=n_shared, Fs=Fs, x_fmt=x_fmt, expert_fmt=ef,
                shared_fmt=sf)


def _np_swiglu(X, wg, wu, wd):
    """numpy/BLAS + scipy expit: Wd (silu(Wg x) * Wu x)."""
    g = X @ wg.T
    return ((g * sps.expit(g)) * (X @ wu.T)) @ wd.T


def test_dense_reduction_E1_k1_against_blas(orc):
    """E=1, k=1, no shared expert: the layer is a dense SwiGLU MLP (weight 1)."""
    rng = np.random.default_rng(8)
    T, d, F = 17, 96, 40
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = rng.standard_normal((1, F, d)).astype(np.float32) / 8
    wu = rng.standard_normal((1, F, d)).astype(np.float32) / 8
    wd = rng.standard_normal((1, d, F)).astype(np.float32) / 6
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    y, oa, _ = orc.moe_experts(_spec(d, 1, 1, F), dict(x=x, wg=wg, wu=wu, wd=wd), ids, w)
    want = _np_swiglu(x.astype(np.float64), wg[0].astype(np.float64), wu[0].astype(np.float64),
                      wd[0].astype(np.float64))
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oa, want, rtol=1e-12, atol=1e-12)


def test_forced_routing_equals_dense_sum_with_shared(orc):
    """Routing forced to experts (3, 1) with known weights, plus a shared expert:
    y = w0*E3(x) + w1*E1(x) + S(x), each term a BLAS product."""
    rng = np.random.default_rng(9)
    T, d, E, F, Fs = 9, 64, 5, 32, 48
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = rng.standard_normal((E, F, d)).astype(np.float32) / 8
    wu = rng.standard_normal((E, F, d)).astype(np.float32) / 8
    wd = rng.standard_normal((E, d, F)).astype(np.float32) / 6
    sg = rng.standard_normal((Fs, d)).astype(np.float32) / 8
    su = rng.standard_normal((Fs, d)).astype(np.float32) / 8
    sd = rng.standard_normal((d, Fs)).astype(np.float32) / 7
    ids = np.tile(np.array([[3, 1]], np.int32), (T, 1))
    w = np.tile(np.array([[0.7, 0.3]]), (T, 1))
    inp = dict(x=x, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    y, oa, so = orc.moe_experts(_spec(d, E, 2, F, 1, Fs), inp, ids, w)
    X = x.astype(np.float64)
    f = lambda e: _np_swiglu(X, wg[e].astype(np.float64), wu[e].astype(np.float64), wd[e].astype(np.float64))
    S = _np_swiglu(X, sg.astype(np.float64), su.astype(np.float64), sd.astype(np.float64))
    np.testing.assert_allclose(y, 0.7 * f(3) + 0.3 * f(1) + S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(so, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oa.reshape(T, 2, d)[:, 0], 0.7 * f(3), rtol=1e-12, atol=1e-12)


def _tiny_inputs(seed=12, T=24, d=64, E=6, F=32, Fs=32, fmt=W.F32, sfmt=W.F32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    st = lambda a: W.store(a, fmt)
    ex = [tuple(st(rng.standard_normal(s).astype(np.float32) / 8) for s in ((F, d), (F, d), (d, F)))
          for _ in range(E)]
    inp = dict(x=x)
    for i, nm in enumerate(("wg", "wu", "wd")):
        inp[nm] = np.stack([e[i][0] for e in ex])
        if ex[0][i][1] is not None:
            inp[nm + "_s"] = np.stack([e[i][1] for e in ex])
    for nm, s in (("sg", (Fs, d)), ("su", (Fs, d)), ("sd", (d, Fs))):
        q, sc = W.store(rng.standard_normal(s).astype(np.float32) / 8, sfmt)
        inp[nm] = q
        if sc is not None:
            inp[nm + "_s"] = sc
    wr = rng.standard_normal((E, d)).astype(np.float32)
    return inp, wr


def _layer(orc, inp, wr, spec, tokens=None):
    x = inp["x"]
    L = orc.router_logits(x, orc.F32, wr, orc.F32, spec["d"], spec["E"], tokens=tokens)
    ids, w = orc.topk_softmax(L, spec["k"])
    y, oa, so = orc.moe_experts(spec, inp, ids, w, tokens=tokens)
    return y, ids, w


def test_zero_input_gives_exact_zero(orc):
    inp, wr = _tiny_inputs()
    inp["x"] = np.zeros_like(inp["x"])
    spec = _spec(64, 6, 2, 32, 1, 32)
    y, _, _ = _layer(orc, inp, wr, spec)
    assert np.all(y == 0.0)


def test_token_permutation_equivariance(orc):
    inp, wr = _tiny_inputs()
    spec = _spec(64, 6, 3, 32, 1, 32)
    y, _, _ = _layer(orc, inp, wr, spec)
    p = np.random.default_rng(1).permutation(inp["x"].shape[0])
    inp2 = dict(inp, x=inp["x"][p])
    y2, _, _ = _layer(orc, inp2, wr, spec)
    np.testing.assert_allclose(y2, y[p], rtol=0, atol=1e-13)


def test_expert_relabeling_invariance(orc):
    """Relabel experts (weights and router rows together): y is unchanged."""
    inp, wr = _tiny_inputs()
    spec = _spec(64, 6, 2, 32, 1, 32)
    y, _, _ = _layer(orc, inp, wr, spec)
    p = np.array([4, 2, 0, 5, 1, 3])
    inp2 = dict(inp, wg=inp["wg"][p], wu=inp["wu"][p], wd=inp["wd"][p])
    y2, _, _ = _layer(orc, inp2, wr[p], spec)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-13)


def test_token_subset_matches_full(orc):
    inp, wr = _tiny_inputs()
    spec = _spec(64, 6, 2, 32, 1, 32)
    y, _, _ = _layer(orc, inp, wr, spec)
    sub = np.array([5, 0, 23, 5])
    ys, _, _ = _layer(orc, inp, wr, spec, tokens=sub)
    np.testing.assert_allclose(ys, y[sub], rtol=0, atol=1e-14)


def test_fold_before_down_equals_weight_after(orc):
    """By linearity Wd (w h) == w (Wd h): the fold point cannot change the result."""
    rng = np.random.default_rng(21)
    d, F = 48, 20
    x = rng.standard_normal((1, d))
    wg, wu = rng.standard_normal((F, d)) / 7, rng.standard_normal((F, d)) / 7
    wd = rng.standard_normal((d, F)) / 5
    o = orc.swiglu_dense(x, wg, wu, wd)
    g = wg @ x[0]
    h = g * sps.expit(g) * (wu @ x[0])
    for wgt in (0.3, 0.9):
        np.testing.assert_allclose(wd @ (wgt * h), wgt * o[0], rtol=1e-13, atol=1e-15)


def test_quantized_layer_equals_decoded_f32_layer(orc):
    """int4/int8 storage: the layer equals the same layer on the decoded values
    (decoded by numpy from the format definition, held exactly in fp32)."""
    inp, wr = _tiny_inputs(fmt=W.I4G32, sfmt=W.I8ROW)
    spec_q = _spec(64, 6, 2, 32, 1, 32, 0, orc.I4G32, orc.I8ROW)

    def dec4(q, s):
        u = np.stack([q & 15, q >> 4], axis=-1).reshape(*q.shape[:-1], -1).astype(np.int16)
        v = np.where(u >= 8, u - 16, u).astype(np.float64)
        return v * np.repeat(s.view(np.float16).astype(np.float64), 32, axis=-1)

    def dec8(q, s):
        return q.astype(np.float64) * s.view(np.float16).astype(np.float64)[:, None]

    inp_f = dict(x=inp["x"], wg=dec4(inp["wg"], inp["wg_s"]).astype(np.float32),
                 wu=dec4(inp["wu"], inp["wu_s"]).astype(np.float32),
                 wd=dec4(inp["wd"], inp["wd_s"]).astype(np.float32),
                 sg=dec8(inp["sg"], inp["sg_s"]).astype(np.float32),
                 su=dec8(inp["su"], inp["su_s"]).astype(np.float32),
                 sd=dec8(inp["sd"], inp["sd_s"]).astype(np.float32))
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):                 # exact in fp32
        assert np.array_equal(inp_f[k].astype(np.float64),
                              (dec4 if k[0] == "w" else dec8)(inp[k], inp[k + "_s"]))
    y_q, _, _ = _layer(orc, inp, wr, spec_q)
    y_f, _, _ = _layer(orc, inp_f, wr, _spec(64, 6, 2, 32, 1, 32))
    np.testing.assert_allclose(y_q, y_f, rtol=0, atol=1e-13)


@pytest.mark.parametrize("b", [2, 3, 6])
def test_bbit_layer_equals_decoded_f32_layer(orc, b):
    """b-bit group-32 routed experts: the layer equals the same layer on the
    decoded values (numpy: code * fp16 group scale, exact in fp32)."""
    fmt = W.IG32[b]
    inp, wr = _tiny_inputs(fmt=fmt, sfmt=W.I8ROW)
    spec_q = _spec(64, 6, 2, 32, 1, 32, 0, orc.FMT_NAMES[fmt], orc.I8ROW)

    def decb(q, s):
        return q.astype(np.float64) * np.repeat(s.view(np.float16).astype(np.float64), 32, axis=-1)

    def dec8(q, s):
        return q.astype(np.float64) * s.view(np.float16).astype(np.float64)[:, None]

    inp_f = dict(x=inp["x"], wg=decb(inp["wg"], inp["wg_s"]).astype(np.float32),
                 wu=decb(inp["wu"], inp["wu_s"]).astype(np.float32),
                 wd=decb(inp["wd"], inp["wd_s"]).astype(np.float32),
                 sg=dec8(inp["sg"], inp["sg_s"]).astype(np.float32),
                 su=dec8(inp["su"], inp["su_s"]).astype(np.float32),
                 sd=dec8(inp["sd"], inp["sd_s"]).astype(np.float32))
    lim = (1 << (b - 1)) - 1
    assert max(np.abs(inp[k]).max() for k in ("wg", "wu", "wd")) <= lim
    y_q, _, _ = _layer(orc, inp, wr, spec_q)
    y_f, _, _ = _layer(orc, inp_f, wr, _spec(64, 6, 2, 32, 1, 32))
    np.testing.assert_allclose(y_q, y_f, rtol=0, atol=1e-13)


# -------------------------------------------------- seeded workload sanity

@pytest.mark.slow
def test_zipf_bias_gives_about_ten_times_mean_load(orc):
    """The skewed T=16384 input: hottest expert ~10x the mean load (fp64 routing)."""
    cfg = W.CONFIGS["zipf_T16384"]
    x, wr, bias = W.hidden(cfg), W.router_weights(cfg), W.zipf_bias(cfg)
    L = orc.router_logits(x, orc.BF16, wr, orc.BF16, cfg.d, cfg.E, bias=bias)
    ids, _ = orc.topk_softmax(L, cfg.k)
    cnt = np.bincount(ids.ravel(), minlength=cfg.E)
    ratio = cnt.max() / cnt.mean()
    assert 8.0 <= ratio <= 12.0, ratio
