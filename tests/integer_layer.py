"""Integer-valued layers whose every intermediate is an exact integer.

Hidden states, router weights and expert codes are small integers (codes in
[-7, 7], or the format's narrower range) and every group or row scale is
1.0, so the router logits and the gate and up pre-activations g = Wg x and
u = Wu x are exact integers in fp32 accumulation.  Each token also carries B
constant "bias" columns (value 8) on which every gate row has a positive
code, which lifts every gate pre-activation to about 256, and at least 40:
there exp(-g) is below half an ulp of 1 in both fp32 and fp64, so
SiLU(g) = g exactly.  With k = 1 the routing weight
is exactly 1.  Then h = g * u is an exact integer, stored as bf16 (round to
nearest even), the down product of those integers is exact while every
partial sum stays below 2^24, and so are out_assign, shared_out and y up to
y's own bf16 rounding.  ``reference`` computes all of them with int64
matrix products.

The up rows have code 0 on the bias columns, so u spans both signs.  An
error of one in g or in u moves g * u by |u| or by g; with g near 256 and
|u| mostly below 100 that is about half a bf16 spacing of g * u or more, so
it changes the stored h in most elements and the exact comparison sees it.
The builder checks every range the argument needs.
"""
from __future__ import annotations

import numpy as np

import workloads as W

ONE_F16 = np.uint16(0x3C00)


def max_code(fmt: str) -> int:
    """Largest code the builder uses: 7, or the format's own maximum below it."""
    if fmt in (W.I4G32, W.BF16, W.I8ROW):
        return 7
    return min(7, (1 << (W.IG32_BITS[fmt] - 1)) - 1)


def _store(codes: np.ndarray, fmt: str):
    """Integer codes [rows, K] in ``fmt`` with every scale 1.0: (q, scales)."""
    rows, K = codes.shape
    if fmt == W.BF16:
        return W.to_bf16_bits(codes.astype(np.float32)), None
    if fmt == W.I4G32:
        return W.pack_int4(codes), np.full((rows, K // 32), ONE_F16, np.uint16)
    if fmt == W.I8ROW:
        return codes.astype(np.int8), np.full(rows, ONE_F16, np.uint16)
    return codes.astype(np.int8), np.full((rows, K // 32), ONE_F16, np.uint16)


def _ffn_codes(rng, rows, d, B, c, c_bias):
    """gate, up [rows, d] and down [d, rows] integer codes in [-c, c]; the
    gate's bias columns hold c_bias, the up's 0."""
    g = rng.integers(-c, c + 1, size=(rows, d))
    g[:, :B] = c_bias
    u = rng.integers(-c, c + 1, size=(rows, d))
    u[:, :B] = 0
    dn = rng.integers(-c, c + 1, size=(d, rows))
    return g, u, dn


def build(name: str, T: int, E: int, expert: str, *, d: int = 256, F: int = 256,
          n_shared: int = 1, Fs: int = 128, seed: int = 0):
    """(cfg, inputs, ints): a k = 1 layer of integer codes; ``ints`` holds the
    int64 matrices the reference multiplies."""
    cfg = W.LayerConfig(name, 900 + seed, T=T, d=d, E=E, k=1, F=F, n_shared=n_shared, Fs=Fs,
                        act=W.BF16, router=W.BF16, expert=expert, shared=W.I8ROW)
    rng = np.random.default_rng(7000 + seed)
    c = max_code(expert)
    B = -(-256 // (8 * c))  # bias columns: every gate pre-activation near 256
    # nonzero share of the other columns: the spread of g about 28
    var = c * (c + 1) / 3.0  # of a code uniform on [-c, c]
    p = min(0.5, 28.0 ** 2 / ((d - B) * var))
    x = rng.choice(np.array([-1, 0, 1]), p=[p / 2, 1 - p, p / 2], size=(T, d)).astype(np.int64)
    x[:, :B] = 8
    wr = rng.integers(-1, 2, size=(E, d)).astype(np.int64)
    wr[:, :B] = 0  # no constant logit shift per expert
    ints = dict(x=x, wr=wr, B=B, wg=[], wu=[], wd=[])
    inp = {"x": W.to_bf16_bits(x.astype(np.float32)),
           "wr": W.to_bf16_bits(wr.astype(np.float32)), "bias": None}
    parts = {n: [] for n in ("wg", "wg_s", "wu", "wu_s", "wd", "wd_s")}
    for _ in range(E):
        g, u, dn = _ffn_codes(rng, F, d, B, c, c)
        ints["wg"].append(g), ints["wu"].append(u), ints["wd"].append(dn)
        for n, m in (("wg", g), ("wu", u), ("wd", dn)):
            q, s = _store(m, expert)
            parts[n].append(q)
            parts[n + "_s"].append(s)
    for n in ("wg", "wu", "wd"):
        inp[n] = np.stack(parts[n])
        if parts[n + "_s"][0] is not None:
            inp[n + "_s"] = np.stack(parts[n + "_s"])
    if n_shared:
        g, u, dn = _ffn_codes(rng, Fs, d, B, c, c)
        ints.update(sg=g, su=u, sd=dn)
        for n, m in (("sg", g), ("su", u), ("sd", dn)):
            inp[n], inp[n + "_s"] = _store(m, W.I8ROW)
    _check_ranges(ints, n_shared)
    return cfg, inp, ints


def _bf16_round(v: np.ndarray) -> np.ndarray:
    """Integers below 2^24 in magnitude -> their bf16 (RNE) values, exact."""
    assert np.abs(v).max(initial=0) < 2 ** 24
    return W.bf16_bits_to_f32(W.to_bf16_bits(v.astype(np.float32))).astype(np.int64)


def _check_ranges(ints, n_shared):
    """Every (token, expert) pair, whatever the routing: g in [40, 1023],
    |g u| < 2^24 and every down sum's absolute terms below 2^24."""
    x = ints["x"]
    mats = [(ints["wg"][e], ints["wu"][e], ints["wd"][e]) for e in range(len(ints["wg"]))]
    if n_shared:
        mats.append((ints["sg"], ints["su"], ints["sd"]))
    for wg, wu, wd in mats:
        g = x @ wg.T
        u = x @ wu.T
        assert g.min() >= 40 and g.max() <= 1023, (g.min(), g.max())
        h = _bf16_round(g * u)
        assert (np.abs(h) @ np.abs(wd).T).max() < 2 ** 24


def reference(ints, n_shared, round_h: bool = True):
    """Exact logits [T, E] (int64), top-1 ids [T] (lower id on ties), and
    out [T, d], shared [T, d] (int64); h is rounded to bf16 unless
    ``round_h`` is False (the fp64 oracle keeps h unrounded)."""
    x = ints["x"]
    logits = x @ ints["wr"].T
    ids = np.argmax(logits, axis=1)  # first maximum: the lower expert id
    rnd = _bf16_round if round_h else (lambda v: v)
    out = np.zeros((x.shape[0], x.shape[1]), np.int64)
    for e in np.unique(ids):
        t = np.nonzero(ids == e)[0]
        h = rnd((x[t] @ ints["wg"][e].T) * (x[t] @ ints["wu"][e].T))
        out[t] = h @ ints["wd"][e].T
    shared = None
    if n_shared:
        hs = rnd((x @ ints["sg"].T) * (x @ ints["su"].T))
        shared = hs @ ints["sd"].T
    return logits, ids, out, shared
