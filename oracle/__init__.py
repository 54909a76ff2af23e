"""Plain fp64 CPU oracle of the expert-grouped MoE layer (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the two share no code.

The arithmetic lives in ``oracle.c`` (double precision, each function the plain
definition of one step of the layer described on the pages about serving
Qwen3.8-Flash-Next: "Qwen3.8-Flash-Next-Dual-GPU" README, section "Dedicated
prefill lane" and section "Independent decode lane"; TandemLLM docs chapter 17,
Table 17.1).  This module only marshals numpy arrays into it.

Parity pins (see tests/test_oracle_*.py): brute-force top-k, softmax
invariants, permutation invariants, the E=1/k=1 dense reduction checked against
numpy's BLAS product, exhaustive decoder checks, integer-exact cases; for the
MXFP4 W4A4 experts the OCP E2M1 table, brute-force rounding, a hand-worked MX
fixture and perturbation checks of the decision slack.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.environ.get("ORC_LIB_OVERRIDE") or os.path.join(_HERE, "liborc.so")

F32, BF16, I4G32, I8ROW = 0, 1, 2, 3
MXFP4 = 4  # OCP MX FP4: e2m1 nibbles + E8M0 scale byte per 32 along K (W4A4 experts)
IG32 = 16  # + b: b-bit symmetric codes, one int8 each, fp16 scale per 32 along K
I2G32, I3G32, I5G32, I6G32, I7G32, I8G32 = (IG32 + b for b in (2, 3, 5, 6, 7, 8))
FMT_NAMES = {"f32": F32, "bf16": BF16, "i4g32": I4G32, "i8row": I8ROW, "i2g32": I2G32,
             "i3g32": I3G32, "i5g32": I5G32, "i6g32": I6G32, "i7g32": I7G32, "i8g32": I8G32,
             "mxfp4": MXFP4}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP) into liborc.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("E", ctypes.c_int64), ("k", ctypes.c_int64),
                ("F", ctypes.c_int64), ("n_shared", ctypes.c_int64), ("Fs", ctypes.c_int64),
                ("x_fmt", ctypes.c_int), ("expert_fmt", ctypes.c_int), ("shared_fmt", ctypes.c_int)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x", "wg", "wg_s", "wu", "wu_s", "wd", "wd_s",
                 "sg", "sg_s", "su", "su_s", "sd", "sd_s")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_decode_matrix.argtypes = [i32, i64, i64, vp, vp, vp]
        L.orc_router_logits.argtypes = [i64, vp, i64, i64, i32, vp, i32, vp, vp, vp]
        L.orc_topk_softmax.argtypes = [i64, i64, i64, vp, vp, vp]
        L.orc_route_plan.argtypes = [i64, i64, vp, vp, vp, vp]
        L.orc_swiglu_dense.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        L.orc_moe_experts.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), i64, vp,
                                      vp, vp, vp, vp, vp]
        L.orc_moe_experts_mx.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), i64,
                                         vp, vp, vp, ctypes.c_double, ctypes.c_double, vp, vp,
                                         vp, vp, vp]
        L.orc_e2m1_to_f64.argtypes = [i32]
        L.orc_e2m1_to_f64.restype = ctypes.c_double
        L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f64.restype = ctypes.c_double
        L.orc_e2m1_round.argtypes = [ctypes.c_double]
        L.orc_e2m1_round.restype = ctypes.c_double
        L.orc_mx_exponent.argtypes = [ctypes.c_double]
        L.orc_mx_exponent.restype = ctypes.c_int
        L.orc_mx_quantize.argtypes = [i64, vp, vp, vp]
        L.orc_mx_slack.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, vp]
        for fn in ("orc_decode_matrix", "orc_router_logits", "orc_topk_softmax",
                   "orc_route_plan", "orc_swiglu_dense", "orc_moe_experts",
                   "orc_moe_experts_mx", "orc_mx_quantize", "orc_mx_slack"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def decode_matrix(fmt: int, rows: int, K: int, q, scales=None) -> np.ndarray:
    """Exact fp64 values of a stored [rows, K] matrix (see oracle.c)."""
    q = np.ascontiguousarray(q)
    scales = None if scales is None else np.ascontiguousarray(scales)
    out = np.empty((rows, K), np.float64)
    _check(lib().orc_decode_matrix(fmt, rows, K, _ptr(q), _ptr(scales), _ptr(out)), "decode")
    return out


def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(int(bits))


def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits))


def e2m1_to_f64(code: int) -> float:
    """Value of a 4-bit OCP MX e2m1 code."""
    return lib().orc_e2m1_to_f64(int(code))


def e8m0_to_f64(bits: int) -> float:
    """Value of an OCP MX E8M0 scale byte (NaN for 255)."""
    return lib().orc_e8m0_to_f64(int(bits))


def e2m1_round(y: float) -> float:
    """Nearest e2m1 value to y, ties to the even mantissa, saturated at +-6."""
    return lib().orc_e2m1_round(float(y))


def mx_exponent(amax: float) -> int:
    """Shared exponent of an MX block with largest magnitude amax."""
    return lib().orc_mx_exponent(float(amax))


def mx_quantize(v):
    """OCP MX (FP4) quantization of the rows of v (last dim % 32 == 0), block
    by block of 32: (dequantized fp64 values, E8M0 scale bytes)."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty_like(v)
    eb = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    _check(lib().orc_mx_quantize(v.size, _ptr(v), _ptr(out), _ptr(eb)), "mx_quantize")
    return out, eb


def mx_slack(h, dh, wd):
    """Decision slack of MX(h) against any h' within dh of h (oracle.c,
    orc_mx_slack): (hq [F], delta [F], slack [d], mag [d]) for wd [d, F]."""
    h = np.ascontiguousarray(h, np.float64)
    dh = np.ascontiguousarray(dh, np.float64)
    wd = np.ascontiguousarray(wd, np.float64)
    d, F = wd.shape
    assert h.shape == (F,) and dh.shape == (F,)
    hq, delta = np.empty(F), np.empty(F)
    slack, mag = np.empty(d), np.empty(d)
    _check(lib().orc_mx_slack(d, F, _ptr(h), _ptr(dh), _ptr(wd), _ptr(hq), _ptr(delta),
                              _ptr(slack), _ptr(mag)), "mx_slack")
    return hq, delta, slack, mag


def router_logits(x, x_fmt, wr, wr_fmt, d, E, bias=None, tokens=None) -> np.ndarray:
    """fp64 router logits [n, E] for the given token rows (all rows if None)."""
    x = np.ascontiguousarray(x)
    wr = np.ascontiguousarray(wr)
    n = x.shape[0] if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    bias = _c(bias, np.float32)
    out = np.empty((n, E), np.float64)
    _check(lib().orc_router_logits(n, _ptr(tok), d, E, x_fmt, _ptr(x), wr_fmt, _ptr(wr),
                                   _ptr(bias), _ptr(out)), "router_logits")
    return out


def topk_softmax(logits, k: int):
    """Stable top-k (ties -> lower id) and softmax over the chosen k."""
    logits = np.ascontiguousarray(logits, np.float64)
    n, E = logits.shape
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    _check(lib().orc_topk_softmax(n, E, k, _ptr(logits), _ptr(ids), _ptr(w)), "topk_softmax")
    return ids, w


def route_plan(ids, E: int):
    """offsets [E+1], perm [n], inv_perm [n] of the flat ids (stable by flat index)."""
    ids = np.ascontiguousarray(ids, np.int32).reshape(-1)
    n = ids.size
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(n, 1), np.int32)
    inv = np.empty(max(n, 1), np.int32)
    _check(lib().orc_route_plan(n, E, _ptr(ids), _ptr(offsets), _ptr(perm), _ptr(inv)),
           "route_plan")
    return offsets, perm[:n], inv[:n]


def swiglu_dense(X, wg, wu, wd) -> np.ndarray:
    """Dense SwiGLU MLP on decoded fp64 weights: rows of X -> Wd(silu(Wg x)*Wu x)."""
    X = np.ascontiguousarray(X, np.float64)
    wg = np.ascontiguousarray(wg, np.float64)
    wu = np.ascontiguousarray(wu, np.float64)
    wd = np.ascontiguousarray(wd, np.float64)
    M, d = X.shape
    F = wg.shape[0]
    out = np.empty((M, d), np.float64)
    _check(lib().orc_swiglu_dense(M, d, F, _ptr(X), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(out)),
           "swiglu_dense")
    return out


def _layer_args(spec, inputs, ids, w, tokens):
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    n, k = ids.shape[0], spec["k"]
    assert ids.shape == (n, k) and w.shape == (n, k)
    D = _Desc(spec["d"], spec["E"], k, spec["F"], spec["n_shared"], spec["Fs"],
              spec["x_fmt"], spec["expert_fmt"], spec["shared_fmt"])
    keep = [ids, w]

    def p(name):
        a = inputs.get(name)
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    W = _Weights(*(p(n_) for n_ in ("x", "wg", "wg_s", "wu", "wu_s", "wd", "wd_s",
                                    "sg", "sg_s", "su", "su_s", "sd", "sd_s")))
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    keep.append(tok)
    return D, W, n, k, tok, ids, w, keep


def moe_experts_mx(spec: dict, inputs: dict, ids, w, gamma: float, eta: float, tokens=None):
    """The layer with MXFP4 W4A4 routed experts, plus the bounds its parity
    check needs (oracle.c, swiglu_row_mx): returns (y, out_assign, shared_out,
    slack, mag), the last two [n*k, d] in slot order like out_assign."""
    D, W, n, k, tok, ids, w, keep = _layer_args(spec, inputs, ids, w, tokens)
    d = spec["d"]
    y = np.empty((n, d), np.float64)
    oa = np.empty((n * k, d), np.float64)
    so = np.empty((n, d), np.float64) if spec["n_shared"] else None
    slack = np.empty((n * k, d), np.float64)
    mag = np.empty((n * k, d), np.float64)
    _check(lib().orc_moe_experts_mx(ctypes.byref(D), ctypes.byref(W), n, _ptr(tok), _ptr(ids),
                                    _ptr(w), gamma, eta, _ptr(oa), _ptr(so), _ptr(y),
                                    _ptr(slack), _ptr(mag)), "moe_experts_mx")
    return y, oa, so, slack, mag


def moe_experts(spec: dict, inputs: dict, ids, w, tokens=None, want_parts: bool = True):
    """Per-expert SwiGLU loop + shared expert + weighted sum, fp64.

    ``spec``: d, E, k, F, n_shared, Fs, x_fmt, expert_fmt, shared_fmt (ints).
    ``inputs``: stored arrays x, wg(, wg_s), wu, wd, sg, su, sd (+ scales).
    ``ids``/``w``: [n, k] routing of the selected rows (``tokens`` maps row ->
    token index of x; all T rows when None).
    Returns (y [n, d], out_assign [n*k, d] or None, shared_out [n, d] or None).
    """
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    n = ids.shape[0]
    k = spec["k"]
    assert ids.shape == (n, k) and w.shape == (n, k)
    D = _Desc(spec["d"], spec["E"], k, spec["F"], spec["n_shared"], spec["Fs"],
              spec["x_fmt"], spec["expert_fmt"], spec["shared_fmt"])
    keep = {}

    def p(name):
        a = inputs.get(name)
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep[name] = a
        return a.ctypes.data

    W = _Weights(*(p(n_) for n_ in ("x", "wg", "wg_s", "wu", "wu_s", "wd", "wd_s",
                                    "sg", "sg_s", "su", "su_s", "sd", "sd_s")))
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    d = spec["d"]
    y = np.empty((n, d), np.float64)
    oa = np.empty((n * k, d), np.float64) if want_parts else None
    so = np.empty((n, d), np.float64) if (want_parts and spec["n_shared"]) else None
    _check(lib().orc_moe_experts(ctypes.byref(D), ctypes.byref(W), n, _ptr(tok), _ptr(ids),
                                 _ptr(w), _ptr(oa), _ptr(so), _ptr(y)), "moe_experts")
    return y, oa, so
