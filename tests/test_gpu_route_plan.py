"""GPU tests of moe_route_plan, the one-call front end (router, top-k, route
plan and the fp16 copy of x; a single launch for bf16 calls of T <= 32).

Its outputs -- logits, ids, weights, offsets, perm, inv_perm, and the row-tile
plan and fp16 copy of x it leaves in the workspace -- must equal those of the
separate moe_route + moe_permute calls bit for bit, and the ids and plan must
equal the oracle's on the GPU's logits; the whole layer run on them is checked
against the oracle (same bar as the other parity tests).  Repeated calls on
one workspace (its block counter must return to zero), a larger call on the
same workspace between them, and the 512-expert decode shape are covered.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuLayer, check_plan, check_route, check_values  # noqa: E402
from expert_grouped_quantized_amd.layer import MoELayer  # noqa: E402


def _say(*a):
    print(*a, flush=True)


FRONT = ("logits", "ids", "w", "offsets", "perm", "inv_perm")


def _front(L, T, k):
    torch.cuda.synchronize()
    n = T * k
    return dict(logits=L.logits[:T].cpu().numpy(), ids=L.ids[:n].cpu().numpy(),
                w=L.w[:n].cpu().numpy(), offsets=L.offsets.cpu().numpy(),
                perm=L.perm[:n].cpu().numpy(), inv_perm=L.inv_perm[:n].cpu().numpy(),
                ws=L.workspace.cpu().numpy())


def _twin(g, T_max):
    """Two layers on g's weights: `sep` runs moe_route + moe_permute, `one`
    runs moe_route_plan; both workspaces start zeroed."""
    L0 = g.layer
    mk = lambda: MoELayer(g.desc, g.cfg.k, T_max)
    sep, one = mk(), mk()
    for L in (sep, one):
        L.set_weights(L0.router_w, L0.routed_blob, L0.shared_blob, L0.bias)
    return sep, one


def _compare_fronts(g, sep, one, x, T, what):
    xt = g.x_tensor(x)
    sep.route(xt, T)
    sep.permute(xt, T)
    a = _front(sep, T, g.cfg.k)
    one.route_plan(xt, T)
    b = _front(one, T, g.cfg.k)
    for key in FRONT:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), f"{what}: {key} differs"
    # tiles, fp16 copy of x and its scales; regions neither call writes stay
    # zero in both (the counters at the workspace's start included)
    assert np.array_equal(a["ws"], b["ws"]), f"{what}: workspace differs"
    assert not b["ws"][:16].any(), f"{what}: block counters not back to zero"


def _finish_and_check(g, sep, one, x, T, what):
    """grouped FFN + combine on both layers' front-end outputs of the same T
    (the caller has just run both front ends on x) -- on both, so their
    workspaces stay alike): y equal bit for bit, and one's outputs checked
    against the oracle."""
    cfg = g.cfg.with_T(T)
    xt = g.x_tensor(x)
    for L in (sep, one):
        L.grouped_ffn(xt, T)
        L.combine(T)
    torch.cuda.synchronize()
    assert np.array_equal(sep.y[:T].view(torch.int16).cpu().numpy(),
                          one.y[:T].view(torch.int16).cpu().numpy()), f"{what}: y differs"
    saved = g.layer
    g.layer = one
    try:
        out = g.collect(T)
    finally:
        g.layer = saved
    inp = dict(g.inputs, x=x)
    ids_o, w_o = check_route(cfg, inp, out)
    check_plan(cfg, out)
    r = check_values(cfg, inp, out, w_o)
    _say(f"[ok] {what}", r)


def _cfg(name, idx, **kw):
    base = dict(T=100, d=256, E=16, k=4, F=256, n_shared=1, Fs=256, act=W.BF16, router=W.BF16,
                expert=W.I4G32, shared=W.I8ROW)
    base.update(kw)
    return W.LayerConfig(name, 300 + idx, **base)


SMALL = [
    _cfg("rp_i4_E16", 0),
    _cfg("rp_bf16_E1024_k8", 1, E=1024, k=8, expert=W.BF16, shared=W.BF16),  # 16 candidates a lane
    _cfg("rp_E48_k6", 2, E=48, k=6),           # a partial last router block
    _cfg("rp_E64_k32", 3, E=64, k=32, n_shared=0, Fs=0),  # the largest k
    _cfg("rp_i3_E200", 4, E=200, k=10, expert=W.IG32[3]),
    _cfg("rp_mx_E40", 5, E=40, k=5, expert=W.MXFP4),  # no fp16 copy of x
    _cfg("rp_zipf_bias_E512", 6, E=512, k=10, zipf=True),  # router bias, skewed routing
    _cfg("rp_E1_k1", 7, E=1, k=1, n_shared=0, Fs=0),        # one expert: a dense layer
    _cfg("rp_E20_k3_bf16", 8, E=20, k=3, expert=W.BF16, shared=W.BF16),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_plan_matches_separate_calls(cfg):
    inp = W.generate(cfg)
    g = GpuLayer(cfg, inp)
    sep, one = _twin(g, cfg.T)
    x = inp["x"]
    x_neg = W.to_bf16_bits(-W.bf16_bits_to_f32(x))
    # T = 1, 5, 16 (one token group), 17, 20 and 32 (two groups, the second
    # ragged or full), repeated on one workspace, with a T = 100 call
    # (separate launches) on the same workspace in between
    for T in (1, 5, 16, 17, 20, 32, 100, 16, 32, 5):
        for xi, tag in ((x, "x"), (x_neg, "-x")):
            _compare_fronts(g, sep, one, xi[:T], T, f"{cfg.name} T={T} {tag}")
    for T in (1, 5, 16, 20, 32):
        _compare_fronts(g, sep, one, x[:T], T, f"{cfg.name} T={T}")
        _finish_and_check(g, sep, one, x[:T], T, f"{cfg.name} T={T} layer vs oracle")


def test_route_plan_decode_shape():
    """d=2560, E=512, k=10 (the decode layer): T = 1, 5, 16, 20, 32."""
    cfg = W.CONFIGS["int4_decode"]
    inp = W.generate(cfg, T=32)
    g = GpuLayer(cfg, inp, T_max=32)
    sep, one = _twin(g, 32)
    for T in (1, 5, 16, 20, 32, 16):
        _compare_fronts(g, sep, one, inp["x"][:T], T, f"decode T={T}")
    for T in (1, 5, 20):
        _compare_fronts(g, sep, one, inp["x"][:T], T, f"decode T={T}")
        _finish_and_check(g, sep, one, inp["x"][:T], T, f"decode T={T} layer vs oracle")
