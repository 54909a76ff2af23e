"""Shared helpers of the GPU parity tests: upload seeded inputs, run the four
C-ABI calls on the GPU, and compare against the fp64 oracle."""
from __future__ import annotations

import numpy as np

import expert_grouped_quantized_amd as M
import oracle
import workloads as W
from expert_grouped_quantized_amd.layer import MoELayer, blobs_from_inputs

ORC_FMT = {W.F32: oracle.F32, W.BF16: oracle.BF16, W.I4G32: oracle.I4G32, W.I8ROW: oracle.I8ROW,
           W.MXFP4: oracle.MXFP4, **{name: oracle.FMT_NAMES[name] for name in W.IG32.values()}}


def desc_of(cfg: W.LayerConfig):
    return M.make_desc(cfg.d, cfg.E, cfg.F, cfg.n_shared, cfg.Fs, act=cfg.act,
                       expert_w=cfg.expert, shared_w=cfg.shared if cfg.n_shared else cfg.act)


def spec_of(cfg: W.LayerConfig) -> dict:
    return dict(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, n_shared=cfg.n_shared, Fs=cfg.Fs,
                x_fmt=ORC_FMT[cfg.act], expert_fmt=ORC_FMT[cfg.expert],
                shared_fmt=ORC_FMT[cfg.shared] if cfg.n_shared else 0)


class GpuLayer:
    """Uploads one layer's weights once; runs it on any hidden input."""

    def __init__(self, cfg: W.LayerConfig, inputs: dict, T_max: int | None = None):
        import torch
        self.torch, self.cfg, self.inputs = torch, cfg, inputs
        self.desc = desc_of(cfg)
        T_max = T_max or inputs["x"].shape[0]
        self.layer = MoELayer(self.desc, cfg.k, T_max)
        routed, shared = blobs_from_inputs(self.desc, inputs)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        wr = inputs["wr"]
        wr_t = dev(wr.view(np.int16)).view(torch.bfloat16) if cfg.act == W.BF16 else dev(wr)
        bias = None if inputs.get("bias") is None else dev(inputs["bias"])
        self.layer.set_weights(wr_t, dev(routed), None if shared is None else dev(shared), bias)

    def x_tensor(self, x):
        t = self.torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
        return t.view(self.torch.bfloat16) if self.cfg.act == W.BF16 else t

    def run(self, x) -> dict:
        T = x.shape[0]
        self.layer.forward(self.x_tensor(x), T)
        return self.collect(T)

    def run_ids(self, x, ids, w) -> dict:
        """moe_permute -> moe_grouped_ffn -> moe_combine on caller-given routing
        (ids [T, k] in [0, E), weights w [T, k]); no router call."""
        torch = self.torch
        T, k = ids.shape
        L = self.layer
        L.ids[:T * k].copy_(torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1)))
        L.w[:T * k].copy_(torch.from_numpy(np.ascontiguousarray(w, np.float32).reshape(-1)))
        xt = self.x_tensor(x)
        L.permute(xt, T)
        L.grouped_ffn(xt, T)
        L.combine(T)
        out = self.collect(T)
        out.pop("logits")
        return out

    def collect(self, T) -> dict:
        torch = self.torch
        torch.cuda.synchronize()
        L = self.layer
        y = L.y[:T]
        n = T * self.cfg.k
        cpu = lambda t: t.cpu().numpy()
        out = dict(logits=cpu(L.logits[:T]), ids=cpu(L.ids[:n]).reshape(T, self.cfg.k),
                   w=cpu(L.w[:n]).reshape(T, self.cfg.k), offsets=cpu(L.offsets),
                   perm=cpu(L.perm[:n]), inv_perm=cpu(L.inv_perm[:n]),
                   out_assign=cpu(L.out_assign[:n]),
                   shared_out=cpu(L.shared_out[:T]) if self.cfg.n_shared else None)
        if self.cfg.act == W.BF16:
            out["y"] = y.float().cpu().numpy()
            out["y_bits"] = y.view(torch.int16).cpu().numpy()
        else:
            out["y"] = cpu(y)
            out["y_bits"] = y.view(torch.int32).cpu().numpy()
        return out


def rel_l2(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(a - ref) / (den if den > 0 else 1.0)


def assert_close(a, ref, fp32: bool, what: str):
    """bf16/int paths: rel-L2 <= 5e-3 and max|a-ref| <= 2e-2 max|ref|;
    fp32 path: rel-L2 <= 1e-5."""
    r = rel_l2(a, ref)
    if fp32:
        assert r <= 1e-5, f"{what}: rel-L2 {r:.3e} > 1e-5"
    else:
        mx = np.max(np.abs(np.asarray(a, np.float64) - ref))
        lim = 2e-2 * np.max(np.abs(ref))
        assert r <= 5e-3, f"{what}: rel-L2 {r:.3e} > 5e-3"
        assert mx <= lim, f"{what}: max abs err {mx:.3e} > {lim:.3e}"
    return r


def _stored_f64(a, fmt):
    """Exact fp64 values of stored activations / router weights (bf16 bits or fp32)."""
    if fmt == W.BF16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def logit_error_bound(cfg, inputs, tokens):
    """Per-element bound on |fp32 logit - exact logit| [n, E].

    bf16 router: every product x_i w_i is exact in fp32, so the error is that of
    the fp32 sums.  The kernels sum K in 8 slices of d/8, each an MFMA chain
    of d/256 steps of 32 elements, then the 8 slices, then the bias.  A term
    passes at most log2(32) + 1 = 6 roundings inside one MFMA step and one per
    later step and slice addition, so with m = 6 d/256 + 8 + 1 roundings the
    error is at most m u sum_i |x_i w_i| (u = 2^-24; first order, m u << 1).
    The MFMA's internal rounding is not documented, so each rounding is
    allowed 2u (a truncating adder's worst case).  fp32 router: one fused
    multiply-add per element in sequence, m = d + 1."""
    x = _stored_f64(inputs["x"], cfg.act)[np.asarray(tokens)]
    wr = _stored_f64(inputs["wr"], cfg.act)
    m = cfg.d + 1 if cfg.act == W.F32 else 6 * (cfg.d // 256) + 9
    gamma = 2 * m * 2.0 ** -24
    absdot = np.abs(x) @ np.abs(wr).T
    if inputs.get("bias") is not None:
        absdot += np.abs(inputs["bias"].astype(np.float64))[None, :]
    return gamma * absdot * 1.01 + 1e-30


def check_route(cfg, inputs, out, tokens=None):
    """ids bit-exact and w close against the oracle fed the GPU's fp32 logits;
    every GPU logit within the fp32 summation bound of the oracle's exact
    (fp64) logit."""
    T = out["ids"].shape[0]
    L64 = out["logits"].astype(np.float64)
    ids_o, w_o = oracle.topk_softmax(L64, cfg.k)
    assert np.array_equal(out["ids"], ids_o), "top-k ids differ from the oracle"
    np.testing.assert_allclose(out["w"], w_o, rtol=2e-6, atol=1e-7)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    lo = oracle.router_logits(inputs["x"], ORC_FMT[cfg.act], inputs["wr"], ORC_FMT[cfg.act],
                              cfg.d, cfg.E, bias=inputs.get("bias"), tokens=tok)
    err = np.abs(out["logits"][tok].astype(np.float64) - lo)
    bound = logit_error_bound(cfg, inputs, tok)
    bad = err > bound
    assert not bad.any(), (f"router logits: {int(bad.sum())} beyond the fp32 bound, worst "
                           f"err {err[bad].max():.3e} vs {bound[bad][np.argmax(err[bad])]:.3e}")
    return ids_o, w_o


def check_plan(cfg, out):
    off, perm, inv = oracle.route_plan(out["ids"].reshape(-1), cfg.E)
    assert np.array_equal(out["offsets"], off), "offsets differ"
    assert np.array_equal(out["perm"], perm), "perm differs"
    assert np.array_equal(out["inv_perm"], inv), "inv_perm differs"


def mx_error_constants(cfg):
    """fp32 error model of the W4A4 path: gamma of the gate/up and of the down
    dot products (one rounding per 32-element block of the MFMA chain,
    doubled, plus eight), eta of the elementwise steps that make h."""
    return (cfg.d / 16 + 8) * 2.0 ** -24, (cfg.F / 16 + 8) * 2.0 ** -24, 2.0 ** -16


def check_values_mx(cfg, inputs, out, w_o, tokens=None):
    """MXFP4 W4A4 routed experts.  x's codes are decisions on exact inputs and
    must match; h's codes are decisions on a computed h, so where h lies within
    its fp32 error of a decision boundary either code is correct: the oracle
    returns, per output element, mag = sum |Wd hq| and the largest change such
    a decision can make (slack).  Bound on out_assign, per element:
    |gpu - ref| <= gamma_F (mag + slack) + slack.  y: rel-L2 <= 5e-3 and
    max-abs <= 2e-2 max|ref| + the slack of its k assignments."""
    T = out["ids"].shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    g_gu, g_dn, eta = mx_error_constants(cfg)
    y_ref, oa_ref, so_ref, slack, mag = oracle.moe_experts_mx(
        spec_of(cfg), inputs, out["ids"][tok], w_o[tok], g_gu, eta, tokens=tok)
    flat = (tok[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    gpu_oa = out["out_assign"][out["inv_perm"][flat]].astype(np.float64)
    err = np.abs(gpu_oa - oa_ref)
    tight = g_dn * (mag + slack)
    bound = tight + slack
    bad = err > bound
    assert not bad.any(), (f"out_assign: {int(bad.sum())} elements beyond the W4A4 bound, worst "
                           f"err {err[bad].max():.3e} vs bound {bound[bad][np.argmax(err[bad])]:.3e}")
    r_oa = rel_l2(gpu_oa, oa_ref)
    assert r_oa <= 5e-3, f"out_assign: rel-L2 {r_oa:.3e} > 5e-3"
    y_gpu = np.asarray(out["y"][tok], np.float64)
    r_y = rel_l2(y_gpu, y_ref)
    assert r_y <= 5e-3, f"y: rel-L2 {r_y:.3e} > 5e-3"
    lim = 2e-2 * np.max(np.abs(y_ref)) + slack.reshape(len(tok), cfg.k, cfg.d).sum(axis=1)
    over = np.abs(y_gpu - y_ref) > lim
    assert not over.any(), f"y: {int(over.sum())} elements beyond 2e-2 max|ref| + slack"
    r_so = None
    if cfg.n_shared:
        r_so = assert_close(out["shared_out"][tok], so_ref, False, "shared_out")
    return dict(y=r_y, out_assign=r_oa, shared_out=r_so,
                rows_with_slack=int((slack > 0).any(axis=1).sum()),
                elements_using_slack=int((err > tight).sum()))


def check_values(cfg, inputs, out, w_o, tokens=None):
    """y, out_assign and shared_out of the chosen tokens against the oracle."""
    if cfg.expert == W.MXFP4:
        return check_values_mx(cfg, inputs, out, w_o, tokens)
    T = out["ids"].shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    fp32 = cfg.act == W.F32
    y_ref, oa_ref, so_ref = oracle.moe_experts(spec_of(cfg), inputs, out["ids"][tok], w_o[tok],
                                               tokens=tok)
    r_y = assert_close(out["y"][tok], y_ref, fp32, "y")
    flat = (tok[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    gpu_oa = out["out_assign"][out["inv_perm"][flat]]
    r_oa = assert_close(gpu_oa, oa_ref, fp32, "out_assign")
    r_so = None
    if cfg.n_shared:
        r_so = assert_close(out["shared_out"][tok], so_ref, fp32, "shared_out")
    return dict(y=r_y, out_assign=r_oa, shared_out=r_so)
