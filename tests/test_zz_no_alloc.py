"""moe_grouped_ffn_noalloc (no workspace, library-held scratch) against
moe_grouped_ffn (caller's workspace), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, each
compared with moe_grouped_ffn on the same inputs: out_assign and shared_out
bit for bit (the same kernels on the same plan), and the combined y against
the oracle at the parity bar.  Host-side checks (too large a call is refused
before anything is enqueued; T = 0 is a no-op) need no GPU."""
import ctypes

import numpy as np
import pytest

import expert_grouped_quantized_amd as M
import oracle
import workloads as W

FAKE = 0x10000


def _desc(**kw):
    base = dict(d=2560, n_experts=512, ffn=1024, n_shared=1, shared_ffn=1024, act="bf16",
                expert_w="i4g32", shared_w="i8row")
    base.update(kw)
    return M.make_desc(**base)


def _noalloc(desc, T, k, **p):
    a = dict(hidden=FAKE, w=FAKE, off=FAKE, perm=FAKE, rb=FAKE, sb=FAKE, oa=FAKE, so=FAKE)
    a.update(p)
    return M.lib().moe_grouped_ffn_noalloc(ctypes.byref(desc), T, k, a["hidden"], a["w"],
                                           a["off"], a["perm"], a["rb"], a["sb"], a["oa"],
                                           a["so"], None)


def test_noalloc_refuses_calls_beyond_its_scratch():
    desc = _desc()
    assert _noalloc(desc, 4096, 10) == M.MOE_EWORKSPACE
    msg = M.moe_last_error()
    assert "static scratch" in msg and "8388608" in msg
    assert M.moe_workspace_bytes(desc, 302, 10) <= 8 << 20 < M.moe_workspace_bytes(desc, 303, 10)
    assert _noalloc(desc, 303, 10) == M.MOE_EWORKSPACE


def test_noalloc_checks_arguments_and_T_zero():
    desc = _desc()
    assert _noalloc(desc, 0, 10) == M.MOE_OK
    assert _noalloc(desc, 4, 10, hidden=None) == M.MOE_EINVAL
    assert "hidden" in M.moe_last_error()
    assert _noalloc(desc, 4, 0) == M.MOE_EINVAL
    assert _noalloc(_desc(n_shared=0, shared_ffn=0), 4, 10) == M.MOE_EINVAL  # shared ptrs given


def _small_cfg(name, idx, **kw):
    base = dict(T=200, d=512, E=32, k=6, F=256, n_shared=1, Fs=256, act=W.BF16, router=W.BF16,
                expert=W.I4G32, shared=W.I8ROW)
    base.update(kw)
    return W.LayerConfig(name, 300 + idx, **base)


@pytest.mark.gpu
@pytest.mark.parametrize("expert,shared,Ts", [(W.I4G32, W.I8ROW, (200, 16)),
                                              (W.MXFP4, W.I8ROW, (120, 24)),
                                              (W.BF16, W.BF16, (64, 5))])
def test_noalloc_matches_workspace_call(expert, shared, Ts):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_harness import GpuLayer, check_values
    cfg = _small_cfg(f"noalloc_{expert}", {W.I4G32: 0, W.MXFP4: 1, W.BF16: 2}[expert],
                     T=Ts[0], expert=expert, shared=shared)
    inp = W.generate(cfg)
    g = GpuLayer(cfg, inp)
    L = g.layer
    k = cfg.k
    for T in Ts:  # the second call is smaller than the first
        print(f"[run] noalloc {expert} T={T}", flush=True)
        x = inp["x"][:T]
        ref = g.run(x)  # route -> permute -> moe_grouped_ffn (workspace) -> combine
        n = T * k
        oa = torch.full((n, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        so = torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        xt = g.x_tensor(x)
        M.moe_grouped_ffn_noalloc(L.desc, T, k, xt, L.w, L.offsets, L.perm, L.routed_blob,
                                  L.shared_blob, oa, so)
        torch.cuda.synchronize()
        oa_h, so_h = oa.cpu().numpy(), so.cpu().numpy()
        assert np.array_equal(oa_h, ref["out_assign"]), f"T={T}: out_assign differs"
        assert np.array_equal(so_h, ref["shared_out"]), f"T={T}: shared_out differs"
        # y from the no-allocation outputs, against the oracle
        y = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
        M.moe_combine(L.desc, T, k, oa, L.inv_perm, so, y)
        torch.cuda.synchronize()
        out = dict(ref, out_assign=oa_h, shared_out=so_h, y=y.float().cpu().numpy())
        assert np.array_equal(y.view(torch.int16).cpu().numpy(), ref["y_bits"])
        r = check_values(cfg, dict(inp, x=x), out, ref["w"].astype(np.float64))
        print(f"[ok] noalloc {expert} T={T}", r, flush=True)
