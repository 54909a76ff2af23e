"""CPU checks of the tolerances the GPU parity tests use (no GPU).

The router-logit bound of gpu_harness.logit_error_bound must hold for an fp32
computation that sums in the kernels' order, and must be tight enough that
plausible mistakes (a dropped K element, logits kept at bf16 precision, a
fp32 sum of bf16-rounded products) fall outside it."""
import numpy as np

import oracle
import workloads as W
from gpu_harness import logit_error_bound


def _fp32_logits_kernel_order(x, wr):
    """fp32 logits summed as the router kernels sum them: K in 8 equal slices,
    each a chain over 32-element blocks (a block summed pairwise, then added
    to the chain), then the slices added in order."""
    T, d = x.shape
    E = wr.shape[0]
    prod = (x[:, None, :].astype(np.float32) * wr[None, :, :].astype(np.float32))  # exact
    sl = d // 8
    tot = np.zeros((T, E), np.float32)
    for s in range(8):
        acc = np.zeros((T, E), np.float32)
        for b0 in range(s * sl, (s + 1) * sl, 32):
            blk = prod[:, :, b0:b0 + 32]
            while blk.shape[2] > 1:
                blk = (blk[:, :, 0::2] + blk[:, :, 1::2]).astype(np.float32)
            acc = (acc + blk[:, :, 0]).astype(np.float32)
        tot = acc if s == 0 else (tot + acc).astype(np.float32)
    return tot


def test_logit_bound_holds_and_is_tight():
    cfg = W.LayerConfig("bound", 900, T=24, d=2560, E=64, k=4, F=256, n_shared=0, Fs=0,
                        act=W.BF16, router=W.BF16, expert=W.BF16, shared=W.BF16)
    rng = np.random.default_rng(9)
    x = W.to_bf16_bits(rng.standard_normal((cfg.T, cfg.d)).astype(np.float32))
    wr = W.to_bf16_bits((rng.standard_normal((cfg.E, cfg.d)) / np.sqrt(cfg.d)).astype(np.float32))
    inputs = {"x": x, "wr": wr}
    xf, wf = W.bf16_bits_to_f32(x), W.bf16_bits_to_f32(wr)
    exact = oracle.router_logits(x, oracle.BF16, wr, oracle.BF16, cfg.d, cfg.E)
    bound = logit_error_bound(cfg, inputs, np.arange(cfg.T))
    gpu_like = _fp32_logits_kernel_order(xf, wf).astype(np.float64)
    assert (np.abs(gpu_like - exact) <= bound).all()
    # tighter than a flat 2e-4 max|logit| everywhere
    assert bound.max() < 2e-4 * np.abs(exact).max() / 2
    # a dropped last K element, bf16-precision logits, bf16-rounded products
    dropped = exact - xf[:, None, -1].astype(np.float64) * wf[None, :, -1]
    assert (np.abs(dropped - exact) > bound).mean() > 0.5
    as_bf16 = W.bf16_bits_to_f32(W.to_bf16_bits(exact.astype(np.float32))).astype(np.float64)
    assert (np.abs(as_bf16 - exact) > bound).mean() > 0.5
    prod16 = W.bf16_bits_to_f32(W.to_bf16_bits(xf[:, None, :] * wf[None, :, :])).astype(np.float64)
    assert (np.abs(prod16.sum(axis=2) - exact) > bound).any()
